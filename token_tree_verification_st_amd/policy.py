"""Host-side scheduling policy around the verification path.

Nothing here touches the GPU: these are decisions a serving loop makes
between verification steps.
"""

from __future__ import annotations


def candidate_length(t: int, T_est: int, K_max: int) -> int:
    """Draft length for the next step (speculative-decoding explainer §3.3,
    dynamic candidate length): K_t = max(1, round(K_max * (1 - t / T_est)))
    for t tokens generated out of an estimated T_est.  Rounds half to even."""
    if T_est <= 0 or K_max < 1:
        raise ValueError("T_est must be positive and K_max at least 1")
    return max(1, int(round(K_max * (1.0 - t / T_est))))
