"""Seeded random weights for a one-layer model (embedding, fused q/k/v
projection, output projection, vocabulary projection), drawn as float32 and
rounded to bfloat16 bit patterns.  Random draws only: nothing here runs the
model.

Draw order (one ``PCG64(seed)`` stream): E [V][d] ~ N(0, 1), Wqkv
[(Hq + 2 Hkv) D][d] ~ N(0, 1/d), Wo [d][Hq D] ~ N(0, 1/(Hq D)),
Wlm [V][d] ~ N(0, logit_sigma^2 / (2 d)), with d = Hq * D.
"""

from __future__ import annotations

import numpy as np

from .workloads import f32_to_bf16_bits


def model_config(V: int, Hq: int, Hkv: int, D: int, theta: float = 10000.0) -> dict:
    return dict(V=V, Hq=Hq, Hkv=Hkv, D=D, d=Hq * D, theta=theta)


def model_weights(seed: int, cfg: dict, logit_sigma: float = 4.0) -> dict:
    """bf16 bit patterns (uint16) of every weight, keyed E, Wqkv, Wo, Wlm."""
    rng = np.random.Generator(np.random.PCG64(seed))
    V, Hq, Hkv, D, d = cfg["V"], cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["d"]

    def draw(shape, sigma):
        x = rng.standard_normal(shape, dtype=np.float32)
        x *= np.float32(sigma)
        return f32_to_bf16_bits(x)

    return dict(
        E=draw((V, d), 1.0),
        Wqkv=draw(((Hq + 2 * Hkv) * D, d), 1.0 / np.sqrt(d)),
        Wo=draw((d, Hq * D), 1.0 / np.sqrt(Hq * D)),
        Wlm=draw((V, d), logit_sigma / np.sqrt(2.0 * d)),
    )
