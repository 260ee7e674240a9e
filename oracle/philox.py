"""Philox4x64-10 counter-based generator, written from its published definition
(Salmon, Moraes, Dror, Shaw: "Parallel random numbers: as easy as 1, 2, 3",
SC'11): a 4 x 64-bit counter and a 2 x 64-bit key, ten rounds; each round
multiplies counter words 0 and 2 by two fixed odd constants, keeps the high and
low halves of the 128-bit products, and xors the high halves with the other
two counter words and the key; between rounds the key is bumped by two Weyl
constants (golden ratio and sqrt(3) - 1, as 64-bit fixed point).

Stochastic acceptance draws two uniforms per tree node (a reading: the pages
only ask for random acceptance, not for a generator):
  key     = (seed, 0)
  counter = (local node index, request index, offset, 0)
  u_acc   = (word0 >> 40) * 2^-24   node's own accept test
  u_smp   = (word1 >> 40) * 2^-24   sample for the replacement token if the
                                    walk stops at this node
Both are multiples of 2^-24 in [0, 1) and so exact in fp32 and fp64.
"""

MASK64 = (1 << 64) - 1
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15
PHILOX_W1 = 0xBB67AE8584CAA73B


def _mulhilo(a: int, b: int):
    p = a * b
    return (p >> 64) & MASK64, p & MASK64


def philox4x64_10(counter, key):
    c0, c1, c2, c3 = (int(x) & MASK64 for x in counter)
    k0, k1 = (int(x) & MASK64 for x in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + PHILOX_W0) & MASK64
            k1 = (k1 + PHILOX_W1) & MASK64
        hi0, lo0 = _mulhilo(PHILOX_M0, c0)
        hi1, lo1 = _mulhilo(PHILOX_M1, c2)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def uniforms_for_node(seed: int, offset: int, request: int, local_node: int):
    """(u_acc, u_smp) for one tree node."""
    w = philox4x64_10((local_node, request, offset, 0), (seed, 0))
    return (w[0] >> 40) * 2.0 ** -24, (w[1] >> 40) * 2.0 ** -24
