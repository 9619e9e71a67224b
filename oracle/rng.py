"""Counter-based random numbers for context drop-off / drop-in (oracle side).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg, never by the product path.

The pages only say that drop-off removes floor(p*k) chunks "at random" with p ~ U(0, p_max)
and that drop-in adds m ~ Poisson(lambda) random chunks (Mixture of Contexts summary, §3.1;
docswell slides, slide 14). They fix no generator, so this build fixes one and implements it
twice from its published definition, once here in plain Python integers and once in HIP:

* SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable pseudorandom number generators",
  OOPSLA 2014): the n-th output of the stream seeded with s is mix64(s + n * GOLDEN) mod 2^64,
  with mix64 the variant-13 finaliser (xor-shift 30 / multiply / xor-shift 27 / multiply /
  xor-shift 31).
* H32(seed; ctr) = high 32 bits of output number ctr+1, where
  ctr = ((((b*H + h)*L + t)*4 + stream) << 8) | j.
* Poisson(lambda) by inversion against integer thresholds
  Thr_i = floor(2^32 * sum_{j<=i} e^-lambda lambda^j / j!), evaluated in IEEE binary64 in the
  order written, with e^-lambda from the C library's exp (Python's math.exp).
"""
from __future__ import annotations

import math
from typing import List

MASK64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
MIX_M1 = 0xBF58476D1CE4E5B9
MIX_M2 = 0x94D049BB133111EB

STREAM_DROP_P = 0     # the uniform that sets p for drop-off
STREAM_DROP_PICK = 1  # which selected chunk to drop, j-th pick
STREAM_IN_COUNT = 2   # the uniform that sets m for drop-in
STREAM_IN_PICK = 3    # which candidate chunk to add, j-th pick


def mix64(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * MIX_M1) & MASK64
    z = ((z ^ (z >> 27)) * MIX_M2) & MASK64
    return z ^ (z >> 31)


def splitmix64_stream(seed: int, n: int) -> List[int]:
    """First n outputs of SplitMix64 seeded with `seed` (state += GOLDEN, then mix)."""
    out = []
    state = seed & MASK64
    for _ in range(n):
        state = (state + GOLDEN) & MASK64
        out.append(mix64(state))
    return out


def counter(b: int, h: int, t: int, stream: int, j: int, H: int, L: int) -> int:
    assert 0 <= stream < 4 and 0 <= j < 256
    return (((((b * H + h) * L + t) * 4 + stream) << 8) | j) & MASK64


def h32(seed: int, ctr: int) -> int:
    return mix64((seed + (ctr + 1) * GOLDEN) & MASK64) >> 32


def poisson_thresholds(lam: float, m_cap: int) -> List[int]:
    """Thr_i for i in [0, m_cap): floor(2^32 * CDF_Poisson(lam)(i)), capped at 2^32."""
    out = []
    term = math.exp(-lam)
    cdf = term
    for i in range(m_cap):
        if i > 0:
            term = term * lam / i
            cdf = cdf + term
        v = math.floor(cdf * 4294967296.0)
        out.append(min(int(v), 1 << 32))
    return out


def poisson_from_word(r: int, thr: List[int], m_cap: int) -> int:
    """Smallest i < m_cap with r < Thr_i; m_cap if none."""
    for i in range(m_cap):
        if r < thr[i]:
            return i
    return m_cap
