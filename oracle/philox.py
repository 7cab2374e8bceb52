"""Counter-based Gaussian noise for the noisy gate (oracle side).

The pages ask for a fresh standard-normal sample per expert component on every
forward pass (Outrageously Large Neural Networks summary, section 3.4, "Noisy
Top-K Gating", Step 1) but fix no generator. The reading used here keys the
sample by (seed, token t, expert e):

  q = e // 4, r = e % 4
  (r0, r1, r2, r3) = Philox4x64-10(counter = (t, q, 0, 0), key = (seed, g))
  with g = 0 for a flat gate (and the primary gate of a hierarchical MoE) and
  g = 1 + i for the secondary gate of group i
  pair a = (r0, r1) feeds experts 4q+0 (cosine) and 4q+1 (sine),
  pair b = (r2, r3) feeds experts 4q+2 (cosine) and 4q+3 (sine):
     u1 = ((hi >> 11) + 1) * 2^-53        in (0, 1]
     u2 = (lo >> 11) * 2^-53              in [0, 1)
     rho = sqrt(-2 ln u1), theta = 2*pi*u2   (fp64)
     eps = float32(rho * cos(theta)) or float32(rho * sin(theta))

Philox4x64-10 follows Salmon, Moraes, Dror and Shaw, "Parallel random numbers:
as easy as 1, 2, 3" (SC'11): ten rounds of two 64x64->128 multiplies with the
published multipliers, key bumped by the published Weyl increments between
rounds. Box-Muller follows Box and Muller (1958).
"""
from __future__ import annotations

import numpy as np

_M0 = np.uint64(0xD2E7470EE14C6C93)
_M1 = np.uint64(0xCA5A826395121157)
_W0 = np.uint64(0x9E3779B97F4A7C15)
_W1 = np.uint64(0xBB67AE8584CAA73B)
_MASK32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def _mulhilo(a: np.ndarray, m: np.uint64):
    """(high, low) 64-bit halves of the 128-bit product a*m, from 32-bit limbs."""
    a_lo, a_hi = a & _MASK32, a >> _S32
    m_lo, m_hi = m & _MASK32, m >> _S32
    ll = a_lo * m_lo
    lh = a_lo * m_hi
    hl = a_hi * m_lo
    hh = a_hi * m_hi
    mid = (ll >> _S32) + (lh & _MASK32) + (hl & _MASK32)
    hi = hh + (lh >> _S32) + (hl >> _S32) + (mid >> _S32)
    lo = a * m  # wraps modulo 2^64
    return hi, lo


def philox4x64_10(c0, c1, c2, c3, k0, k1):
    """Philox4x64 with 10 rounds on uint64 arrays (broadcast). Returns 4 words."""
    with np.errstate(over="ignore"):
        c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) for c in (c0, c1, c2, c3))
        k0 = np.asarray(k0, dtype=np.uint64)
        k1 = np.asarray(k1, dtype=np.uint64)
        for rnd in range(10):
            if rnd:
                k0 = k0 + _W0
                k1 = k1 + _W1
            hi0, lo0 = _mulhilo(c0, _M0)
            hi1, lo1 = _mulhilo(c2, _M1)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        return c0, c1, c2, c3


_TWO_POW_M53 = 2.0 ** -53
_TWO_PI = 2.0 * np.pi


def _box_muller(a, b):
    u1 = ((a >> np.uint64(11)).astype(np.float64) + 1.0) * _TWO_POW_M53
    u2 = (b >> np.uint64(11)).astype(np.float64) * _TWO_POW_M53
    rho = np.sqrt(-2.0 * np.log(u1))
    theta = _TWO_PI * u2
    return rho * np.cos(theta), rho * np.sin(theta)


def gaussian_noise(seed: int, T: int, E: int, t0: int = 0, key1: int = 0,
                   tokens=None) -> np.ndarray:
    """eps [T, E] fp32 for tokens t0 .. t0+T-1, or for the listed token indices
    (counter-keyed; any slice is reproducible). key1 is the second key word: 0
    for a flat gate and for the primary gate of a hierarchical one, 1 + i for
    the secondary gate of group i (an independent stream per gate)."""
    Q = (E + 3) // 4
    if tokens is None:
        t = np.arange(t0, t0 + T, dtype=np.uint64)[:, None]
    else:
        t = np.asarray(tokens, dtype=np.uint64).reshape(-1, 1)
        T = t.shape[0]
    q = np.arange(Q, dtype=np.uint64)[None, :]
    zero = np.uint64(0)
    r0, r1, r2, r3 = philox4x64_10(t, q, zero, zero, np.uint64(seed), np.uint64(key1))
    ca, sa = _box_muller(r0, r1)
    cb, sb = _box_muller(r2, r3)
    out = np.stack([ca, sa, cb, sb], axis=-1).reshape(T, 4 * Q)[:, :E]
    return out.astype(np.float32)
