"""Philox4x64-10 counter-based generator (TEST INFRASTRUCTURE ONLY).

The pages fix only that A is drawn independently of the batch, kept fixed
while S accumulates, never learned ([LoGRA] Sketch) and that the rollout side
rebuilds it from a seed ([LoGRA] Sync).  They do not name a generator.  The
reading taken here is the published Philox4x64 with 10 rounds [SALMON11]:

  state: counter (x0, x1, x2, x3) and key (k0, k1), all 64-bit words.
  one round: multiply x0 by M0 and x2 by M1 to full 128-bit products,
             then the new state is (hi(M1*x2) ^ x1 ^ k0,  lo(M1*x2),
                                    hi(M0*x0) ^ x3 ^ k1,  lo(M0*x0)).
  between consecutive rounds the key is bumped by the Weyl constants
  (k0 += W0, k1 += W1, modulo 2**64).  Ten rounds give four output words.

`philox4x64_10` is the scalar definition with Python integers (obviously
correct).  `philox4x64_10_np` is the same map over NumPy uint64 arrays, built
from 32-bit limbs because NumPy has no 128-bit integer; tests pin it to the
scalar form and both to NumPy's independent `numpy.random.Philox`.
"""
import numpy as np

MASK64 = (1 << 64) - 1
M0 = 0xD2E7470EE14C6C93
M1 = 0xCA5A826395121157
W0 = 0x9E3779B97F4A7C15
W1 = 0xBB67AE8584CAA73B
ROUNDS = 10


def philox4x64_10(ctr, key):
    """Philox4x64-10 of one 4-word counter under a 2-word key (Python ints)."""
    x0, x1, x2, x3 = (int(c) & MASK64 for c in ctr)
    k0, k1 = (int(c) & MASK64 for c in key)
    for rnd in range(ROUNDS):
        if rnd:
            k0 = (k0 + W0) & MASK64
            k1 = (k1 + W1) & MASK64
        p0 = M0 * x0
        p1 = M1 * x2
        x0, x1, x2, x3 = ((p1 >> 64) ^ x1 ^ k0, p1 & MASK64,
                          (p0 >> 64) ^ x3 ^ k1, p0 & MASK64)
    return x0, x1, x2, x3


_L32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def _mulhilo(a, b):
    """(hi, lo) 64-bit halves of the 128-bit product of constant a and array b."""
    a_lo = np.uint64(a & 0xFFFFFFFF)
    a_hi = np.uint64(a >> 32)
    b_lo = b & _L32
    b_hi = b >> _S32
    ll = a_lo * b_lo
    lh = a_lo * b_hi
    hl = a_hi * b_lo
    hh = a_hi * b_hi
    mid = (ll >> _S32) + (lh & _L32) + (hl & _L32)     # < 3 * 2**32, no wrap
    lo = (ll & _L32) | ((mid & _L32) << _S32)
    hi = hh + (lh >> _S32) + (hl >> _S32) + (mid >> _S32)
    return hi, lo


def philox4x64_10_np(x0, x1, x2, x3, k0, k1):
    """Vectorised Philox4x64-10; counter words are broadcastable uint64 arrays."""
    x0, x1, x2, x3 = (np.asarray(v, dtype=np.uint64) for v in (x0, x1, x2, x3))
    x0, x1, x2, x3 = np.broadcast_arrays(x0, x1, x2, x3)
    k0 = np.uint64(int(k0) & MASK64)
    k1 = np.uint64(int(k1) & MASK64)
    w0, w1 = np.uint64(W0), np.uint64(W1)
    with np.errstate(over="ignore"):
        for rnd in range(ROUNDS):
            if rnd:
                k0 = k0 + w0
                k1 = k1 + w1
            hi0, lo0 = _mulhilo(M0, x0)
            hi1, lo1 = _mulhilo(M1, x2)
            x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return x0, x1, x2, x3
