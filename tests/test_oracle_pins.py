"""Known-answer pins of the oracle that tie it to sources outside itself.

- q(D) is the MEAN of the per-row forward KLs ([LoGRA] PKL: the controller
  works on the mean predicted KL over the sampled responses' token
  positions).  Rows over a two-word vocabulary have a closed-form KL (the
  Bernoulli KL), so q is checked against the average of those closed forms,
  with rows chosen so that a sum, a KL of the averaged distributions or a
  reverse KL all miss it.
- The projection A's layout (counter, output word and bit per entry) is
  recomputed here entry by entry from NumPy's own Philox4x64-10
  (`numpy.random.Philox`, an implementation independent of oracle.philox),
  following the layout the library documents for its sign and Gaussian bases
  ([LoGRA] Sketch: entries are random signs scaled by 1/sqrt(r); [LoGRA]
  Rank: the Gaussian basis).  NumPy's first block for counter c is the Philox
  block at counter c + 1, so every counter below is passed minus one.
"""
import math

import numpy as np
import pytest

from oracle import kl
from oracle import projection


# ------------------------------------------------------------ q(D) is a mean

def _bernoulli_kl(a, b):
    """KL(softmax([0, a]) || softmax([0, b])) in closed form."""
    p = 1.0 / (1.0 + math.exp(-a))
    q = 1.0 / (1.0 + math.exp(-b))
    return p * math.log(p / q) + (1.0 - p) * math.log((1.0 - p) / (1.0 - q))


def test_predicted_kl_is_the_mean_of_bernoulli_rows():
    tau = 2.0
    # rows [0, a_t] -> [0, b_t] (the common zero column makes the softmax of
    # each row a Bernoulli with logit a / tau); distinct KLs per row
    a = [1.3, -0.6, 2.9, 0.1]
    b = [0.2, 0.8, 3.5, -1.7]
    z = np.array([[0.0, x] for x in a])
    zp = np.array([[0.0, x] for x in b])
    rows = [_bernoulli_kl(x / tau, y / tau) for x, y in zip(a, b)]
    q = kl.predicted_kl(z, zp, tau)
    want = sum(rows) / len(rows)
    assert abs(q - want) <= 1e-14 * want
    # what a plausible slip would give instead is far away
    assert abs(sum(rows) - want) > 1.0 * want                     # sum, not mean
    pa = np.mean([1 / (1 + math.exp(-x / tau)) for x in a])       # KL of the averages
    pb = np.mean([1 / (1 + math.exp(-y / tau)) for y in b])
    kl_avg = pa * math.log(pa / pb) + (1 - pa) * math.log((1 - pa) / (1 - pb))
    assert abs(kl_avg - want) > 0.2 * want
    rev = sum(_bernoulli_kl(y / tau, x / tau) for x, y in zip(a, b)) / len(a)
    assert abs(rev - want) > 0.01 * want                          # reverse KL
    no_tau = sum(_bernoulli_kl(x, y) for x, y in zip(a, b)) / len(a)
    assert abs(no_tau - want) > 0.2 * want                        # temperature dropped
    # equal weight per row: repeating one row moves the mean accordingly
    z5 = np.vstack([z, z[2:3]])
    zp5 = np.vstack([zp, zp[2:3]])
    assert abs(kl.predicted_kl(z5, zp5, tau) - (sum(rows) + rows[2]) / 5) <= 1e-14 * want


# ------------------------------------------------- A's layout, entry by entry

def _numpy_block(c0, c1, c2, c3, seed, stream):
    """Philox4x64-10 block at counter (c0, c1, c2, c3), key (seed, stream), from
    NumPy (c0 >= 1, so subtracting one never borrows)."""
    assert c0 >= 1
    bg = np.random.Philox(counter=np.array([c0 - 1, c1, c2, c3], dtype=np.uint64),
                          key=np.array([seed, stream], dtype=np.uint64))
    return [int(w) for w in bg.random_raw(4)]


# (seed, stream, r, k, entries (i, j)); columns >= 256 (sign) / >= 4 (Gaussian)
SIGN_CASES = [
    (1234, 0, 64, 4096, [(0, 256), (0, 4095), (63, 300), (17, 1023), (5, 3333), (40, 2048)]),
    (1234 + 27, 3, 256, 25600, [(255, 25599), (128, 256), (1, 12345), (200, 777)]),
    (2**64 - 1, 2**63 + 1, 4, 1536, [(3, 511), (0, 1535), (2, 1280)]),
]


@pytest.mark.parametrize("seed,stream,r,k,entries", SIGN_CASES)
def test_sign_basis_entries_from_numpy_philox(seed, stream, r, k, entries):
    A = projection.projection(seed, stream, projection.RADEMACHER, r, k)
    c = float(np.float32(1.0 / math.sqrt(r)))
    for i, j in entries:
        words = _numpy_block(j // 256, i, 0, 0, seed, stream)   # one block per 256 columns
        word = words[(j % 256) // 64]                            # 64 columns per word
        bit = (word >> (j % 64)) & 1                             # set bit = negative
        assert A[i, j] == (-c if bit else c), (i, j)


GAUSS_CASES = [
    (1234, 0, 64, 4096, [(0, 4), (0, 5), (0, 6), (0, 7), (63, 4095), (31, 2050), (9, 1001)]),
    (1234 + 5, 2, 256, 8960, [(255, 8959), (100, 4), (7, 6003)]),
]


def _bf16_neighbours(x):
    """The two bf16 values around x (bf16 = the top 16 bits of an fp32)."""
    f = np.float32(x)
    bits = int(np.array(f, np.float32).view(np.uint32))
    lo = np.array((bits & 0xFFFF0000) & 0xFFFFFFFF, np.uint32).view(np.float32)
    hi = np.array(((bits & 0xFFFF0000) + 0x10000) & 0xFFFFFFFF, np.uint32).view(np.float32)
    return sorted([float(lo), float(hi)])


@pytest.mark.parametrize("seed,stream,r,k,entries", GAUSS_CASES)
def test_gaussian_basis_entries_from_numpy_philox(seed, stream, r, k, entries):
    A = projection.projection(seed, stream, projection.GAUSSIAN, r, k)
    for i, j in entries:
        w = _numpy_block(j // 4, i, 1, 0, seed, stream)          # one block per 4 columns
        u = [((x >> 41) * 2 + 1) * 2.0 ** -24 for x in w]        # 24-bit uniforms in (0, 1)
        pair = (j % 4) // 2                                      # (u0, u1) or (u2, u3)
        rad = math.sqrt(-2.0 * math.log(u[2 * pair]))
        ang = 2.0 * math.pi * u[2 * pair + 1]
        z = rad * (math.cos(ang) if j % 2 == 0 else math.sin(ang))
        want = z / math.sqrt(r)
        # the stored entry is want rounded to bf16: one of its two neighbours,
        # the nearer one unless want sits within fp64 noise of the midpoint
        lo, hi = _bf16_neighbours(want)
        assert A[i, j] in (lo, hi), (i, j)
        nearer = lo if abs(want - lo) <= abs(hi - want) else hi
        if abs(abs(want - lo) - abs(hi - want)) > 1e-12 * abs(want):
            assert A[i, j] == nearer, (i, j)
