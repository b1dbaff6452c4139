"""Parity bars shared by the GPU tests (no method arithmetic here).

Frobenius bars of the pages' workloads: 2e-3 relative on the S delta and on
the merged-W delta, 1e-3 relative on q(D).  Beside them, elementwise bars so
that one wrong entry cannot hide in a norm:
  S   every entry of the delta within S_ELEM of the largest oracle entry (the
      hi/lo bf16 pair of P keeps ~16 bits and fp32 sums over the tokens ~20;
      measured differences are ~100x smaller);
  W   every merged element within one bf16 spacing of the oracle's (the single
      rounding of W - alpha eta S A can fall on the other side of a rounding
      boundary: S A is formed in fp32 on the GPU and in fp64 by the oracle),
      plus W_ELEM of the largest delta (where W - alpha eta S A cancels to
      nearly zero, that small fp32/fp64 difference is all that is left).
The Gaussian basis gets looser elementwise bars: its exact values are not
pinned (fp64 Box-Muller in the oracle, fp32 hardware transcendentals on the
GPU), and about 0.1 % of its entries differ by one bf16 spacing (up to 2^-7
relative).  One such entry of A row j moves S column j by up to ~3e-4 of the
largest entry, and every element of a W column that meets it by up to
~0.02 / sqrt(r) of the largest delta (~5e-3 at r = 16).  The bars stay far
below what one wrong entry would cost (order 1).
"""
import numpy as np

S_TOL = 2e-3
W_TOL = 2e-3
Q_TOL = 1e-3
S_ELEM = 1e-4
W_ELEM = 1e-4
S_ELEM_GAUSS = 2e-3
W_ELEM_GAUSS = 1e-2


def s_elem_bar(kind):
    """Elementwise S bar for projection kind 0 (signs) or 1 (Gaussian)."""
    return S_ELEM_GAUSS if kind == 1 else S_ELEM


def w_elem_bar(kind):
    """Elementwise W bar for projection kind 0 (signs) or 1 (Gaussian)."""
    return W_ELEM_GAUSS if kind == 1 else W_ELEM


def rel_fro(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def max_rel(a, b):
    """max |a - b| over max |b|: the largest entry error on the scale of the result."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if b.size == 0:
        return 0.0
    mb = np.abs(b).max()
    return float(np.abs(a - b).max() / (mb if mb > 0 else 1.0))


def _bits_to_f64(bits):
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_spacing(x):
    """Distance from |x| to the next larger bf16 value (0 for x = 0)."""
    m = np.abs(np.asarray(x, np.float64))
    _, e = np.frexp(m)                      # m = f 2^e, f in [0.5, 1)
    return np.where(m > 0, np.ldexp(1.0, e - 8), 0.0)


def w_excess(bits_gpu, bits_ref, delta_ref):
    """Largest elementwise |W_gpu - W_ref| beyond one bf16 spacing, over the
    largest |oracle delta| (the W bar is w_excess <= W_ELEM)."""
    a = _bits_to_f64(bits_gpu)
    b = _bits_to_f64(bits_ref)
    if a.size == 0:
        return 0.0
    sp = bf16_spacing(np.maximum(np.abs(a), np.abs(b)))
    over = np.maximum(np.abs(a - b) - sp, 0.0)
    md = np.abs(np.asarray(delta_ref, np.float64)).max()
    return float(over.max() / (md if md > 0 else 1.0))
