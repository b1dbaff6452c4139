"""The seeded projection A (r x k) (TEST INFRASTRUCTURE ONLY).

What the pages fix ([LoGRA] Sketch; [LoGRA] Sync; [LoGRA] Rank):
  * A is r x k, drawn independently of the batch, held fixed while S
    accumulates and never learned;
  * by default its entries are independent random signs scaled by 1/sqrt(r);
  * the design study also uses a per-step refreshed sign basis and a
    refreshed Gaussian basis;
  * the rollout engine rebuilds A from the seed instead of receiving it.

Readings taken where the pages are silent:
  * generator: Philox4x64-10 [SALMON11] keyed by (seed, stream); "stream" is
    the refresh index (0 for the fixed basis, the step number for a refreshed
    basis).
  * Rademacher layout: one Philox block per (row i, 256-column group):
        counter = (j >> 8, i, 0, 0), key = (seed, stream)
    column j takes bit (j & 63) of output word ((j >> 6) & 3); a set bit means
    a negative entry.  Entry value is +-c with c = 1/sqrt(r) rounded once to
    fp32.
  * Gaussian layout: one Philox block per (row i, 4-column group):
        counter = (j >> 2, i, 1, 0), key = (seed, stream)
    each output word w gives a uniform u = (2 * (w >> 41) + 1) * 2**-24 in
    (0, 1) (24 significant bits, exact in fp32); Box-Muller [BOXMULLER58]
    turns (u0, u1) into columns 4q, 4q+1 and (u2, u3) into 4q+2, 4q+3:
        R = sqrt(-2 ln u_even),  z_even = R cos(2 pi u_odd),
                                 z_odd  = R sin(2 pi u_odd);
    the stored entry is z / sqrt(r) rounded once to bf16 (N(0, 1/r)).
"""
import numpy as np

from .bf16 import round_f64
from .philox import philox4x64_10_np

RADEMACHER = 0
GAUSSIAN = 1


def rademacher_scale(r):
    """c = 1/sqrt(r), computed in fp64 and rounded once to fp32 (as float)."""
    return float(np.float32(1.0 / np.sqrt(float(r))))


def sign_bits(seed, stream, r, k):
    """uint8 r x k matrix of sign bits (1 = negative entry) of the sign basis."""
    n_blocks = (k + 255) // 256
    bi = np.arange(n_blocks, dtype=np.uint64)[None, :]
    ri = np.arange(r, dtype=np.uint64)[:, None]
    w = philox4x64_10_np(bi, ri, np.uint64(0), np.uint64(0), seed, stream)
    words = np.stack(w, axis=-1)                     # r x n_blocks x 4
    j = np.arange(k)
    sel = words[:, j >> 8, (j >> 6) & 3]             # r x k
    return ((sel >> (j & 63).astype(np.uint64)) & np.uint64(1)).astype(np.uint8)


def gaussian_normals(seed, stream, r, k):
    """fp64 r x k standard normals from the Gaussian layout (before scaling)."""
    n_groups = (k + 3) // 4
    qi = np.arange(n_groups, dtype=np.uint64)[None, :]
    ri = np.arange(r, dtype=np.uint64)[:, None]
    w = philox4x64_10_np(qi, ri, np.uint64(1), np.uint64(0), seed, stream)
    u = [((wa >> np.uint64(41)).astype(np.float64) * 2.0 + 1.0) * 2.0 ** -24
         for wa in w]
    rad0 = np.sqrt(-2.0 * np.log(u[0]))
    rad1 = np.sqrt(-2.0 * np.log(u[2]))
    z = np.stack([rad0 * np.cos(2.0 * np.pi * u[1]),
                  rad0 * np.sin(2.0 * np.pi * u[1]),
                  rad1 * np.cos(2.0 * np.pi * u[3]),
                  rad1 * np.sin(2.0 * np.pi * u[3])], axis=-1)   # r x groups x 4
    return z.reshape(r, 4 * n_groups)[:, :k]


def projection(seed, stream, kind, r, k):
    """A as an fp64 r x k array, exactly the values the method multiplies by."""
    if kind == RADEMACHER:
        c = rademacher_scale(r)
        return np.where(sign_bits(seed, stream, r, k) == 1, -c, c)
    if kind == GAUSSIAN:
        return round_f64(gaussian_normals(seed, stream, r, k) / np.sqrt(float(r)))
    raise ValueError("kind must be 0 (Rademacher) or 1 (Gaussian)")
