"""Sketch accumulation S = G A^T (TEST INFRASTRUCTURE ONLY).

[LoGRA] Sketch: for a d x k weight, the method keeps an r x k projection A and
accumulates the d x r sketch S = G A^T in fp32 instead of the d x k gradient
G; each microbatch's contribution is added to S by projecting the inputs of the
weight-gradient product first and only then multiplying with the backward
derivatives, so no full gradient buffer is formed.  [EVAL] section 3 describes
the same mechanism (sketch accumulated during backward, not compressed after).

With Y = X W^T, the weight gradient of one microbatch is G_mb = dY^T X, hence
    S += dY^T (X A^T)   ("input-first"),   equal in exact arithmetic to
    S += (dY^T X) A^T   ("brute force", forms G; used only as a check).
All arithmetic here is fp64 on the exact bf16 input values.
"""
import numpy as np


def weight_gradient(X, dY):
    """G = dY^T X (d x k), the dense gradient the method avoids forming."""
    return np.asarray(dY, np.float64).T @ np.asarray(X, np.float64)


def sketch_brute_force(X, dY, A):
    """G A^T with G formed explicitly."""
    return weight_gradient(X, dY) @ np.asarray(A, np.float64).T


def project_inputs(X, A):
    """P = X A^T (T x r): the projected layer inputs."""
    return np.asarray(X, np.float64) @ np.asarray(A, np.float64).T


def sketch_input_first(X, dY, A):
    """dY^T (X A^T): one microbatch's contribution to S, inputs projected first."""
    return np.asarray(dY, np.float64).T @ project_inputs(X, A)


def accumulate(S, microbatches, A):
    """S plus the sum of every microbatch's contribution (plain sum, no 1/n).

    `microbatches` is an iterable of (X, dY) pairs.  Loss scaling, if any,
    is already inside dY.
    """
    S = np.array(S, dtype=np.float64, copy=True)
    for X, dY in microbatches:
        S += sketch_input_first(X, dY, A)
    return S


def accumulator_bytes(d, r):
    """Bytes of the fp32 sketch accumulator S (d x r)."""
    return 4 * d * r


def dense_accumulator_bytes(d, k):
    """Bytes of an fp32 full-gradient accumulator (d x k)."""
    return 4 * d * k
