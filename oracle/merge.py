"""Rank-r merge into the bf16 weights (TEST INFRASTRUCTURE ONLY).

[LoGRA] Sketch: the update is W <- W - alpha * eta * U A, where U equals S in
the basic SGD variant and alpha is the step-size multiplier chosen by the
controller; the update is merged directly into the weights, with no adapter
branch kept around.  [LoGRA] Sync: the rollout side receives alpha*eta*U and
the seed, rebuilds A and applies the same merge.

Reading: W is stored in bf16 and the new W is W - alpha*eta*(S A) computed in
exact (here fp64) arithmetic and rounded ONCE to bf16, ties to even.  alpha
and eta are fp32 scalars; their product is taken in fp64 here.
"""
import numpy as np

from .bf16 import bits_to_f64, f64_to_bits


def update_direction(S, A):
    """U A with U = S (basic SGD variant): the d x k rank-r direction."""
    return np.asarray(S, np.float64) @ np.asarray(A, np.float64)


def merge_bits(W_bits, S, A, alpha, eta):
    """New bf16 bits of W after W <- RNE_bf16(W - alpha*eta*S A)."""
    step = float(np.float32(alpha)) * float(np.float32(eta))
    W = bits_to_f64(W_bits)
    return f64_to_bits(W - step * update_direction(S, A))


def merged_delta(W_bits, S, A, alpha, eta):
    """W_new - W_old in fp64 (the rounded delta the GPU result is compared to)."""
    return bits_to_f64(merge_bits(W_bits, S, A, alpha, eta)) - bits_to_f64(W_bits)
