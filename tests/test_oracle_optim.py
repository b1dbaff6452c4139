"""Pins of the oracle's sketch-space update rules (oracle/optim.py).

The pages define no stateful rule (parity unpinned); these tests pin the
textbook momentum / Adam arithmetic the oracle restates, against closed forms
and a hand-worked two-step example, so a dropped bias correction, a missing
(1 - beta) factor, a missing square root or a sign error fails here.
"""
import math

import numpy as np
import pytest

from oracle import optim


def _rng(seed):
    return np.random.default_rng(seed)


def test_sgd_is_the_sketch():
    S = _rng(1).standard_normal((7, 5))
    U = optim.step(optim.SGD, S)
    np.testing.assert_array_equal(U, S)
    U[0, 0] += 1.0                    # a copy, not a view of S
    assert U[0, 0] != S[0, 0]


def test_momentum_hand_example():
    # beta = 0.5: m1 = S1; m2 = 0.5 m1 + S2
    m = np.zeros((1, 2))
    U1 = optim.step(optim.MOMENTUM, np.array([[2.0, -1.0]]), m, beta1=0.5)
    U2 = optim.step(optim.MOMENTUM, np.array([[0.0, 3.0]]), m, beta1=0.5)
    np.testing.assert_array_equal(U1, [[2.0, -1.0]])
    np.testing.assert_array_equal(U2, [[1.0, 2.5]])


def test_momentum_constant_sketch_is_a_geometric_series():
    S = _rng(2).standard_normal((4, 3))
    beta = 0.9
    m = np.zeros_like(S)
    for n in range(1, 30):
        U = optim.step(optim.MOMENTUM, S, m, beta1=beta)
        np.testing.assert_allclose(U, S * (1 - beta ** n) / (1 - beta), rtol=1e-13)


def test_momentum_beta_zero_and_linearity():
    rng = _rng(3)
    seq1 = [rng.standard_normal((5, 4)) for _ in range(6)]
    seq2 = [rng.standard_normal((5, 4)) for _ in range(6)]
    m0 = np.zeros((5, 4))
    for S in seq1:
        np.testing.assert_array_equal(optim.step(optim.MOMENTUM, S, m0, beta1=0.0), S)
    ma, mb, mc = np.zeros((5, 4)), np.zeros((5, 4)), np.zeros((5, 4))
    for S1, S2 in zip(seq1, seq2):
        Ua = optim.step(optim.MOMENTUM, S1, ma, beta1=0.7)
        Ub = optim.step(optim.MOMENTUM, S2, mb, beta1=0.7)
        Uc = optim.step(optim.MOMENTUM, S1 + S2, mc, beta1=0.7)
        np.testing.assert_allclose(Uc, Ua + Ub, rtol=1e-12, atol=1e-12)


def test_adam_hand_example():
    # beta1 = beta2 = 0.5, eps = 0: U1 = [1, -1]; U2 = [1/sqrt(3), 5/sqrt(57)]
    m, v = np.zeros((1, 2)), np.zeros((1, 2))
    U1 = optim.step(optim.ADAM, np.array([[2.0, -1.0]]), m, v, 0.5, 0.5, 0.0, t=1)
    U2 = optim.step(optim.ADAM, np.array([[0.0, 3.0]]), m, v, 0.5, 0.5, 0.0, t=2)
    np.testing.assert_allclose(U1, [[1.0, -1.0]], rtol=1e-15)
    np.testing.assert_allclose(U2, [[1 / math.sqrt(3), 5 / math.sqrt(57)]], rtol=1e-14)


def test_adam_constant_gradient_gives_the_sign_step():
    # m_t = g (1 - b1^t), v_t = g^2 (1 - b2^t): after bias correction
    # U = g / (|g| + eps) at every step.
    g = _rng(4).standard_normal((6, 4))
    m, v = np.zeros_like(g), np.zeros_like(g)
    for t in range(1, 40):
        U = optim.step(optim.ADAM, g, m, v, 0.9, 0.999, 1e-3, t=t)
        np.testing.assert_allclose(U, g / (np.abs(g) + 1e-3), rtol=1e-9)


def test_adam_first_step_and_symmetries():
    rng = _rng(5)
    S = rng.standard_normal((8, 8))
    for b1, b2 in [(0.9, 0.999), (0.0, 0.0), (0.5, 0.95)]:
        m, v = np.zeros_like(S), np.zeros_like(S)
        U = optim.step(optim.ADAM, S, m, v, b1, b2, 1e-6, t=1)
        np.testing.assert_allclose(U, S / (np.abs(S) + 1e-6), rtol=1e-12)
    seq = [rng.standard_normal((8, 8)) for _ in range(5)]
    st = [(np.zeros((8, 8)), np.zeros((8, 8))) for _ in range(3)]
    for t, S in enumerate(seq, start=1):
        U = optim.step(optim.ADAM, S, *st[0], 0.9, 0.99, 0.0, t=t)
        Un = optim.step(optim.ADAM, -S, *st[1], 0.9, 0.99, 0.0, t=t)
        Us = optim.step(optim.ADAM, 1e3 * S, *st[2], 0.9, 0.99, 0.0, t=t)
        np.testing.assert_allclose(Un, -U, rtol=1e-13)       # odd in S
        np.testing.assert_allclose(Us, U, rtol=1e-12)        # scale-free when eps = 0


def test_adam_rejects_step_zero():
    with pytest.raises(ValueError):
        optim.step(optim.ADAM, np.ones((1, 1)), np.zeros((1, 1)), np.zeros((1, 1)), t=0)
