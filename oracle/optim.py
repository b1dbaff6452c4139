"""Sketch-space update rules U(S) (TEST INFRASTRUCTURE ONLY).

[LoGRA] Sketch: the weight update is W <- W - alpha eta U A, where U equals
the sketch S in the basic SGD variant; the pages add that stateful sketch
optimizers keep state of their own (extra storage), without defining one.

PARITY UNPINNED: the pages define no stateful rule.  The two rules below are
the plainest reading - the textbook optimizers applied entrywise to the d x r
sketch instead of the d x k gradient - and their arithmetic is pinned against
closed forms (tests/test_oracle_optim.py), not against the pages.

  rule 0  SGD       U = S
  rule 1  momentum  m <- beta1 m + S;  U = m            (heavy ball, no dampening)
  rule 2  Adam      m <- beta1 m + (1 - beta1) S
                    v <- beta2 v + (1 - beta2) S^2
                    U = (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
                    t = 1, 2, ... the step number            [KINGMA15]
All arithmetic is fp64 on the beta / eps values as given (a caller comparing
with an fp32 interface passes the fp32-rounded values).  State arrays are
updated in place.

[KINGMA15] Kingma & Ba, "Adam: A Method for Stochastic Optimization", ICLR 2015,
           Algorithm 1.
"""
import numpy as np

SGD = 0
MOMENTUM = 1
ADAM = 2


def step(rule, S, m=None, v=None, beta1=0.9, beta2=0.999, eps=1e-8, t=1):
    """One update: returns U (fp64 d x r); m and v (fp64 arrays) change in place."""
    S = np.asarray(S, np.float64)
    if rule == SGD:
        return S.copy()
    if rule == MOMENTUM:
        m *= beta1
        m += S
        return m.copy()
    if rule == ADAM:
        if t < 1:
            raise ValueError("Adam step numbers start at 1")
        m *= beta1
        m += (1.0 - beta1) * S
        v *= beta2
        v += (1.0 - beta2) * S * S
        m_hat = m / (1.0 - beta1 ** t)
        v_hat = v / (1.0 - beta2 ** t)
        return m_hat / (np.sqrt(v_hat) + eps)
    raise ValueError(f"unknown rule {rule}")
