"""Model-space recurrence in FP64, product form.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

"DAMP: Decay-Aware Mixed-Precision Recurrent-State Quantization" (arXiv
2608.27513, HTML), section 3.1, Eq.(2):

    S_t = A_t S_{t-1} + beta_t k_t v_t^T,   A_t = (I - beta_t k_t k_t^T) Lambda_t,
    o_t = S_t^T q_t,

with Lambda_t = alpha_t I for GDN (kind 0), diag(exp(g_t)) for KDA (kind 1),
and diag(lambda_t) for KDA with the decay factors given (kind 2).  This is written
with an explicit transition matrix and numpy matrix products, independently
of the delta form used by the C oracle, so that the two pin each other.

The quantized trajectory of section 3.3, Eq.(4), and the error identity
Eqs.(5)-(6) are expressed with the same transition matrices.
"""
from __future__ import annotations

import numpy as np


def transition(k, gate, beta, kind):
    """A_t = (I - beta k k^T) Lambda_t for one head, FP64."""
    k = np.asarray(k, dtype=np.float64)
    d = k.shape[0]
    if kind == 0:
        lam = np.full(d, float(gate))
    elif kind == 1:
        lam = np.exp(np.asarray(gate, dtype=np.float64))
    else:
        lam = np.asarray(gate, dtype=np.float64)
    return (np.eye(d) - float(beta) * np.outer(k, k)) @ np.diag(lam)


def step(S, q, k, v, gate, beta, kind):
    """One product-form step of one head: returns (S_t, o_t, A_t)."""
    A = transition(k, gate, beta, kind)
    S_new = A @ np.asarray(S, dtype=np.float64) + float(beta) * np.outer(
        np.asarray(k, dtype=np.float64), np.asarray(v, dtype=np.float64))
    o = S_new.T @ np.asarray(q, dtype=np.float64)
    return S_new, o, A


def run(S0, qs, ks, vs, gates, betas, kind):
    """Trajectory of one head over len(qs) steps.

    Returns (states [T+1][dk][dv], outputs [T][dv], transitions [T][dk][dk]).
    """
    S = np.asarray(S0, dtype=np.float64)
    states = [S]
    outs = []
    As = []
    for t in range(len(qs)):
        S, o, A = step(S, qs[t], ks[t], vs[t], gates[t], betas[t], kind)
        states.append(S)
        outs.append(o)
        As.append(A)
    return np.stack(states), np.stack(outs), np.stack(As)
