"""Oracle for the offline choice of the FP16 key channels (the DAMP layout).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  Shares no code with
the HIP library.

Sources: "DAMP: Decay-Aware Mixed-Precision Recurrent-State Quantization"
(arXiv 2608.27513, HTML), section 4 "Key-channel budget", "Accumulated-error
risk" and "Budgeted selection" (Eqs.(7)-(10)), Appendix A.2 (calibration,
Eqs.(13)-(15), tau = 1e-4), Appendix A.3 (decay-based persistence, Eq.(16)),
Appendix A.4 (Algorithm 1, offline layout construction); and the reading
notes on its v2, section 2.5 (e_{t,u}, the finite-horizon weight W_{t,u} with
H = 256, C_u = E_cal[e W]).

Steps, in the pages' order:
  1. e[s, h, u]: squared error of key channel u of calibration state s under
     the INT8 storage mapping (Eq.(14) integrand; v2 notes e_{t,u}) --
     ``channel_error`` (the arithmetic is in qrs_oracle.c).
  2. Persistence of an error injected in channel u:
       HTML: a_eff = exp(E_cal[log a]), P = 1 / max(1 - a_eff^2, tau)
             (Eq.(15)) -- ``persistence_geometric``;
       v2:   W[s, h, u] = 1 + sum_{j=1..H} prod_{r=1..j} a_{t+r,u}^2 over the
             same trajectory's next H decays -- ``persistence_window``.
  3. Score: HTML C = E_cal[e] * P (Eq.(10) with Eqs.(14)-(15)); v2
     C = E_cal[e W], multiplied per sample before averaging --
     ``channel_scores``.  E_cal is the domain-balanced mean of Eq.(13)
     (``domain_weights``).
  4. Top-16 key channels per head, and the permutation by a stable partition
     that puts them first (Algorithm 1) -- ``select_protected``.

Readings where the pages leave a step open (listed in the design notes):
  * the v2 window stops at the end of the trajectory (a sample with fewer
    than H later steps sums the ones it has);
  * the decay a_{x,t,u} paired with a sampled state write is the one applied
    at that write (Lambda_t of the step that produced S_t);
  * equal scores rank the lower key-channel index first.
"""
from __future__ import annotations

import numpy as np

from . import DK, _f32, _ptr, load


def channel_error(S: np.ndarray, c: np.ndarray | None = None) -> np.ndarray:
    """e [n][H][DK] (FP64) for calibration states S [n][H][DK][DV] in model
    coordinates and smoothing scales c [H][DV] (None = ones)."""
    S = _f32(S)
    n, H = S.shape[0], S.shape[1]
    e = np.zeros((n, H, DK), np.float64)
    cc = None if c is None else _f32(c)
    load().orc_channel_error(_ptr(S), n, H, None if cc is None else _ptr(cc), _ptr(e))
    return e


def domain_weights(domains) -> np.ndarray:
    """Per-sample weights of the domain-balanced mean (HTML Eq.(13)):
    w_s = 1 / (|D| |Omega_d(s)|)."""
    domains = np.asarray(domains)
    labels, counts = np.unique(domains, return_counts=True)
    size = dict(zip(labels.tolist(), counts.tolist()))
    return np.array([1.0 / (len(labels) * size[d]) for d in domains.tolist()], np.float64)


def persistence_window(a_traj: np.ndarray, sample_seq, sample_t, horizon: int) -> np.ndarray:
    """v2 notes section 2.5: W[s, h, u] = 1 + sum_{j=1..horizon}
    prod_{r=1..j} a[seq_s, t_s + r, h, u]^2, the sum stopping at the end of
    the trajectory.  a_traj: [n_seq][T][H][DK] decays."""
    a = np.asarray(a_traj, np.float32)
    T = a.shape[1]
    n = len(sample_seq)
    W = np.empty((n, a.shape[2], DK), np.float64)
    for s in range(n):
        x, t = int(sample_seq[s]), int(sample_t[s])
        p = np.ones((a.shape[2], DK), np.float64)
        acc = np.ones((a.shape[2], DK), np.float64)
        for j in range(1, horizon + 1):
            if t + j >= T:
                break
            aj = a[x, t + j].astype(np.float64)
            p = p * (aj * aj)
            acc = acc + p
        W[s] = acc
    return W


def persistence_geometric(a_traj: np.ndarray, sample_seq, sample_t, weight,
                          tau: float = 1e-4) -> np.ndarray:
    """HTML Eq.(15): a_eff = exp(E_cal[log a]) over the sampled writes,
    P = 1 / max(1 - a_eff^2, tau).  Returns P [H][DK]."""
    a = np.asarray(a_traj, np.float32)
    L = np.zeros((a.shape[2], DK), np.float64)
    for s in range(len(sample_seq)):
        if weight[s] == 0:
            continue
        with np.errstate(divide="ignore"):
            L = L + weight[s] * np.log(a[int(sample_seq[s]), int(sample_t[s])].astype(np.float64))
    a_eff = np.exp(L)
    return 1.0 / np.maximum(1.0 - a_eff * a_eff, tau)


def channel_scores(e: np.ndarray, weight, W: np.ndarray | None = None,
                   P: np.ndarray | None = None) -> np.ndarray:
    """Key-channel risk C [H][DK].  With W (v2 notes): C = sum_s w_s e_s W_s,
    each sample's product formed before the average.  With P (HTML
    Eqs.(14)-(15)): C = (sum_s w_s e_s) P."""
    assert (W is None) != (P is None), "give exactly one of W and P"
    acc = np.zeros(e.shape[1:], np.float64)
    for s in range(e.shape[0]):
        term = weight[s] * e[s]
        if W is not None:
            term = term * W[s]
        acc = acc + term
    return acc if W is not None else acc * P


def select_protected(score: np.ndarray, k_hi: int = 16):
    """Algorithm 1: per head, the k_hi key channels of largest score (ties to
    the lower index), and the permutation placing them first, each part in
    ascending channel order.  Returns (protected [H][k_hi], perm [H][DK])."""
    H = score.shape[0]
    prot = np.empty((H, k_hi), np.int32)
    perm = np.empty((H, DK), np.int32)
    for h in range(H):
        ranked = sorted(range(DK), key=lambda u: (-float(score[h, u]), u))
        chosen = sorted(ranked[:k_hi])
        rest = [u for u in range(DK) if u not in set(chosen)]
        prot[h] = chosen
        perm[h] = chosen + rest
    return prot, perm
