"""Pins of the key-channel selection oracle (oracle/selector.py) against what
the pages print and what the mathematics fixes.

Sources: DAMP arXiv HTML, section 4 (Eqs.(8)-(10)), Appendix A.2
(Eqs.(13)-(15), tau = 1e-4), A.3 (Eq.(16)), A.4 (Algorithm 1); v2 reading
notes, section 2.5 (e_{t,u}, W_{t,u}, worked example with H = 256).
"""
import math

import numpy as np

import oracle
from oracle import selector as sel

DK = DV = 128


def _const_traj(a, T=300, H=1):
    return np.full((1, T, H, DK), a, np.float32)


# ---------------------------------------------------------------------------
# persistence
# ---------------------------------------------------------------------------

def test_window_printed_example():
    """v2 notes section 2.5: for a constant per-step decay a and H = 256,
    W = (1 - a^(2(H+1))) / (1 - a^2); the notes print W ~ 1.33 for a = 0.5 and
    W ~ 49.96 for a = 0.99, a ratio of about 37.5."""
    w05 = sel.persistence_window(_const_traj(0.5), [0], [0], 256)[0, 0, 0]
    assert abs(w05 - (1 - 0.25 ** 257) / 0.75) <= 1e-15 * w05
    assert round(w05, 2) == 1.33
    a = float(np.float32(0.99))
    w99 = sel.persistence_window(_const_traj(0.99), [0], [0], 256)[0, 0, 0]
    assert abs(w99 - (1 - a ** 514) / (1 - a * a)) <= 1e-12 * w99
    assert round(w99, 2) == 49.96
    assert round(w99 / w05, 1) == 37.5


def test_window_bruteforce_and_truncation():
    """Explicit products on a random trajectory, and the window stopping at
    the last step of the trajectory."""
    r = np.random.default_rng(5)
    a = r.uniform(0.3, 1.0, (2, 12, 3, DK)).astype(np.float32)
    seqs, ts, horizon = [0, 1, 1], [2, 0, 9], 6
    W = sel.persistence_window(a, seqs, ts, horizon)
    for s, (x, t) in enumerate(zip(seqs, ts)):
        for h in range(3):
            for u in (0, 17, 127):
                want = 1.0
                for j in range(1, horizon + 1):
                    if t + j >= a.shape[1]:
                        break
                    want += math.prod(float(a[x, t + r_, h, u]) ** 2 for r_ in range(1, j + 1))
                assert abs(W[s, h, u] - want) <= 1e-13 * want
    # t = 9 of T = 12: only steps 10 and 11 remain
    x, t = 1, 9
    a10, a11 = a[x, 10, 0, 5].astype(np.float64), a[x, 11, 0, 5].astype(np.float64)
    assert abs(W[2, 0, 5] - (1 + a10 ** 2 + a10 ** 2 * a11 ** 2)) <= 1e-15 * W[2, 0, 5]


def test_geometric_persistence_cap_and_mean():
    """Eq.(15) with tau = 1e-4: a_eff = 1 hits the cap 1/tau; a_eff = 0 gives
    1; the decay is averaged geometrically (a = 0.25 and 1 give a_eff = 0.5,
    P = 4/3, where an arithmetic mean would give 1/(1 - 0.625^2))."""
    one = sel.persistence_geometric(_const_traj(1.0), [0, 0], [3, 4], [0.5, 0.5])
    assert np.all(one == 1e4)
    zero = sel.persistence_geometric(_const_traj(0.0), [0], [3], [1.0])
    assert np.all(zero == 1.0)
    a = _const_traj(0.25)
    a[0, 7] = 1.0
    P = sel.persistence_geometric(a, [0, 0], [3, 7], [0.5, 0.5])
    assert np.allclose(P, 4.0 / 3.0, rtol=1e-15, atol=0)
    # Appendix A.3: P is the infinite-horizon limit of the window weight
    W = sel.persistence_window(_const_traj(0.5), [0], [0], 256)
    assert np.allclose(W[0], sel.persistence_geometric(_const_traj(0.5), [0], [0], [1.0]),
                       rtol=1e-15, atol=0)


def test_domain_weights():
    """Eq.(13): every domain carries 1/|D| of the mass, split evenly over its
    samples."""
    w = sel.domain_weights([0, 0, 0, 1])
    assert np.allclose(w, [1 / 6, 1 / 6, 1 / 6, 1 / 2], rtol=1e-15, atol=0)
    assert abs(w.sum() - 1) < 1e-15


# ---------------------------------------------------------------------------
# quantization-error energy
# ---------------------------------------------------------------------------

def test_channel_error_closed_forms():
    S = np.zeros((1, 2, DK, DV), np.float32)
    S[0, 0, 1, :32] = np.arange(-16, 16)          # integers, amax 16 -> s = 16/127
    S[0, 0, 2, :32] = np.arange(-127, 128, 8)[:32]  # integers with |max| 127 -> s = 1, exact
    S[0, 0, 2, 0] = -127
    S[0, 0, 3, 0], S[0, 0, 3, 1] = 127, 0.5      # 0.5 ties to code 0: error 0.25
    S[0, 0, 4, 40], S[0, 0, 4, 41] = 127, 1.5    # 1.5 ties to code 2: error 0.25
    S[0, 0, 4, 100] = -127                       # another group, exact
    S[0, 1, 3, 0], S[0, 1, 3, 1] = 254, 1.0      # head 1: c = 2 on every column
    c = np.ones((2, DV), np.float32)
    c[1] = 2
    e = sel.channel_error(S, c)
    assert e[0, 0, 0] == 0 and e[0, 0, 2] == 0
    assert e[0, 0, 3] == 0.25 and e[0, 0, 4] == 0.25
    assert e[0, 1, 3] == 1.0                     # c^2 * 0.25: error measured in model coordinates
    # row 1 against the pinned group codec, error summed in FP64
    codes, s = oracle.quantize_group(S[0, 0, 1, :32])
    want = sum((float(np.float32(s) * np.float32(cd)) - float(x)) ** 2
               for cd, x in zip(codes, S[0, 0, 1, :32]))
    assert abs(e[0, 0, 1] - want) <= 1e-15 * want


def test_channel_error_smoothing_and_groups():
    """A random state: the error equals the sum over the four 32-value groups
    of the pinned codec's error in stored value coordinates, mapped back by c."""
    r = np.random.default_rng(9)
    S = r.normal(0, 1, (2, 1, DK, DV)).astype(np.float32)
    c = np.exp(r.uniform(np.log(0.5), np.log(2), (1, DV))).astype(np.float32)
    e = sel.channel_error(S, c)
    for n_ in range(2):
        for u in (0, 63, 127):
            x = S[n_, 0, u] / c[0]
            want = 0.0
            for g in range(4):
                codes, s = oracle.quantize_group(x[32 * g:32 * g + 32])
                back = (np.float32(s) * codes.astype(np.float32)) * c[0, 32 * g:32 * g + 32]
                want += float(np.sum((back.astype(np.float64) - S[n_, 0, u, 32 * g:32 * g + 32]) ** 2))
            assert abs(e[n_, 0, u] - want) <= 1e-13 * want


# ---------------------------------------------------------------------------
# scores and selection
# ---------------------------------------------------------------------------

def test_window_score_multiplies_before_averaging():
    """v2 notes section 2.5: C = E[e W], not E[e] E[W]."""
    e = np.zeros((2, 1, DK))
    W = np.ones((2, 1, DK))
    e[0, 0, 0], W[1, 0, 0] = 1.0, 100.0
    C = sel.channel_scores(e, [0.5, 0.5], W=W)
    assert C[0, 0] == 0.5
    assert C[0, 0] != np.mean(e[:, 0, 0]) * np.mean(W[:, 0, 0])
    P = np.full((1, DK), 3.0)
    assert sel.channel_scores(e, [0.5, 0.5], P=P)[0, 0] == 1.5


def test_shared_decay_time_varying_weight_can_reorder():
    """v2 notes, GDN detail: with one decay for every channel of a head, a
    constant weight ranks by error alone, while a weight that varies in time
    can reorder channels whose errors occur at different times."""
    e = np.zeros((2, 1, DK))
    e[0, 0, 0] = 1.0   # channel 0: error at sample 0
    e[1, 0, 1] = 2.0   # channel 1: larger error, at sample 1
    w = [0.5, 0.5]
    const = np.full((2, 1, DK), 7.0)
    C = sel.channel_scores(e, w, W=const)
    assert C[0, 1] > C[0, 0]
    varying = np.ones((2, 1, DK))
    varying[0] = 10.0
    C = sel.channel_scores(e, w, W=varying)
    assert C[0, 0] > C[0, 1]


def test_select_stable_partition_with_ties():
    r = np.random.default_rng(3)
    score = r.integers(0, 40, (4, DK)).astype(np.float64)   # many ties
    prot, perm = sel.select_protected(score, 16)
    for h in range(4):
        chosen = set(prot[h].tolist())
        assert len(chosen) == 16
        assert sorted(perm[h].tolist()) == list(range(DK))
        assert perm[h, :16].tolist() == sorted(chosen)
        assert perm[h, 16:].tolist() == sorted(set(range(DK)) - chosen)
        lo = min(score[h, u] for u in chosen)
        for u in set(range(DK)) - chosen:
            assert score[h, u] <= lo
            if score[h, u] == lo:   # a tie at the boundary goes to the lower index
                assert all(v < u for v in chosen if score[h, v] == lo)


def test_selects_outlier_rows():
    """States whose rows 7 and 90 are scaled by 20: those two rows carry the
    largest quantization error and are chosen first."""
    r = np.random.default_rng(1)
    S = (0.1 * r.normal(0, 1, (4, 1, DK, DV))).astype(np.float32)
    S[:, :, [7, 90], :] *= 20
    e = sel.channel_error(S)
    C = sel.channel_scores(e, sel.domain_weights([0, 0, 1, 1]),
                           P=np.ones((1, DK)))
    prot, _ = sel.select_protected(C, 16)
    order = np.argsort(-C[0], kind="stable")
    assert set(order[:2].tolist()) == {7, 90}
    assert {7, 90} <= set(prot[0].tolist())
