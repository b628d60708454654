"""Key-channel selection on the GPU (qrs_channel_error, qrs_persistence_window,
qrs_persistence_geometric, qrs_channel_scores) and on the host
(qrs_select_protected_channels) against the oracle (oracle/selector.py).

* Per-channel INT8 error energy: the codes are decided in FP32 exactly as the
  oracle decides them, so the FP64 errors agree up to summation order
  (relative 1e-13); edge rows (zeros, exact ties, an underflowing scale).
* Window weight and scores: the same FP64 operations in the same order, so
  bit-identical; the geometric persistence within 1e-14 (device log / exp).
* End to end on FP32 reference trajectories of synthetic GDN and KDA states
  (the oracle's uncompressed recurrence), states sampled every eight steps
  from two domains: the GPU and oracle pipelines choose the same channels.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import selector as sel
from quantized_recurrent_state_02_amd import binding, inputs
from tests.parity_util import to_dev

pytestmark = pytest.mark.gpu
DK = DV = 128


def _states(seed, n, H):
    r = np.random.default_rng(seed)
    S = r.normal(0, 0.1, (n, H, DK, DV))
    S[:, :, 3, :] *= 20
    S[:, :, :, 9] *= 20
    S = S.astype(np.float32)
    S[0, 0, 1] = 0
    S[0, 0, 2, :32] = np.arange(-16, 16) + 0.5          # half-integers: exact ties
    S[0, 0, 2, 31] = 127
    S[0, 1, 4] = 0
    S[0, 1, 4, 7] = np.float32(2.0 ** -149) * 50         # amax / 127 underflows to 0
    return S


def test_channel_error_matches_oracle():
    n, H = 6, 4
    S = _states(21, n, H)
    c = np.exp(np.random.default_rng(2).uniform(np.log(0.5), np.log(2), (H, DV))).astype(np.float32)
    for smooth in (None, c):
        eg = binding.channel_error(to_dev(S), None if smooth is None else to_dev(smooth)).cpu().numpy()
        eo = sel.channel_error(S, smooth)
        assert eg[0, 0, 1] == 0 and eo[0, 0, 1] == 0
        rel = np.abs(eg - eo) / np.maximum(np.abs(eo), 1e-300)
        assert rel.max() <= 1e-13, rel.max()


def _traj_decays(seed, n_seq, T, H):
    r = np.random.default_rng(seed)
    a = r.uniform(0.0, 1.0, (n_seq, T, H, DK)).astype(np.float32)
    a[:, :, 0, :3] = 1.0      # never decays: the tau cap
    a[1, 5, 1, 4] = 0.0       # a zero decay inside a window
    a[1, 4, 1, 4] = 0.0       # and at a sampled write (log 0)
    return a


def test_persistence_and_scores_match_oracle():
    n_seq, T, H, horizon = 3, 40, 4, 16
    a = _traj_decays(8, n_seq, T, H)
    seqs = np.array([0, 0, 1, 2, 2, 1], np.int32)
    ts = np.array([3, 39, 0, 10, 30, 4], np.int32)     # t = 39: no later step
    w = sel.domain_weights([0, 0, 0, 1, 1, 1])
    da, ds, dt = to_dev(a), to_dev(seqs, torch.int32), to_dev(ts, torch.int32)
    dw = to_dev(w, torch.float64)
    Wg = binding.persistence_window(da, ds, dt, horizon).cpu().numpy()
    Wo = sel.persistence_window(a, seqs, ts, horizon)
    assert np.array_equal(Wg, Wo)
    assert np.all(Wg[1] == 1.0)
    Pg = binding.persistence_geometric(da, ds, dt, dw, 1e-4).cpu().numpy()
    Po = sel.persistence_geometric(a, seqs, ts, w, 1e-4)
    assert np.allclose(Pg, Po, rtol=1e-14, atol=0)
    assert np.all(Pg[0, :3] == 1e4) and Pg[1, 4] == 1.0
    e = np.abs(np.random.default_rng(4).normal(0, 1, (6, H, DK)))
    de = to_dev(e, torch.float64)
    Cw = binding.channel_scores(de, dw, W=to_dev(Wo, torch.float64)).cpu().numpy()
    assert np.array_equal(Cw, sel.channel_scores(e, w, W=Wo))
    Cp = binding.channel_scores(de, dw, P=to_dev(Po, torch.float64)).cpu().numpy()
    assert np.array_equal(Cp, sel.channel_scores(e, w, P=Po))


def test_persistence_and_scores_many_samples():
    """300 samples: the window kernel's blocks of 16 samples (runs of one
    sequence inside a block, and runs cut by block edges), and the summation
    kernels' passes of 128 samples through both LDS buffers and a partial last
    pass; zero weights skip their samples.  Window and scores bit for bit, the
    geometric persistence to the oracle's rounding of the logarithms."""
    n_seq, T, H, horizon, n = 4, 64, 3, 20, 300
    rng = np.random.default_rng(11)
    a = _traj_decays(9, n_seq, T, H)
    seqs = np.sort(rng.integers(0, n_seq, n)).astype(np.int32)
    seqs[::7] = rng.integers(0, n_seq, len(seqs[::7]))    # some runs broken up
    ts = rng.integers(0, T, n).astype(np.int32)
    w = sel.domain_weights(rng.integers(0, 3, n))
    w[rng.choice(n, 25, replace=False)] = 0.0
    da, ds, dt = to_dev(a), to_dev(seqs, torch.int32), to_dev(ts, torch.int32)
    dw = to_dev(w, torch.float64)
    Wg = binding.persistence_window(da, ds, dt, horizon).cpu().numpy()
    Wo = sel.persistence_window(a, seqs, ts, horizon)
    assert np.array_equal(Wg, Wo)
    Pg = binding.persistence_geometric(da, ds, dt, dw, 1e-4).cpu().numpy()
    Po = sel.persistence_geometric(a, seqs, ts, w, 1e-4)
    assert np.allclose(Pg, Po, rtol=1e-14, atol=0)
    e = np.abs(rng.normal(0, 1, (n, H, DK)))
    de = to_dev(e, torch.float64)
    Cw = binding.channel_scores(de, dw, W=to_dev(Wo, torch.float64)).cpu().numpy()
    assert np.array_equal(Cw, sel.channel_scores(e, w, W=Wo))
    Cp = binding.channel_scores(de, dw, P=to_dev(Po, torch.float64)).cpu().numpy()
    assert np.array_equal(Cp, sel.channel_scores(e, w, P=Po))


def test_invalid_sample_gives_nan():
    a = _traj_decays(1, 2, 8, 2)
    W = binding.persistence_window(to_dev(a), to_dev(np.array([0, 2], np.int32), torch.int32),
                                   to_dev(np.array([2, 0], np.int32), torch.int32), 4).cpu().numpy()
    assert np.all(np.isfinite(W[0])) and np.all(np.isnan(W[1]))
    P = binding.persistence_geometric(to_dev(a), to_dev(np.array([0], np.int32), torch.int32),
                                      to_dev(np.array([9], np.int32), torch.int32),
                                      to_dev(np.ones(1), torch.float64)).cpu().numpy()
    assert np.all(np.isnan(P))


def _reference_trajectories(cfg, kind, n_seq, H, T):
    """FP32 trajectories of the uncompressed recurrence (the oracle, model
    coordinates) and the per-step decay of every key channel."""
    pool = oracle.OracleDensePool(n_seq, H)
    slots = np.arange(n_seq, dtype=np.int32)
    pool.set_model(slots, inputs.initial_state(cfg, n_seq, H))
    states = np.empty((n_seq, T, H, DK, DV), np.float32)
    a = np.empty((n_seq, T, H, DK), np.float32)
    for t in range(T):
        d = inputs.step_inputs(cfg, t, n_seq, H, kind)
        if kind == "gdn":
            pool.decode_step(slots, d["q"], d["k"], d["v"], d["alpha"], d["beta"], 0)
            a[:, t] = np.repeat(d["alpha"][:, :, None], DK, axis=2)
        else:
            pool.decode_step(slots, d["q"], d["k"], d["v"], d["g"], d["beta"], 1)
            a[:, t] = np.exp(d["g"])
        states[:, t] = pool.get_model(slots)
    return states, a


@pytest.mark.parametrize("kind,cfg", [("gdn", 1), ("kda", 2)])
def test_selection_pipeline_on_reference_trajectories(kind, cfg):
    n_seq, H, T = 4, 4, 48
    states, a = _reference_trajectories(cfg, kind, n_seq, H, T)
    c = inputs.smoothing(cfg, H, True)
    seqs = np.repeat(np.arange(n_seq), T // 8).astype(np.int32)
    ts = np.tile(np.arange(7, T, 8), n_seq).astype(np.int32)
    S = np.ascontiguousarray(states[seqs, ts])
    w = sel.domain_weights(seqs // 2)                      # two domains of two sequences
    # oracle pipeline
    eo = sel.channel_error(S, c)
    Wo = sel.persistence_window(a, seqs, ts, 256)
    Po = sel.persistence_geometric(a, seqs, ts, w, 1e-4)
    # GPU pipeline
    dw = to_dev(w, torch.float64)
    eg = binding.channel_error(to_dev(S), to_dev(c))
    ds, dt = to_dev(seqs, torch.int32), to_dev(ts, torch.int32)
    Wg = binding.persistence_window(to_dev(a), ds, dt, 256)
    Pg = binding.persistence_geometric(to_dev(a), ds, dt, dw, 1e-4)
    assert np.array_equal(Wg.cpu().numpy(), Wo)
    for Cg, Co in ((binding.channel_scores(eg, dw, W=Wg), sel.channel_scores(eo, w, W=Wo)),
                   (binding.channel_scores(eg, dw, P=Pg), sel.channel_scores(eo, w, P=Po))):
        Cg = Cg.cpu().numpy()
        assert np.allclose(Cg, Co, rtol=1e-12, atol=0)
        perm_g = binding.select_protected_channels(Cg)
        _, perm_o = sel.select_protected(Co, 16)
        # the 16th and 17th scores are far apart compared with the tolerance,
        # so both sides must pick the same channels
        srt = -np.sort(-Co, axis=1)
        assert np.all((srt[:, 15] - srt[:, 16]) > 1e-9 * srt[:, 15])
        assert np.array_equal(perm_g, perm_o)
