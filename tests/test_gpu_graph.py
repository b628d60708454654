"""Decode steps captured in a HIP graph (the launch form bench.py times)
against the same steps launched eagerly, at the serving shape.

One pool holds two copies of the same 256 x 32 initial states (slot sets A
and B).  The steps on B are captured once; every round runs the steps
eagerly on A, then replays the graph on B, and the outputs of every step and
the packed bytes of every unit must be equal bit for bit (same kernels, same
inputs, deterministic arithmetic).  The graph is replayed three times with
the eager work and synchronizations in between.  The serving shape also
takes the decode kernel's staggered-start path (more than two generations of
resident workgroups).
"""
import numpy as np
import pytest
import torch

from quantized_recurrent_state_02_amd import binding, inputs
from tests.parity_util import to_dev

pytestmark = pytest.mark.gpu

N, H, ROUNDS = 256, 32, 3


def _twin_pool(cfg, n, H):
    perm = inputs.protected_perm(cfg, H)
    c = inputs.smoothing(cfg, H, True)
    pool = binding.StatePool(binding.FMT_I8F16, 2 * n, H, perm, c)
    S0 = to_dev(inputs.initial_state(cfg, n, H))
    a = torch.arange(n, dtype=torch.int32, device="cuda")
    b = a + n
    pool.store(a, S0)
    pool.store(b, S0)
    del S0
    return pool, a, b


def _assert_twins_equal(pool, a, b, outs_a, outs_b, what):
    u = pool.units().view(2 * N, H, -1)
    assert torch.equal(u[a.long()], u[b.long()]), f"{what}: packed states differ"
    for t, (x, y) in enumerate(zip(outs_a, outs_b)):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32)), f"{what}: output {t} differs"


@pytest.mark.parametrize("kind,cfg", [("gdn", 1), ("kda", 2)])
def test_graph_replay_equals_eager(kind, cfg):
    steps = 6
    pool, a, b = _twin_pool(cfg, N, H)
    gate = "alpha" if kind == "gdn" else "g"
    d = [{key: to_dev(val) for key, val in inputs.step_inputs(cfg, t, N, H, kind).items()}
         for t in range(steps)]
    fn = pool.gdn_step if kind == "gdn" else pool.kda_step
    outs_a = [torch.empty((N, H, 128), device="cuda") for _ in range(steps)]
    outs_b = [torch.empty((N, H, 128), device="cuda") for _ in range(steps)]

    def run(slots, outs):
        for t in range(steps):
            fn(slots, d[t]["q"], d[t]["k"], d[t]["v"], d[t][gate], d[t]["beta"], outs[t])

    # warm-up on both sets (first launches outside the capture), then capture B
    run(a, outs_a)
    run(b, outs_b)
    torch.cuda.synchronize()
    _assert_twins_equal(pool, a, b, outs_a, outs_b, "eager warm-up")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(b, outs_b)
    torch.cuda.synchronize()
    # capturing launches nothing: advance A once to match B's state again
    u = pool.units().view(2 * N, H, -1)
    assert torch.equal(u[a.long()], u[b.long()]), "capture changed the pool"
    for r in range(ROUNDS):
        run(a, outs_a)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _assert_twins_equal(pool, a, b, outs_a, outs_b, f"replay {r}")
    del g
    pool.close()


def test_window_graph_replay_equals_eager():
    cfg, window = 1, 16
    pool, a, b = _twin_pool(cfg, N, H)
    buf = pool.window_buffer("gdn", window)
    d = [{key: to_dev(val) for key, val in inputs.step_inputs(cfg, t, N, H, "gdn").items()}
         for t in range(window)]
    pos = [torch.full((N,), j, dtype=torch.int32, device="cuda") for j in range(window)]
    outs_a = [torch.empty((N, H, 128), device="cuda") for _ in range(window)]
    outs_b = [torch.empty((N, H, 128), device="cuda") for _ in range(window)]

    def run(slots, outs):
        for t in range(window):
            pool.window_step("gdn", window, buf, slots, pos[t], d[t]["q"], d[t]["k"], d[t]["v"],
                             d[t]["alpha"], d[t]["beta"], out=outs[t])

    run(a, outs_a)
    run(b, outs_b)
    torch.cuda.synchronize()
    _assert_twins_equal(pool, a, b, outs_a, outs_b, "eager warm-up")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(b, outs_b)
    torch.cuda.synchronize()
    for r in range(ROUNDS):
        run(a, outs_a)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _assert_twins_equal(pool, a, b, outs_a, outs_b, f"window replay {r}")
    del g
    pool.close()
