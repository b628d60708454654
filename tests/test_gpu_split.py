"""The value-column-half decode kernel (two workgroups per unit) against the
whole-unit kernel: both perform the same operations in the same order, so on
identical stored bytes and operands they must give the same outputs and the
same stored bytes, bit for bit, at every step.  Both are also checked against
the oracle in test_gpu_decode.py (exact trajectories and derived bounds).  The
default mode's mix of the two in one launch (whole units, then a tail of
half-unit workgroups, on large grids) is checked against each."""
import numpy as np
import pytest
import torch

from quantized_recurrent_state_02_amd import binding, inputs
from tests.parity_util import to_dev

pytestmark = pytest.mark.gpu
DK = DV = 128


def _run(mode, kind, io_bf16, S0, slots, heads, steps_in, num_slots, H, perm, c):
    prev = binding.set_decode_split(mode)
    try:
        gp = binding.StatePool(binding.FMT_I8F16, num_slots, H, perm, c)
        gp.units().zero_()
        ok_slots = slots[(slots >= 0) & (slots < num_slots)]
        gp.store(to_dev(ok_slots, torch.int32), to_dev(S0[:len(ok_slots)]))
        ds = to_dev(slots, torch.int32)
        outs, states = [], []
        gate = "alpha" if kind == "gdn" else "g"
        for d in steps_in:
            if io_bf16 or heads is not None:
                dt = torch.bfloat16 if io_bf16 else torch.float32
                o = gp.step_ex(kind, ds, to_dev(d["q"]).to(dt), to_dev(d["k"]).to(dt),
                               to_dev(d["v"]).to(dt), to_dev(d[gate]), to_dev(d["beta"]), heads=heads)
            else:
                fn = gp.gdn_step if kind == "gdn" else gp.kda_step
                o = fn(ds, to_dev(d["q"]), to_dev(d["k"]), to_dev(d["v"]), to_dev(d[gate]),
                       to_dev(d["beta"]))
            outs.append(o.float().cpu().numpy())
            states.append(gp.units().cpu().numpy().copy())
        return outs, states
    finally:
        binding.set_decode_split(prev)


@pytest.mark.parametrize("kind,cfg", [("gdn", 1), ("kda", 2)])
@pytest.mark.parametrize("io_bf16,heads", [(False, None), (True, None), (False, (1, 3))])
def test_halves_equal_whole_unit(kind, cfg, io_bf16, heads):
    H, num_slots, n, steps = 5, 11, 7, 6
    perm = inputs.protected_perm(cfg, H)
    c = inputs.smoothing(cfg, H, True)
    slots = np.array([10, 0, 4, 13, 7, 2, 9], np.int32)      # 13 is out of range
    S0 = inputs.initial_state(cfg, n, H)
    steps_in = [inputs.step_inputs(cfg, t, n, H, kind) for t in range(steps)]
    ow, sw = _run(binding.DECODE_SPLIT_WHOLE, kind, io_bf16, S0, slots, heads, steps_in, num_slots,
                  H, perm, c)
    oh, sh = _run(binding.DECODE_SPLIT_HALVES, kind, io_bf16, S0, slots, heads, steps_in,
                  num_slots, H, perm, c)
    for t in range(steps):
        assert np.array_equal(ow[t].view(np.uint32), oh[t].view(np.uint32)), f"step {t}: outputs differ"
        assert np.array_equal(sw[t], sh[t]), f"step {t}: stored bytes differ"
    bad = slots == 13
    assert np.all(np.isnan(oh[-1][bad]))


@pytest.mark.parametrize("kind,cfg", [("gdn", 1), ("kda", 2)])
def test_halves_equal_whole_unit_full_heads(kind, cfg):
    """64 slots x 32 heads (2,048 units, two per workgroup group of 16 with no
    tail) and 45 slots (1,440 units, a partial last group), 3 steps."""
    H = 32
    perm = inputs.protected_perm(cfg, H)
    c = inputs.smoothing(cfg, H, True)
    for n in (64, 45):
        slots = np.arange(n, dtype=np.int32)[::-1].copy()
        S0 = inputs.initial_state(cfg, n, H)
        steps_in = [inputs.step_inputs(cfg, t, n, H, kind) for t in range(3)]
        ow, sw = _run(binding.DECODE_SPLIT_WHOLE, kind, False, S0, slots, None, steps_in, n, H,
                      perm, c)
        oh, sh = _run(binding.DECODE_SPLIT_HALVES, kind, False, S0, slots, None, steps_in, n, H,
                      perm, c)
        for t in range(3):
            assert np.array_equal(ow[t].view(np.uint32), oh[t].view(np.uint32)), f"n={n} step {t}"
            assert np.array_equal(sw[t], sh[t]), f"n={n} step {t}: stored bytes differ"


@pytest.mark.parametrize("kind,cfg", [("gdn", 1), ("kda", 2)])
@pytest.mark.parametrize("io_bf16", [False, True])
@pytest.mark.parametrize("n", [100, 65])
def test_half_unit_tail_equals_whole_unit(kind, cfg, io_bf16, n):
    """Grids of at least 4/3 of a generation of resident workgroups (100 or
    65 slots x 32 heads = 3,200 or 2,080 units, against 1,536 resident on
    MI355X) in the default mode end with half-unit workgroups; outputs and
    stored bytes equal those of whole units only and of halves only, bit for
    bit, including unknown slot ids inside and outside the tail."""
    H, steps = 32, 3
    num_slots = n + 3
    perm = inputs.protected_perm(cfg, H)
    c = inputs.smoothing(cfg, H, True)
    slots = np.random.default_rng(41).permutation(num_slots)[:n].astype(np.int32)
    slots[3] = -1
    slots[n - 3] = num_slots + 5
    S0 = inputs.initial_state(cfg, n, H)
    steps_in = [inputs.step_inputs(cfg, t, n, H, kind) for t in range(steps)]
    runs = {m: _run(m, kind, io_bf16, S0, slots, None, steps_in, num_slots, H, perm, c)
            for m in (binding.DECODE_SPLIT_AUTO, binding.DECODE_SPLIT_WHOLE,
                      binding.DECODE_SPLIT_HALVES)}
    oa, sa = runs[binding.DECODE_SPLIT_AUTO]
    for m in (binding.DECODE_SPLIT_WHOLE, binding.DECODE_SPLIT_HALVES):
        om, sm = runs[m]
        for t in range(steps):
            assert np.array_equal(oa[t].view(np.uint32), om[t].view(np.uint32)), f"mode {m} step {t}"
            assert np.array_equal(sa[t], sm[t]), f"mode {m} step {t}: stored bytes differ"
    bad = (slots < 0) | (slots >= num_slots)
    assert np.all(np.isnan(oa[-1][bad])) and np.all(np.isfinite(oa[-1][~bad]))
