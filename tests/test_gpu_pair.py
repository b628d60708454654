"""qrs_decode_step_pair (a GDN step and a KDA step on disjoint slots of one
pool in one call) against the two separate calls, qrs_gdn_decode_step then
qrs_kda_decode_step, which the decode tests check against the oracle: outputs
and stored bytes equal bit for bit at every step.  Cases: a grid large enough
for the one-launch kernel with its half-unit tail (and without the tail, whole
units only), a small grid (the two calls), an empty group, unknown slot ids in
both groups, head counts that are not powers of two (the kernel's XCD-aware
order deals slots in runs of H heads), and the paged workload at full size in
random and ascending slot order."""
import numpy as np
import pytest
import torch

from quantized_recurrent_state_02_amd import binding, inputs
from tests.parity_util import to_dev

pytestmark = pytest.mark.gpu
DK = DV = 128


def _setup(H, n_g, n_k, num_slots, seed, fmt=binding.FMT_I8F16):
    perm = None if fmt == binding.FMT_FP32 else inputs.protected_perm(1, H)
    c = None if fmt == binding.FMT_FP32 else inputs.smoothing(1, H, True)
    ids = np.random.default_rng(seed).permutation(num_slots).astype(np.int32)
    sg, sk = ids[:n_g].copy(), ids[n_g:n_g + n_k].copy()
    S = inputs.initial_state(1, n_g + n_k, H)
    pools = []
    for _ in range(2):
        gp = binding.StatePool(fmt, num_slots, H, perm, c)
        gp.units().zero_()
        gp.store(to_dev(ids[:n_g + n_k], torch.int32), to_dev(S))
        pools.append(gp)
    return pools, sg, sk


def _steps(H, n_g, n_k, steps, seed):
    out = []
    for t in range(steps):
        dg = inputs.step_inputs(1, seed + t, max(n_g, 1), H, "gdn")
        dk = inputs.step_inputs(2, seed + t, max(n_k, 1), H, "kda")
        dk["g"][0, 0, :7] = -np.inf                       # zero decays on some channels
        out.append(({key: val[:n_g] for key, val in dg.items()},
                    {key: val[:n_k] for key, val in dk.items()}))
    return out


def _run_both(H, n_g, n_k, num_slots, steps, seed, bad_g=None, bad_k=None, fmt=binding.FMT_I8F16):
    (pa, pb), sg, sk = _setup(H, n_g, n_k, num_slots, seed, fmt)
    if bad_g is not None and n_g:
        sg[bad_g] = -1
    if bad_k is not None and n_k:
        sk[bad_k] = num_slots + 7
    dsg, dsk = to_dev(sg, torch.int32), to_dev(sk, torch.int32)
    for t, (dg, dk) in enumerate(_steps(H, n_g, n_k, steps, seed)):
        g_args = (dsg, to_dev(dg["q"]), to_dev(dg["k"]), to_dev(dg["v"]), to_dev(dg["alpha"]),
                  to_dev(dg["beta"]))
        k_args = (dsk, to_dev(dk["q"]), to_dev(dk["k"]), to_dev(dk["v"]), to_dev(dk["g"]),
                  to_dev(dk["beta"]))
        og_a, ok_a = pa.pair_step(g_args, k_args)
        og_b = pb.gdn_step(*g_args) if n_g else torch.empty((0, H, DV), device="cuda")
        ok_b = pb.kda_step(*k_args) if n_k else torch.empty((0, H, DV), device="cuda")
        for a, b, nm in ((og_a, og_b, "gdn"), (ok_a, ok_b, "kda")):
            a, b = a.cpu().numpy(), b.cpu().numpy()
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"step {t}: {nm} outputs differ"
        assert torch.equal(pa.units(), pb.units()), f"step {t}: stored bytes differ"
    return og_a.cpu().numpy(), ok_a.cpu().numpy(), sg, sk


@pytest.mark.parametrize("mode", [binding.DECODE_SPLIT_AUTO, binding.DECODE_SPLIT_WHOLE])
def test_pair_one_launch_equals_two_calls(mode):
    """60 GDN + 60 KDA requests x 32 heads = 3,840 units: the one-launch
    kernel, with the half-unit tail on the KDA units in the default mode."""
    prev = binding.set_decode_split(mode)
    try:
        og, ok, sg, sk = _run_both(32, 60, 60, 131, 3, 5, bad_g=17, bad_k=59)
    finally:
        binding.set_decode_split(prev)
    assert np.all(np.isnan(og[17])) and np.all(np.isfinite(np.delete(og, 17, axis=0)))
    assert np.all(np.isnan(ok[59])) and np.all(np.isfinite(ok[:59]))


@pytest.mark.parametrize("n_g,n_k", [(3, 2), (0, 5), (4, 0)])
def test_pair_small_and_empty_groups(n_g, n_k):
    _run_both(4, n_g, n_k, 11, 2, 9)


@pytest.mark.parametrize("fmt", [binding.FMT_U8H16, binding.FMT_FP32])
def test_pair_other_pool_formats(fmt):
    """On the other pool formats the pair call makes the two calls."""
    _run_both(4, 3, 2, 9, 2, 13, bad_g=1, fmt=fmt)


@pytest.mark.parametrize("H,n_g,n_k", [(5, 110, 109), (12, 150, 150), (32, 16, 16), (32, 30, 34)])
def test_pair_xcd_order_other_head_counts(H, n_g, n_k):
    """The one-launch kernel deals each group's slots whole to the XCDs, in
    runs of H heads: head counts that are not powers of two, a GDN group
    whose unit count is not a multiple of 8 (so the KDA units start off an
    XCD boundary), slots past the last full round of 8, the half-unit tail
    at 3,600 and 2,048 units (the smallest grid that takes it), and exactly
    1,024 units (the smallest grid that takes the one-launch kernel),
    against the two calls bit for bit."""
    _run_both(H, n_g, n_k, n_g + n_k + 3, 2, 21, bad_g=n_g - 1, bad_k=0)


@pytest.mark.parametrize("order", ["random", "ascending"])
def test_pair_full_paged_shape(order):
    """The paged workload at full size, in the launch that the benchmark's
    one-launch legs time: 4,096 slots x 32 heads, 512 GDN and 512 KDA
    requests on distinct random slots (16,384 units per group, the KDA group
    ending in the half-unit tail), in random slot order and in ascending
    order.  One qrs_decode_step_pair call per step against the two calls on
    a copy of the pool, outputs and every byte of the pool equal over three
    steps."""
    cfg, H, num_slots = 4, 32, 4096
    perm = inputs.protected_perm(cfg, H)
    c = inputs.smoothing(cfg, H, True)
    gs, ks = inputs.paged_slots(cfg, num_slots, 1024)    # in random order
    if order == "ascending":
        gs, ks = np.sort(gs), np.sort(ks)
    pa = binding.StatePool(binding.FMT_I8F16, num_slots, H, perm, c)
    pa.units().zero_()
    active = np.concatenate([gs, ks]).astype(np.int32)
    for i in range(0, len(active), 64):
        S = inputs.initial_state_device(cfg, min(64, len(active) - i), H, perm, first=i)
        pa.store(to_dev(active[i:i + 64], torch.int32), S)
    pb = binding.StatePool(binding.FMT_I8F16, num_slots, H, perm, c)
    pb.units().copy_(pa.units())
    dgs, dks = to_dev(gs, torch.int32), to_dev(ks, torch.int32)
    for t in range(3):
        dg = inputs.step_inputs_device(cfg, t, len(gs), H, "gdn")
        dk = inputs.step_inputs_device(cfg, t, len(ks), H, "kda")
        g_args = (dgs, dg["q"], dg["k"], dg["v"], dg["alpha"], dg["beta"])
        k_args = (dks, dk["q"], dk["k"], dk["v"], dk["g"], dk["beta"])
        og_a, ok_a = pa.pair_step(g_args, k_args)
        og_b = pb.gdn_step(*g_args)
        ok_b = pb.kda_step(*k_args)
        assert torch.equal(og_a.view(torch.int32), og_b.view(torch.int32)), f"step {t}: gdn outputs"
        assert torch.equal(ok_a.view(torch.int32), ok_b.view(torch.int32)), f"step {t}: kda outputs"
        assert bool(torch.isfinite(og_a).all()) and bool(torch.isfinite(ok_a).all())
        assert torch.equal(pa.units(), pb.units()), f"step {t}: stored bytes differ"
