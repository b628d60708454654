#!/usr/bin/env python3
"""Benchmark: compressed-state GDN / KDA decode on one MI355X.

Metric: state updates per second and achieved HBM bandwidth (algorithmic
bytes) against the MI355X peak, for GDN and KDA decode at batch 256,
32 heads, d_k = d_v = 128.  A step is one decode step of all 256 x 32
(slot, head) units through the fused kernel: packed-state load, dequantize,
FP32 delta-rule update and readout, requantize, store.

Algorithmic bytes per update (one unit advanced by one token):
  state read 20,224 + state write 20,224 + q, k, v 3 x 512
  + GDN alpha, beta 8  (= 41,992)   /  KDA g 512 + beta 4  (= 42,500).
The FP32-state kernel on the same inputs moves 65,536 x 2 + 1,544 = 132,616.

Inputs are the seeded synthetic workload (quantized_recurrent_state_02_amd/
inputs.py), staged in device memory before the timed region.  The step loop
is captured once in a HIP graph.  After a few seconds of device warm-up and
one untimed replay left in the queue, `--reps` replays are timed back to
back, each bracketed by HIP events on the launch stream; the median per-step
time is reported, with the minimum and maximum beside it.  By default 4
disjoint slot sets of 256 requests are rotated step by step so the packed
states (4 x 165.7 MB) exceed the 256 MB Infinity Cache and every state read
comes from HBM; the single-set figure is reported beside it.

The CPU baseline is the oracle (oracle/, FP32 C code with OpenMP over units)
on the full GDN decode workload (256 x 32 units, 256 steps); `detail` also
carries the oracle on the full KDA decode and prefill workloads and on 1,024
units of the paged workload, with the thread count, the physical cores and
the CPU model.

`detail` also reports KDA decode, the single-set variants, the FP32-state
kernel on the same inputs, a batch sweep (16 to 512 requests) of the
compressed kernels against the FP32-state kernel, paged decode over a mixed
GDN/KDA pool (4,096 slots, 1,024 active), the chunked prefill kernel (8 x 32
heads x 4096 tokens, chunks of 64, FP32 and bf16 q/k/v) against the FP32
matrix-core peak, the key-channel selection kernels on a calibration-shaped
sample, per-window decode, and the first revision's low tier (block-32
Hadamard + UINT8 with FP16 scale and zero point) on the decode workload,
with its trajectory error next to the INT8 tier's.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
BYTES_GDN = 20224 * 2 + 3 * 512 + 8
BYTES_KDA = 20224 * 2 + 3 * 512 + 512 + 4
BYTES_F32_GDN = 65536 * 2 + 3 * 512 + 8
BYTES_GDN_BF16IO = 20224 * 2 + 3 * 256 + 8
COUNTERS_FILE = os.path.join(ROOT, "profiles", "decode_gdn_b256_h32_counters.json")
TRACE_FILE = os.path.join(ROOT, "profiles", "decode_gdn_b256_h32_kernel_trace.json")
KERNEL_SOURCES = ["quantized_recurrent_state_02_amd/csrc/qrs_decode.hip",
                  "quantized_recurrent_state_02_amd/csrc/qrs_decode_half.h",
                  "quantized_recurrent_state_02_amd/csrc/qrs_hadamard.h",
                  "quantized_recurrent_state_02_amd/csrc/qrs_internal.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_digest():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stage_inputs(torch, inputs, cfg, kind, n, H, steps):
    """All per-step operands of `steps` steps, stacked on the device."""
    t0 = time.time()
    keys = ["q", "k", "v", "beta", "alpha" if kind == "gdn" else "g"]
    host = {key: [] for key in keys}
    for t in range(steps):
        d = inputs.step_inputs(cfg, t, n, H, kind)
        for key in keys:
            host[key].append(d[key])
    dev = {key: torch.from_numpy(np.stack(v)).to("cuda") for key, v in host.items()}
    log(f"[bench] staged {steps} steps of {kind} inputs in {time.time() - t0:.1f}s")
    return dev


def time_loop(torch, launch, steps, warmup, use_graph, reps=5, warm_s=0.0, side=None):
    """Run `launch(t)` for t < warmup (eager), then time `reps` passes over the
    steps t in [warmup, warmup + steps), back to back.

    With use_graph the pass is captured once in a HIP graph and replayed.
    Before the timed passes the device is kept busy for `warm_s` seconds of
    wall time (clocks and caches settle), and one more untimed pass is
    enqueued without a synchronization: each timed pass is bracketed by HIP
    events on the launch stream that are recorded behind work already in the
    queue, so neither the host's graph submission nor an idle GPU falls
    inside a timed window.
    `side`: a second stream that `launch` also issues work on; it is forked
    from the launch stream before a pass's first step and joined after its
    last (one fork and one join per pass, none per step).
    Returns (seconds of each timed pass, seconds of device warm-up)."""
    stream = torch.cuda.current_stream()

    def steps_of(ts):
        if side is not None:
            side.wait_stream(torch.cuda.current_stream())
        for t in ts:
            launch(t)
        if side is not None:
            torch.cuda.current_stream().wait_stream(side)

    steps_of(range(warmup))
    torch.cuda.synchronize()
    if use_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            steps_of(range(warmup, warmup + steps))
        torch.cuda.synchronize()
        g.replay()                       # graph upload
        torch.cuda.synchronize()
        run = g.replay
    else:
        def run():
            steps_of(range(warmup, warmup + steps))
    warm = 0.0
    if warm_s > 0:
        t0 = time.perf_counter()
        i = 0
        while time.perf_counter() - t0 < warm_s:
            run()
            i += 1
            if i % 4 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        warm = time.perf_counter() - t0
    run()                                # untimed, still running when the first window opens
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
    for start, end in events:
        start.record(stream)
        run()
        end.record(stream)
    torch.cuda.synchronize()
    return [start.elapsed_time(end) / 1e3 for start, end in events], warm


def pass_stats(passes, steps):
    """Per-step time of timed passes: the median is the reported figure."""
    per = sorted(p / steps for p in passes)
    m = len(per)
    med = per[m // 2] if m % 2 else 0.5 * (per[m // 2 - 1] + per[m // 2])
    return {"per_step": med, "per_step_min": per[0], "per_step_max": per[-1], "passes": m}


def run_decode(torch, binding, inputs, kind, fmt, dev_in, perm, c, n, H, steps, warmup, pools,
               use_graph, io_bf16=False, reps=5, warm_s=0.0):
    """Decode at the serving shape over `pools` rotated slot sets; returns the
    pass_stats dict (seconds per step) with "ok" (finite outputs) and
    "device_warmup_s"."""
    total_slots = n * pools
    pool = binding.StatePool(fmt, total_slots, H, perm, c)
    cfg = 1 if kind == "gdn" else 2
    S0 = inputs.initial_state(cfg, n, H)
    S0d = torch.from_numpy(S0).to("cuda")
    slot_sets = []
    for p in range(pools):
        s = torch.arange(p * n, (p + 1) * n, dtype=torch.int32, device="cuda")
        pool.store(s, S0d)
        slot_sets.append(s)
    gate_key = "alpha" if kind == "gdn" else "g"
    if io_bf16:
        # q, k, v and the readout in bf16 through qrs_decode_step_ex
        ops = {x: dev_in[x].to(torch.bfloat16) for x in ("q", "k", "v")}
        out = torch.empty((n, H, 128), dtype=torch.bfloat16, device="cuda")

        def launch(t):
            pool.step_ex(kind, slot_sets[t % pools], ops["q"][t], ops["k"][t], ops["v"][t],
                         dev_in[gate_key][t], dev_in["beta"][t], out=out)
    else:
        out = torch.empty((n, H, 128), dtype=torch.float32, device="cuda")
        step_fn = pool.gdn_step if kind == "gdn" else pool.kda_step

        def launch(t):
            step_fn(slot_sets[t % pools], dev_in["q"][t], dev_in["k"][t], dev_in["v"][t],
                    dev_in[gate_key][t], dev_in["beta"][t], out)

    passes, warm = time_loop(torch, launch, steps, warmup, use_graph, reps=reps, warm_s=warm_s)
    st = pass_stats(passes, steps)
    st["ok"] = bool(torch.isfinite(out.float()).all().item())
    st["device_warmup_s"] = warm
    pool.close()
    del pool
    torch.cuda.empty_cache()
    return st


# Chunked prefill (FP32 matrix cores): algorithmic FLOP per (chunk, head) of
# the chunk form, C = 64 tokens, d = 128: the two masked Gram products and the
# triangular solve (5 C^2 d) plus W S0, Q S0 and K^T Delta (6 C d^2).
PREFILL_CHUNK = 64
PREFILL_FLOP_PER_CHUNK_HEAD = 5 * 64 * 64 * 128 + 6 * 64 * 128 * 128
PEAK_FP32_MFMA_TFLOPS = 157.3


def run_prefill(torch, binding, inputs, bf16, reps=5, fmt=None):
    """Prefill workload: 8 sequences x 32 heads x 4096 tokens in chunks of 64,
    GDN gating, fresh requests (zero initial state), compressed pool (the
    INT8 tier unless fmt names another).  Returns (seconds per call, stats
    dict)."""
    fmt = binding.FMT_I8F16 if fmt is None else fmt
    wl = inputs.WORKLOADS[3]
    n, H, T = wl.n, wl.heads, wl.steps
    t0 = time.time()
    d = inputs.prefill_inputs(3, n, H, T)
    dt = torch.bfloat16 if bf16 else torch.float32
    dev = {key: torch.from_numpy(d[key]).to("cuda").to(dt) for key in ("q", "k", "v")}
    for key in ("alpha", "beta"):
        dev[key] = torch.from_numpy(d[key]).to("cuda")
    del d
    log(f"[bench] staged prefill inputs ({'bf16' if bf16 else 'fp32'}) in {time.time() - t0:.1f}s")
    pool = binding.StatePool(fmt, n, H, inputs.protected_perm(3, H), inputs.smoothing(3, H, False))
    slots = torch.arange(n, dtype=torch.int32, device="cuda")
    out = torch.empty((n, T, H, 128), dtype=torch.float32, device="cuda")

    def call():
        pool.prefill(slots, dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"],
                     chunk=PREFILL_CHUNK, init_from_pool=False, out=out)

    passes, _ = time_loop(torch, lambda t: call(), 1, 1, False, reps=reps, warm_s=0.5)
    pst = pass_stats(passes, 1)
    secs = pst["per_step"]
    ok = bool(torch.isfinite(out).all().item())
    flop = n * H * (T // PREFILL_CHUNK) * PREFILL_FLOP_PER_CHUNK_HEAD
    in_bytes = 3 * n * T * H * 128 * (2 if bf16 else 4) + 2 * n * T * H * 4
    hbm = in_bytes + n * T * H * 128 * 4 + n * H * (T // PREFILL_CHUNK) * 20224
    pool.close()
    del pool, dev, out
    torch.cuda.empty_cache()
    return secs, {"ms_per_call": secs * 1e3, "ms_per_call_min": pst["per_step_min"] * 1e3,
                  "ms_per_call_max": pst["per_step_max"] * 1e3, "timed_calls": pst["passes"],
                  "tokens_per_s": n * T / secs,
                  "tflops_fp32_mfma": flop / secs / 1e12,
                  "frac_of_fp32_mfma_peak": flop / secs / 1e12 / PEAK_FP32_MFMA_TFLOPS,
                  "hbm_gbs_algorithmic": hbm / secs / 1e9, "flop_per_call": flop,
                  "finite_outputs": ok,
                  "workload": f"prefill {n} x {H} heads x {T} tokens, chunk {PREFILL_CHUNK}, "
                              f"{'bf16' if bf16 else 'fp32'} q/k/v, zero initial state, "
                              f"{'INT8+Hadamard (v1)' if fmt == binding.FMT_U8H16 else 'INT8'} tier"}


def run_codec_compare(torch, binding, inputs, dev_in, perm, c, n, H, steps):
    """GDN at the serving shape, the INT8 tier and the first revision's tier
    (block-32 Hadamard + UINT8, FP16 s and z) against the uncompressed FP32
    recurrence on identical inputs: RRMSE of every step's readout and of the
    final state (model coordinates)."""
    S0 = torch.from_numpy(inputs.initial_state(1, n, H)).to("cuda")
    slots = torch.arange(n, dtype=torch.int32, device="cuda")
    pools = {name: binding.StatePool(fmt, n, H, perm, c)
             for name, fmt in (("int8", binding.FMT_I8F16), ("u8_hadamard", binding.FMT_U8H16),
                               ("fp32", binding.FMT_FP32))}
    for p in pools.values():
        p.store(slots, S0)
    outs = {name: torch.empty((n, H, 128), device="cuda") for name in pools}
    num = {name: torch.zeros((), dtype=torch.float64, device="cuda") for name in ("int8", "u8_hadamard")}
    den = torch.zeros((), dtype=torch.float64, device="cuda")
    for t in range(steps):
        for name, p in pools.items():
            p.gdn_step(slots, dev_in["q"][t], dev_in["k"][t], dev_in["v"][t], dev_in["alpha"][t],
                       dev_in["beta"][t], outs[name])
        ref = outs["fp32"].double()
        for name in num:
            num[name] += ((outs[name].double() - ref) ** 2).sum()
        den += (ref ** 2).sum()
    Sref = pools["fp32"].dequant(slots).double()
    res = {"workload": f"GDN, {n} slots x {H} heads, {steps} steps from the same stored start"}
    for name in num:
        Sq = pools[name].dequant(slots).double()
        res[name] = {"readout_rrmse": float(torch.sqrt(num[name] / den)),
                     "final_state_rrmse": float(torch.sqrt(((Sq - Sref) ** 2).sum() / (Sref ** 2).sum()))}
    for p in pools.values():
        p.close()
    torch.cuda.empty_cache()
    return res


# Per-window quantization (LeapQuant section 3.2): algorithmic bytes per GDN
# update averaged over a 16-token window -- the state read every token, written
# once per window, the window's records (528 B: k, v FP16, beta, alpha) read
# (7.5 on average) and written (15 of 16 tokens), q, k, v and gates.
WINDOW = 16
BYTES_GDN_WINDOW = (20224 + 20224 / WINDOW + 528 * (WINDOW - 1) / 2 + 528 * (WINDOW - 1) / WINDOW
                    + 3 * 512 + 8)
# KDA: records of 784 B (k, v, exp(g) FP16 [128], beta), gates g and beta.
BYTES_KDA_WINDOW = (20224 + 20224 / WINDOW + 784 * (WINDOW - 1) / 2 + 784 * (WINDOW - 1) / WINDOW
                    + 3 * 512 + 512 + 4)


def run_window(torch, binding, inputs, dev_in, perm, c, n, H, warmup, use_graph, reps=16,
               staggered=False, ends_first=False, kind="gdn", warm_s=0.5):
    """GDN per-window decode at the serving shape, `reps` whole windows timed;
    returns (seconds per token step, ok).  Every slot in the same phase, or
    (staggered) slot s at position (s + t) mod window at step t, so that each
    step has slots at every position and 1/window of them end their window.
    ends_first: the batch lists the slots by descending window position at
    every step (a scheduling choice of the caller), so the requests that
    replay their window come first in the grid."""
    pool = binding.StatePool(binding.FMT_I8F16, n, H, perm, c)
    slots = torch.arange(n, dtype=torch.int32, device="cuda")
    pool.store(slots, torch.from_numpy(inputs.initial_state(1 if kind == "gdn" else 2, n, H)).to("cuda"))
    buf = pool.window_buffer(kind, WINDOW)
    gate = "alpha" if kind == "gdn" else "g"
    order = [slots] * WINDOW
    if staggered:
        pos = [((torch.arange(n, device="cuda") + j) % WINDOW).to(torch.int32) for j in range(WINDOW)]
        if ends_first:
            order = [torch.sort(pj.long(), descending=True, stable=True).indices.to(torch.int32)
                     for pj in pos]
            pos = [pj[o.long()].contiguous() for pj, o in zip(pos, order)]
    else:
        pos = [torch.full((n,), j, dtype=torch.int32, device="cuda") for j in range(WINDOW)]
    out = torch.empty((n, H, 128), dtype=torch.float32, device="cuda")
    T = dev_in["q"].shape[0]

    def launch(t):
        tt = t % T
        pool.window_step(kind, WINDOW, buf, order[t % WINDOW], pos[t % WINDOW], dev_in["q"][tt],
                         dev_in["k"][tt], dev_in["v"][tt], dev_in[gate][tt], dev_in["beta"][tt],
                         out=out)

    steps = reps * WINDOW
    passes, _ = time_loop(torch, launch, steps, WINDOW, use_graph, warm_s=warm_s)
    ok = bool(torch.isfinite(out).all().item())
    pool.close()
    torch.cuda.empty_cache()
    return pass_stats(passes, steps)["per_step"], ok


# Key-channel selection, calibration-shaped: 32 sequences of 256 steps, 32
# heads, one sampled state every 8 steps (1,024 samples per head).  The error
# kernel reads every sampled FP32 state once (64 KiB per sample and head).
SELECT_SEQ, SELECT_T, SELECT_EVERY = 32, 256, 8


def run_copy_reference(torch, nbytes, reps=20):
    """A plain device copy (torch copy_) of nbytes, reading nbytes and writing
    nbytes: the rate a kernel that reads and writes each byte once can expect
    on this machine.  Two source/destination pairs alternate, so the working set
    exceeds the 256 MB Infinity Cache.  Returns (seconds per copy, GB/s)."""
    bufs = [(torch.empty(nbytes, dtype=torch.uint8, device="cuda"),
             torch.empty(nbytes, dtype=torch.uint8, device="cuda")) for _ in range(2)]
    for a, b in bufs:
        b.copy_(a)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(reps):
        a, b = bufs[i % 2]
        b.copy_(a)
    end.record()
    torch.cuda.synchronize()
    secs = start.elapsed_time(end) / 1e3 / reps
    del bufs
    torch.cuda.empty_cache()
    return secs, 2 * nbytes / secs / 1e9


def run_select(torch, binding, H, reps=3):
    g = torch.Generator(device="cuda")
    g.manual_seed(1234)
    n_seq, T = SELECT_SEQ, SELECT_T
    seqs = torch.arange(n_seq, dtype=torch.int32, device="cuda").repeat_interleave(T // SELECT_EVERY)
    ts = torch.arange(SELECT_EVERY - 1, T, SELECT_EVERY, dtype=torch.int32,
                      device="cuda").repeat(n_seq)
    n = seqs.numel()
    S = 0.1 * torch.randn((n, H, 128, 128), generator=g, device="cuda", dtype=torch.float32)
    a = 0.5 + 0.5 * torch.rand((n_seq, T, H, 128), generator=g, device="cuda", dtype=torch.float32)
    c = torch.exp(torch.empty((H, 128), device="cuda").uniform_(-0.69, 0.69, generator=g))
    w = torch.full((n,), 1.0 / n, dtype=torch.float64, device="cuda")
    stream = torch.cuda.current_stream()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            r = fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / reps, r

    t_err, e = timed(lambda: binding.channel_error(S, c))
    t_win, W = timed(lambda: binding.persistence_window(a, seqs, ts, 256))
    t_geo, P = timed(lambda: binding.persistence_geometric(a, seqs, ts, w, 1e-4))
    t_sw, C = timed(lambda: binding.channel_scores(e, w, W=W))
    t_sp, _ = timed(lambda: binding.channel_scores(e, w, P=P))
    t0 = time.perf_counter()
    perm = binding.select_protected_channels(C)
    t_sel = time.perf_counter() - t0
    ok = bool(torch.isfinite(C).all().item()) and perm.shape == (H, 128)
    err_bytes = n * H * (128 * 128 * 4 + 128 * 8)
    del S, a
    torch.cuda.empty_cache()
    return {"workload": f"{n_seq} sequences x {T} steps x {H} heads, a state every "
                        f"{SELECT_EVERY} steps ({n} samples), window 256",
            "channel_error_ms": t_err * 1e3, "channel_error_gbs": err_bytes / t_err / 1e9,
            "channel_error_frac_of_peak": err_bytes / t_err / 1e9 / PEAK_HBM_GBS,
            "persistence_window_ms": t_win * 1e3, "persistence_geometric_ms": t_geo * 1e3,
            "scores_window_ms": t_sw * 1e3, "scores_geometric_ms": t_sp * 1e3,
            "select_host_ms": t_sel * 1e3, "finite": ok}


def cpu_select_baseline(H, samples=192):
    """The oracle's channel-error step on a bounded sample (samples x H states)."""
    from oracle import selector

    r = np.random.default_rng(5)
    S = (0.1 * r.standard_normal((samples, H, 128, 128))).astype(np.float32)
    c = np.exp(r.uniform(-0.69, 0.69, (H, 128))).astype(np.float32)
    t0 = time.perf_counter()
    selector.channel_error(S, c)
    dt = time.perf_counter() - t0
    import oracle

    return {"channel_error_samples_per_s": samples / dt,
            "sample": f"{samples} states x {H} heads", "seconds": dt,
            "cores": oracle.max_threads()}


def cpu_prefill_baseline(inputs, seqs=8, tokens=4096):
    """The oracle's chunked prefill (sequential FP32 recurrence inside each
    chunk of 64, compressed chunk ends) on a bounded sample of the prefill
    workload: `seqs` sequences x 32 heads x `tokens` tokens, zero start."""
    import oracle

    H = 32
    d = inputs.prefill_inputs(3, seqs, H, tokens)
    op = oracle.OraclePool(seqs, H, inputs.protected_perm(3, H), inputs.smoothing(3, H, False))
    slots = np.arange(seqs, dtype=np.int32)
    t0 = time.perf_counter()
    op.prefill(slots, d["q"], d["k"], d["v"], d["alpha"], d["beta"], PREFILL_CHUNK, False)
    dt = time.perf_counter() - t0
    return {"tokens_per_s": seqs * tokens / dt, "head_updates_per_s": seqs * tokens * H / dt,
            "sample": f"{seqs} sequence(s) x {H} heads x {tokens} tokens, chunks of {PREFILL_CHUNK}, "
                      "zero initial state, INT8 tier",
            "seconds": dt, "kind": "oracle", "cores": oracle.max_threads()}


def cpu_baseline(inputs, kind, budget_s=None):
    """The oracle on the decode workload: all 256 slots x 32 heads, all 256
    steps (the full workload), or only the first consecutive steps that fit
    in about `budget_s` seconds of step-loop time (at least 2)."""
    import oracle

    cfg = 1 if kind == "gdn" else 2
    n, H = 256, 32
    perm = inputs.protected_perm(cfg, H)
    c = inputs.smoothing(cfg, H, True)
    op = oracle.OraclePool(n, H, perm, c)
    slots = np.arange(n, dtype=np.int32)
    op.store(slots, inputs.initial_state(cfg, n, H))
    gate = "alpha" if kind == "gdn" else "g"
    elapsed, steps = 0.0, 0
    while steps < 256 and (budget_s is None or elapsed < budget_s or steps < 2):
        d = inputs.step_inputs(cfg, steps, n, H, kind)
        t0 = time.perf_counter()
        op.decode_step(slots, d["q"], d["k"], d["v"], d[gate], d["beta"], 0 if kind == "gdn" else 1)
        elapsed += time.perf_counter() - t0
        steps += 1
    ups = n * H * steps / elapsed
    return {"value": ups, "unit": "state updates/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"{kind.upper()} decode, {n} slots x {H} heads x {steps} consecutive steps "
                      f"({n * H * steps} updates, {elapsed:.1f} s of step-loop time)"
                      + (" -- the full workload" if steps == 256 else ""),
            "gbs_algorithmic": ups * (BYTES_GDN if kind == "gdn" else BYTES_KDA) / 1e9}


# Paged decode over a shared pool: 4,096 slots x 32 heads (GDN-typed slots
# [0, 2048), KDA-typed [2048, 4096)), 1,024 active requests (512 of each type,
# distinct random ids); a step is one GDN call and one KDA call.  Algorithmic
# bytes per step: 16,384 GDN updates x 41,992 + 16,384 KDA updates x 42,500.
PAGED_SLOTS, PAGED_ACTIVE = 4096, 1024
PAGED_BYTES_PER_STEP = (PAGED_ACTIVE // 2) * 32 * (BYTES_GDN + BYTES_KDA)
PAGED_UPDATES_PER_STEP = PAGED_ACTIVE * 32


def run_paged(torch, binding, inputs, steps, warmup, use_graph, reps=5, warm_s=0.5, streams=1,
              sorted_slots=False, pair=False):
    """Paged decode, inputs drawn on the device with the workload's recipe
    (heavy-tailed initial states with outlier rows in the FP16 channels,
    smoothing on).  streams=1: both calls of a step on one stream, in order;
    streams=2: the KDA calls on a second stream (the two request groups share
    no slot, so each group's steps stay in order on its own stream and the
    two chains overlap).  sorted_slots: each call lists its requests in
    ascending slot order (the same random slot ids; the order of requests in
    a batch is the caller's choice), so the workgroups resident at any time
    touch nearby parts of the 2.65 GB pool.  pair: both groups in one
    qrs_decode_step_pair call per step (one launch).  Returns the pass_stats
    dict (seconds per step)."""
    cfg, H = 4, 32
    perm = inputs.protected_perm(cfg, H)
    c = inputs.smoothing(cfg, H, True)
    gdn_slots, kda_slots = inputs.paged_slots(cfg, PAGED_SLOTS, PAGED_ACTIVE)
    if sorted_slots:
        gdn_slots, kda_slots = np.sort(gdn_slots), np.sort(kda_slots)
    t0 = time.time()
    pool = binding.StatePool(binding.FMT_I8F16, PAGED_SLOTS, H, perm, c)
    active = np.concatenate([gdn_slots, kda_slots])
    for i in range(0, len(active), 64):
        S = inputs.initial_state_device(cfg, min(64, len(active) - i), H, perm, first=i)
        pool.store(torch.from_numpy(np.ascontiguousarray(active[i:i + 64])).to("cuda"), S)
        del S
    total = steps + warmup
    ins = {kind: [inputs.step_inputs_device(cfg, t, PAGED_ACTIVE // 2, H, kind)
                  for t in range(total)] for kind in ("gdn", "kda")}
    torch.cuda.synchronize()
    log(f"[bench] staged the paged pool and {total} steps of inputs in {time.time() - t0:.1f}s")
    dsl = {"gdn": torch.from_numpy(gdn_slots).to("cuda"), "kda": torch.from_numpy(kda_slots).to("cuda")}
    out = {kind: torch.empty((PAGED_ACTIVE // 2, H, 128), device="cuda") for kind in ("gdn", "kda")}

    side = torch.cuda.Stream() if streams == 2 else None

    def launch(t):
        a, b = ins["gdn"][t], ins["kda"][t]
        if pair:
            pool.pair_step((dsl["gdn"], a["q"], a["k"], a["v"], a["alpha"], a["beta"]),
                           (dsl["kda"], b["q"], b["k"], b["v"], b["g"], b["beta"]),
                           out["gdn"], out["kda"])
            return
        pool.gdn_step(dsl["gdn"], a["q"], a["k"], a["v"], a["alpha"], a["beta"], out["gdn"])
        if side is None:
            pool.kda_step(dsl["kda"], b["q"], b["k"], b["v"], b["g"], b["beta"], out["kda"])
        else:
            with torch.cuda.stream(side):
                pool.kda_step(dsl["kda"], b["q"], b["k"], b["v"], b["g"], b["beta"], out["kda"])

    passes, _ = time_loop(torch, launch, steps, warmup, use_graph, reps=reps, warm_s=warm_s,
                          side=side)
    st = pass_stats(passes, steps)
    st["ok"] = all(bool(torch.isfinite(o).all().item()) for o in out.values())
    pool.close()
    del pool, ins, out
    torch.cuda.empty_cache()
    return st


# Batch sweep: the kernel speedup of the compressed state over the FP32 state
# (the pages' kernel metric, reported for batches 16 to 256 and beyond), one
# GPU, 32 heads.  Each leg rotates enough disjoint slot sets that its working
# set exceeds 640 MB (2.5x the 256 MB Infinity Cache), so every state read
# comes from HBM as it would for the layers of a model.
SWEEP_BATCHES = (16, 32, 64, 128, 256, 512)
SWEEP_INPUT_STEPS = 32
SWEEP_MIN_WORKING_SET = 640 << 20


def run_sweep(torch, binding, inputs, steps, warmup, use_graph, reps=5, warm_s=0.25):
    H, nmax = 32, max(SWEEP_BATCHES)
    t0 = time.time()
    perm = inputs.protected_perm(1, H)
    c = inputs.smoothing(1, H, True)
    S0 = inputs.initial_state_device(1, nmax, H, perm)
    ins = {kind: [inputs.step_inputs_device(1 if kind == "gdn" else 2, t, nmax, H, kind)
                  for t in range(SWEEP_INPUT_STEPS)] for kind in ("gdn", "kda")}
    torch.cuda.synchronize()
    log(f"[bench] staged sweep states and inputs in {time.time() - t0:.1f}s")
    out = {}
    for n in SWEEP_BATCHES:
        row = {}
        for kind in ("gdn", "kda"):
            gate = "alpha" if kind == "gdn" else "g"
            for fmt, name in ((binding.FMT_I8F16, "compressed"), (binding.FMT_FP32, "fp32_state")):
                unit = 20224 if fmt == binding.FMT_I8F16 else 65536
                sets = max(1, -(-SWEEP_MIN_WORKING_SET // (n * H * unit)))
                pool = binding.StatePool(fmt, n * sets, H, perm, c)
                slot_sets = [torch.arange(p * n, (p + 1) * n, dtype=torch.int32, device="cuda")
                             for p in range(sets)]
                for sl in slot_sets:
                    pool.store(sl, S0[:n])
                o = torch.empty((n, H, 128), device="cuda")
                fn = pool.gdn_step if kind == "gdn" else pool.kda_step

                def launch(t, fn=fn, slot_sets=slot_sets, o=o, n=n, kind=kind, gate=gate):
                    d = ins[kind][t % SWEEP_INPUT_STEPS]
                    fn(slot_sets[t % len(slot_sets)], d["q"][:n], d["k"][:n], d["v"][:n],
                       d[gate][:n], d["beta"][:n], o)

                passes, _ = time_loop(torch, launch, steps, warmup, use_graph, reps=reps,
                                      warm_s=warm_s)
                st = pass_stats(passes, steps)
                nb = (BYTES_GDN if kind == "gdn" else BYTES_KDA) if fmt == binding.FMT_I8F16 else \
                    (65536 * 2 + (BYTES_GDN if kind == "gdn" else BYTES_KDA) - 2 * 20224)
                row[f"{kind}_{name}"] = {
                    "us_per_step": st["per_step"] * 1e6, "us_min": st["per_step_min"] * 1e6,
                    "us_max": st["per_step_max"] * 1e6, "slot_sets": sets,
                    "updates_per_s": n * H / st["per_step"],
                    "frac_of_peak": n * H * nb / st["per_step"] / 1e9 / PEAK_HBM_GBS,
                    "finite_outputs": bool(torch.isfinite(o).all().item())}
                pool.close()
                del pool, o
                torch.cuda.empty_cache()
            row[f"{kind}_speedup_vs_fp32_state"] = (row[f"{kind}_fp32_state"]["us_per_step"]
                                                    / row[f"{kind}_compressed"]["us_per_step"])
        out[str(n)] = row
        log(f"[bench] sweep batch {n}: gdn {row['gdn_compressed']['us_per_step']:.2f} us "
            f"(x{row['gdn_speedup_vs_fp32_state']:.2f}), kda {row['kda_compressed']['us_per_step']:.2f} us "
            f"(x{row['kda_speedup_vs_fp32_state']:.2f})")
    del S0, ins
    torch.cuda.empty_cache()
    return {"workload": "GDN and KDA decode, batch x 32 heads, d_k = d_v = 128, heavy-tailed "
                        "initial states, smoothing on; compressed state (16 FP16 + 112 INT8 rows) "
                        "against the FP32-state kernel on the same inputs; slot sets rotated so "
                        "each leg's working set exceeds 640 MB",
            "input_steps_cycled": SWEEP_INPUT_STEPS, "batches": out}


def host_cpu_info():
    """The host CPU model, the logical CPUs this process may run on, and the
    physical cores behind them (Linux /proc and /sys)."""
    model, ident = None, {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                key, _, val = line.partition(":")
                key = key.strip()
                if key == "model name" and model is None:
                    model = val.strip()
                elif key in ("vendor_id", "cpu family", "model", "stepping", "cpu MHz") \
                        and key not in ident:
                    ident[key] = val.strip()
                elif not line.strip() and model is not None:
                    break
    except OSError:
        pass
    if ident:
        model = (f"{model} ({ident.get('vendor_id', '?')} family {ident.get('cpu family', '?')} "
                 f"model {ident.get('model', '?')} stepping {ident.get('stepping', '?')}, "
                 f"{ident.get('cpu MHz', '?')} MHz)")
    try:
        cpus = sorted(os.sched_getaffinity(0))
    except AttributeError:
        cpus = list(range(os.cpu_count() or 1))
    cores = set()
    for cpu in cpus:
        base = f"/sys/devices/system/cpu/cpu{cpu}/topology/"
        try:
            with open(base + "physical_package_id") as f:
                pkg = f.read().strip()
            with open(base + "core_id") as f:
                core = f.read().strip()
            cores.add((pkg, core))
        except OSError:
            cores.add(("?", str(cpu)))
    return {"cpu_model": model, "logical_cpus_available": len(cpus),
            "physical_cores_available": len(cores)}


def cpu_paged_baseline(inputs, units_per_kind=512, steps=1024):
    """The oracle on 1,024 seeded units of the paged workload (16 GDN and 16
    KDA slots x 32 heads) over all 1,024 steps, host-drawn inputs of the same
    recipe.  Units are independent, so the rate per update extrapolates to
    the full 32,768 units per step."""
    import oracle

    cfg, H = 4, 32
    nb = units_per_kind // H
    perm = inputs.protected_perm(cfg, H)
    c = inputs.smoothing(cfg, H, True)
    op = oracle.OraclePool(2 * nb, H, perm, c)
    sl = {"gdn": np.arange(nb, dtype=np.int32), "kda": np.arange(nb, 2 * nb, dtype=np.int32)}
    for kind in ("gdn", "kda"):
        op.store(sl[kind], inputs.initial_state(cfg, nb, H, perm, heavy_tailed=True,
                                                first=0 if kind == "gdn" else PAGED_ACTIVE // 2))
    elapsed = 0.0
    for t in range(steps):
        for kind in ("gdn", "kda"):
            d = inputs.step_inputs(cfg, t, nb, H, kind)
            t0 = time.perf_counter()
            op.decode_step(sl[kind], d["q"], d["k"], d["v"], d["alpha" if kind == "gdn" else "g"],
                           d["beta"], 0 if kind == "gdn" else 1)
            elapsed += time.perf_counter() - t0
    ups = 2 * units_per_kind * steps / elapsed
    return {"value": ups, "unit": "state updates/s", "kind": "oracle", "cores": oracle.max_threads(),
            "sample": f"{2 * units_per_kind} units ({nb} GDN + {nb} KDA slots x {H} heads) x "
                      f"{steps} steps ({elapsed:.1f} s of step-loop time); extrapolated per update "
                      "to the 32,768 units of a full step",
            "us_per_full_step_extrapolated": PAGED_UPDATES_PER_STEP / ups * 1e6,
            "gbs_algorithmic": ups * (BYTES_GDN + BYTES_KDA) / 2 / 1e9, "seconds": elapsed}


def traffic_from_profile(units):
    """HBM bytes per launch from committed rocprofv3 counter summaries, when
    they were taken on the current kernel source."""
    try:
        with open(COUNTERS_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_digest") != kernel_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


def profile_from_trace():
    """The headline kernel's average launch duration in the timed passes of
    the committed rocprofv3 kernel trace, when it was taken on the current
    kernel source (the figure the roofline's achieved bandwidth must agree
    with)."""
    try:
        with open(TRACE_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_digest") != kernel_digest():
        return None
    return {key: rec.get(key) for key in ("kernel", "command", "timed_launches",
                                         "us_per_launch_avg", "us_per_launch_median")}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=248)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--reps", type=int, default=5,
                    help="timed passes over the steps per leg (the median is reported)")
    ap.add_argument("--device-warmup-s", type=float, default=2.0,
                    help="seconds of decode steps run before the first leg's timed passes")
    ap.add_argument("--leg-warmup-s", type=float, default=0.5,
                    help="seconds of each later leg's own steps run before its timed passes "
                         "(the GPU idles while a leg's inputs and pool are set up)")
    ap.add_argument("--pools", type=int, default=4,
                    help="slot sets rotated per step (4 = cache-cold working set)")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["gdn", "kda", "f32", "v1", "bf16", "window", "prefill",
                                       "select", "paged", "sweep", "all"],
                    default="all")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="also run a plain device copy of this size (counter calibration)")
    ap.add_argument("--windows", type=int, default=16,
                    help="whole windows per timed pass of the per-window legs")
    ap.add_argument("--decode-split", choices=["auto", "whole", "halves"], default="auto",
                    help="INT8-tier decode kernel: by grid size (default), one workgroup per "
                         "unit, or two per unit (value-column halves)")
    ap.add_argument("--oracle-only", action="store_true",
                    help="time the oracle alone (CPU; used for the single-thread figure)")
    args = ap.parse_args()

    if args.oracle_only:
        from quantized_recurrent_state_02_amd import inputs
        print(json.dumps(cpu_baseline(inputs, "gdn", budget_s=4.0)))
        return

    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; it has no multi-GPU "
                                   "mode (decode units would shard by slot or head with no "
                                   "exchange)", "n_gpus": args.gpus}))
        sys.exit(2)

    # The oracle on one thread, in a child process started before this one
    # touches the GPU (OpenMP fixes its thread count when the library loads).
    cpu_1t = None
    if not args.no_cpu_baseline and args.only == "all":
        import subprocess
        env = dict(os.environ, OMP_NUM_THREADS="1")
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--oracle-only"],
                           env=env, capture_output=True, text=True, timeout=300)
        if r.returncode == 0 and r.stdout.strip():
            cpu_1t = json.loads(r.stdout.strip().splitlines()[-1])
            log(f"[bench] cpu oracle, 1 thread: {cpu_1t['value']:.3e} updates/s")

    import torch
    from quantized_recurrent_state_02_amd import binding, inputs

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    binding.load()
    binding.set_decode_split({"auto": binding.DECODE_SPLIT_AUTO, "whole": binding.DECODE_SPLIT_WHOLE,
                              "halves": binding.DECODE_SPLIT_HALVES}[args.decode_split])
    torch.cuda.set_device(0)
    n, H = 256, 32
    steps, warmup, reps = args.steps, args.warmup, args.reps
    total = steps + warmup
    use_graph = not args.no_graph
    units = n * H
    res = {}
    kda_cpu = None
    kda_window = None
    warm_s = args.device_warmup_s   # the first timed leg; later legs warm up for leg_warm
    leg_warm = args.leg_warmup_s

    if args.calib_copy_mb:
        nb = args.calib_copy_mb << 20
        a = torch.empty(nb, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {nb} bytes done (3 launches)")

    def decode(key, *a, **kw):
        nonlocal warm_s
        st = run_decode(torch, binding, inputs, *a, reps=reps, warm_s=warm_s, **kw)
        warm_s = leg_warm
        res[key] = st
        log(f"[bench] {key[0]} pools={key[1]}: {st['per_step'] * 1e6:.2f} us/step "
            f"(min {st['per_step_min'] * 1e6:.2f}, max {st['per_step_max'] * 1e6:.2f}) ok={st['ok']}")
        return st

    perm1 = inputs.protected_perm(1, H)
    c1 = inputs.smoothing(1, H, True)
    codec_cmp = None
    window_res = None
    copy_ref = None
    if args.only in ("gdn", "f32", "v1", "bf16", "window", "all"):
        gdn_in = stage_inputs(torch, inputs, 1, "gdn", n, H, total)
        if args.only in ("gdn", "all"):
            for pools in sorted({args.pools, 1}, reverse=True):
                decode(("gdn", pools), "gdn", binding.FMT_I8F16, gdn_in, perm1, c1, n, H, steps,
                       warmup, pools, use_graph)
            if args.only == "all":
                # one GPU's share under 8-way tensor parallelism: 4 of the 32
                # heads of every slot (1,024 units per step)
                h4 = 4
                in4 = {key: val[:, :, :h4].contiguous() for key, val in gdn_in.items()}
                decode(("gdnh4", args.pools), "gdn", binding.FMT_I8F16, in4,
                       inputs.protected_perm(1, h4), inputs.smoothing(1, h4, True), n, h4, steps,
                       warmup, args.pools, use_graph)
                del in4
            if use_graph:
                # the same steps as launched one by one (no graph)
                decode(("gdneager", args.pools), "gdn", binding.FMT_I8F16, gdn_in, perm1, c1, n,
                       H, steps, warmup, args.pools, False)
            # the same bytes as one decode step, half read and half written
            copy_ref = run_copy_reference(torch, n * H * BYTES_GDN // 2)
            log(f"[bench] device copy of the same bytes: {copy_ref[0] * 1e6:.2f} us, {copy_ref[1]:.0f} GB/s")
        if args.only in ("f32", "all"):
            decode(("f32", 1), "gdn", binding.FMT_FP32, gdn_in, perm1, c1, n, H, steps, warmup, 1,
                   use_graph)
        if args.only in ("bf16", "all"):
            decode(("gdnbf16io", args.pools), "gdn", binding.FMT_I8F16, gdn_in, perm1, c1, n, H,
                   steps, warmup, args.pools, use_graph, io_bf16=True)
        if args.only in ("window", "all"):
            sec_w, ok_w = run_window(torch, binding, inputs, gdn_in, perm1, c1, n, H, warmup,
                                     use_graph, reps=args.windows, warm_s=leg_warm)
            window_res = {"workload": f"GDN, {n} slots x {H} heads, windows of {WINDOW} tokens, "
                                      "all slots in phase, 16 windows per timed pass",
                          "us_per_step": sec_w * 1e6, "updates_per_s": n * H / sec_w,
                          "bytes_per_update": BYTES_GDN_WINDOW,
                          "gbs": n * H * BYTES_GDN_WINDOW / sec_w / 1e9,
                          "frac_of_peak": n * H * BYTES_GDN_WINDOW / sec_w / 1e9 / PEAK_HBM_GBS,
                          "finite_outputs": ok_w}
            log(f"[bench] gdn per-window (16): {sec_w * 1e6:.2f} us/step ok={ok_w}")
            sec_s, ok_s = run_window(torch, binding, inputs, gdn_in, perm1, c1, n, H, warmup,
                                     use_graph, reps=args.windows, staggered=True, warm_s=leg_warm)
            window_res["staggered"] = {
                "workload": "the same, slot s at position (s + t) mod 16 at step t",
                "us_per_step": sec_s * 1e6, "updates_per_s": n * H / sec_s,
                "gbs": n * H * BYTES_GDN_WINDOW / sec_s / 1e9,
                "frac_of_peak": n * H * BYTES_GDN_WINDOW / sec_s / 1e9 / PEAK_HBM_GBS,
                "finite_outputs": ok_s}
            log(f"[bench] gdn per-window (16), staggered phases: {sec_s * 1e6:.2f} us/step ok={ok_s}")
            sec_e, ok_e = run_window(torch, binding, inputs, gdn_in, perm1, c1, n, H, warmup,
                                     use_graph, reps=args.windows, staggered=True, ends_first=True,
                                     warm_s=leg_warm)
            window_res["staggered_ends_first"] = {
                "workload": "the same staggered phases, the batch ordered by descending window "
                            "position at every step (the caller listing the window-end requests first, "
                            "the order the kernel itself gives a mixed call)",
                "us_per_step": sec_e * 1e6, "updates_per_s": n * H / sec_e,
                "gbs": n * H * BYTES_GDN_WINDOW / sec_e / 1e9,
                "frac_of_peak": n * H * BYTES_GDN_WINDOW / sec_e / 1e9 / PEAK_HBM_GBS,
                "finite_outputs": ok_e}
            log(f"[bench] gdn per-window (16), staggered, window ends first: {sec_e * 1e6:.2f} us/step")
        if args.only in ("v1", "all"):
            decode(("gdnv1", args.pools), "gdn", binding.FMT_U8H16, gdn_in, perm1, c1, n, H, steps,
                   warmup, args.pools, use_graph)
            codec_cmp = run_codec_compare(torch, binding, inputs, gdn_in, perm1, c1, n, H,
                                          min(256, total))
            log(f"[bench] codec comparison: {codec_cmp}")
        del gdn_in
        torch.cuda.empty_cache()
    if args.only in ("kda", "window", "all"):
        perm2 = inputs.protected_perm(2, H)
        c2 = inputs.smoothing(2, H, True)
        kda_in = stage_inputs(torch, inputs, 2, "kda", n, H, total)
        if args.only != "window":
            for pools in sorted({args.pools, 1}, reverse=True):
                decode(("kda", pools), "kda", binding.FMT_I8F16, kda_in, perm2, c2, n, H, steps,
                       warmup, pools, use_graph)
        if args.only in ("all", "window"):
            sec_k, ok_k = run_window(torch, binding, inputs, kda_in, perm2, c2, n, H, warmup,
                                     use_graph, reps=args.windows, kind="kda", warm_s=leg_warm)
            kda_window = {
                "workload": "KDA, 256 slots x 32 heads, windows of 16 tokens, all slots in phase",
                "us_per_step": sec_k * 1e6, "updates_per_s": n * H / sec_k,
                "bytes_per_update": BYTES_KDA_WINDOW,
                "gbs": n * H * BYTES_KDA_WINDOW / sec_k / 1e9,
                "frac_of_peak": n * H * BYTES_KDA_WINDOW / sec_k / 1e9 / PEAK_HBM_GBS,
                "finite_outputs": ok_k}
            log(f"[bench] kda per-window (16): {sec_k * 1e6:.2f} us/step ok={ok_k}")
        del kda_in
        torch.cuda.empty_cache()

    paged = None
    if args.only in ("paged", "all"):
        st = run_paged(torch, binding, inputs, steps, warmup, use_graph, reps=reps, warm_s=leg_warm)
        per = st["per_step"]
        paged = {"workload": "paged decode: 4,096 slots x 32 heads (2,048 GDN-typed + 2,048 "
                             "KDA-typed), 1,024 active requests with distinct random slot ids "
                             "(512 + 512), one GDN call and one KDA call per step, heavy-tailed "
                             "initial states, smoothing on",
                 "us_per_step": per * 1e6, "us_min": st["per_step_min"] * 1e6,
                 "us_max": st["per_step_max"] * 1e6, "timed_passes": st["passes"],
                 "updates_per_s": PAGED_UPDATES_PER_STEP / per,
                 "bytes_per_step": PAGED_BYTES_PER_STEP,
                 "gbs": PAGED_BYTES_PER_STEP / per / 1e9,
                 "frac_of_peak": PAGED_BYTES_PER_STEP / per / 1e9 / PEAK_HBM_GBS,
                 "us_per_step_at_70pct_of_peak": PAGED_BYTES_PER_STEP / (0.7 * PEAK_HBM_GBS * 1e9) * 1e6,
                 "finite_outputs": st["ok"]}
        log(f"[bench] paged mixed pool: {per * 1e6:.2f} us/step, {paged['frac_of_peak'] * 100:.1f}% of peak")
        for key, streams, srt, pr, what in (
                ("two_streams", 2, False, False,
                 "the same steps, the KDA request group's calls on a second stream (one fork and one join "
                 "per timed pass; each group's steps stay in order)"),
                ("one_launch", 1, False, True,
                 "the same steps, both request groups in one qrs_decode_step_pair call per step (one launch)"),
                ("sorted", 1, True, False,
                 "the same random slot ids, each call listing its requests in ascending slot order (a "
                 "scheduling choice of the caller), one stream"),
                ("sorted_two_streams", 2, True, False,
                 "ascending slot order and the KDA calls on a second stream"),
                ("sorted_one_launch", 1, True, True, "ascending slot order, one pair call per step")):
            st2 = run_paged(torch, binding, inputs, steps, warmup, use_graph, reps=reps, warm_s=leg_warm,
                            streams=streams, sorted_slots=srt, pair=pr)
            per2 = st2["per_step"]
            paged[key] = {
                "workload": what,
                "us_per_step": per2 * 1e6, "us_min": st2["per_step_min"] * 1e6,
                "us_max": st2["per_step_max"] * 1e6, "updates_per_s": PAGED_UPDATES_PER_STEP / per2,
                "gbs": PAGED_BYTES_PER_STEP / per2 / 1e9,
                "frac_of_peak": PAGED_BYTES_PER_STEP / per2 / 1e9 / PEAK_HBM_GBS,
                "finite_outputs": st2["ok"]}
            log(f"[bench] paged mixed pool, {key}: {per2 * 1e6:.2f} us/step, "
                f"{paged[key]['frac_of_peak'] * 100:.1f}% of peak")

    sweep = None
    if args.only in ("sweep", "all"):
        sweep = run_sweep(torch, binding, inputs, steps, warmup, use_graph, reps=reps,
                          warm_s=min(leg_warm, 0.25))

    prefill = {}
    if args.only in ("prefill", "all"):
        for bf16 in (False, True):
            secs, st = run_prefill(torch, binding, inputs, bf16)
            prefill["bf16" if bf16 else "fp32"] = st
            log(f"[bench] prefill {'bf16' if bf16 else 'fp32'}: {secs * 1e3:.3f} ms/call, "
                f"{st['tflops_fp32_mfma']:.1f} TFLOP/s fp32 mfma")
        secs, st = run_prefill(torch, binding, inputs, False, fmt=binding.FMT_U8H16)
        prefill["v1_fp32"] = st
        log(f"[bench] prefill v1 tier fp32: {secs * 1e3:.3f} ms/call")

    select = {}
    if args.only in ("select", "all"):
        select = run_select(torch, binding, H)
        log(f"[bench] channel selection: error {select['channel_error_ms']:.3f} ms "
            f"({select['channel_error_gbs']:.0f} GB/s), window {select['persistence_window_ms']:.3f} ms")

    # ---- the oracle on the host's cores (after all GPU legs) ----
    host = host_cpu_info()
    if not args.no_cpu_baseline:
        if args.only in ("kda", "all"):
            kda_cpu = cpu_baseline(inputs, "kda")
            log(f"[bench] kda cpu oracle: {kda_cpu['value']:.3e} updates/s")
        if prefill:
            prefill["cpu_oracle"] = cpu_prefill_baseline(inputs)
            log(f"[bench] prefill cpu oracle: {prefill['cpu_oracle']['tokens_per_s']:.3e} tokens/s")
        if paged is not None:
            paged["cpu_oracle"] = cpu_paged_baseline(inputs)
            log(f"[bench] paged cpu oracle: {paged['cpu_oracle']['value']:.3e} updates/s")
        if select:
            select["cpu_oracle"] = cpu_select_baseline(H)

    def rate(key, nbytes):
        st = res[key]
        per_step = st["per_step"]
        ups = (n * 4 if key[0] == "gdnh4" else units) / per_step
        return {"us_per_step": per_step * 1e6, "us_min": st["per_step_min"] * 1e6,
                "us_max": st["per_step_max"] * 1e6, "timed_passes": st["passes"],
                "updates_per_s": ups, "gbs": ups * nbytes / 1e9,
                "frac_of_peak": ups * nbytes / 1e9 / PEAK_HBM_GBS, "finite_outputs": st["ok"]}

    def diag(metric, value, unit, workload, roof, det):
        print(json.dumps({"metric": metric, "value": value, "unit": unit, "n_gpus": 1,
                          "higher_is_better": True, "dtype": "f32", "data": "synthetic",
                          "config": {"workload": workload}, "roofline": roof, "detail": det}))

    if not res and window_res:   # --only window: a diagnostic line for per-window decode
        diag("per-window decode: state updates/s (windows of 16 tokens)",
             window_res["updates_per_s"], "state updates/s", window_res["workload"],
             {"bound": "hbm", "achieved": window_res["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
              "frac": window_res["frac_of_peak"], "traffic": None},
             {"window": window_res, "kda_window": kda_window})
        return
    if not res and select:   # --only select: a diagnostic line for the selection kernels
        diag("key-channel selection: calibration states scored per second",
             1024 / (select["channel_error_ms"] / 1e3), "samples/s", select["workload"],
             {"bound": "hbm", "achieved": select["channel_error_gbs"], "peak": PEAK_HBM_GBS,
              "unit": "GB/s", "frac": select["channel_error_frac_of_peak"], "traffic": None},
             {"select": select})
        return
    if not res and paged:    # --only paged
        diag("paged decode: state updates/s over a mixed GDN/KDA pool", paged["updates_per_s"],
             "state updates/s", paged["workload"],
             {"bound": "hbm", "achieved": paged["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
              "frac": paged["frac_of_peak"], "traffic": None}, {"paged": paged})
        return
    if not res and sweep:    # --only sweep
        sweep["decode_split"] = args.decode_split
        b256 = sweep["batches"]["256"]
        diag("decode speedup of the compressed state over the FP32 state, batch sweep",
             b256["gdn_speedup_vs_fp32_state"], "x", sweep["workload"],
             {"bound": "hbm", "achieved": None, "peak": PEAK_HBM_GBS, "unit": "GB/s",
              "frac": b256["gdn_compressed"]["frac_of_peak"], "traffic": None}, {"sweep": sweep})
        return
    if not res:   # --only prefill: a diagnostic line for the prefill kernel alone
        st = prefill["fp32"]
        diag("prefill tokens/s (chunked, compressed state)", st["tokens_per_s"], "tokens/s",
             st["workload"],
             {"bound": "mfma", "achieved": st["tflops_fp32_mfma"], "peak": PEAK_FP32_MFMA_TFLOPS,
              "unit": "TFLOP/s", "frac": st["frac_of_fp32_mfma_peak"], "traffic": None},
             {"prefill": prefill})
        return

    head_key = ("gdn", args.pools) if ("gdn", args.pools) in res else next(iter(res))
    kind0 = head_key[0]
    NB = {"gdn": BYTES_GDN, "gdneager": BYTES_GDN, "gdnh4": BYTES_GDN, "gdnv1": BYTES_GDN,
          "gdnbf16io": BYTES_GDN_BF16IO,
          "kda": BYTES_KDA,
          "f32": BYTES_F32_GDN}
    nbytes0 = NB[kind0]
    head = rate(head_key, nbytes0)
    detail = {"device_warmup_s": res[head_key]["device_warmup_s"], "decode_split": args.decode_split,
              "timing": f"median of {reps} timed passes of {steps} steps each, every pass "
                        "bracketed by HIP events recorded behind an already-enqueued untimed "
                        "pass; min and max beside each figure"}
    for key in res:
        nb = NB[key[0]]
        detail[f"{key[0]}_pools{key[1]}"] = rate(key, nb)
    if ("gdn", 1) in res and ("f32", 1) in res:
        detail["speedup_vs_fp32_state"] = res[("f32", 1)]["per_step"] / res[("gdn", 1)]["per_step"]
    if paged:
        detail["paged"] = paged
    if sweep:
        detail["sweep"] = sweep
    if prefill:
        detail["prefill"] = prefill
    if select:
        detail["select"] = select
    if codec_cmp:
        detail["codec_comparison"] = codec_cmp
    if window_res:
        detail["window"] = window_res
    if kda_cpu:
        detail["kda_cpu_oracle"] = kda_cpu
    if kda_window:
        detail["kda_window"] = kda_window
    if copy_ref and ("gdn", args.pools) in res:
        dec = rate(("gdn", args.pools), BYTES_GDN)
        detail["copy_reference"] = {
            "what": "torch copy_ of the bytes of one GDN decode step (half read, half written), "
                    "two buffer pairs alternating",
            "us": copy_ref[0] * 1e6, "gbs": copy_ref[1],
            "decode_gbs_over_copy_gbs": dec["gbs"] / copy_ref[1]}
    prof = profile_from_trace()
    if prof is not None:
        detail["kernel_trace"] = prof

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inputs, "gdn" if kind0 != "kda" else "kda")
        cpu.update(host)
        if cpu_1t is not None:
            cpu["one_thread"] = {"value": cpu_1t["value"], "sample": cpu_1t["sample"]}
        log(f"[bench] cpu oracle: {cpu['value']:.3e} updates/s on {cpu['cores']} threads")

    traffic = traffic_from_profile(units) if kind0 == "gdn" else None
    out = {
        "metric": "state updates/s + achieved HBM GB/s (% of peak), GDN/KDA decode B=256 H=32 d=128",
        "value": head["updates_per_s"],
        "unit": "state updates/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": head["us_per_step"] / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": {"gdn": "gdn_decode_compressed_state",
                                "kda": "kda_decode_compressed_state",
                                "gdnv1": "gdn_decode_u8_hadamard_state",
                                "gdnbf16io": "gdn_decode_compressed_state_bf16_io",
                                "f32": "gdn_decode_fp32_state"}[kind0],
                   "batch": n, "heads": H, "d_k": 128, "d_v": 128,
                   "state_format": "16 FP16 + 112 INT8 key rows, FP32 absmax/127 scale per 32",
                   "slot_sets_rotated": args.pools if kind0 != "f32" else 1,
                   "graph": use_graph,
                   "bytes_per_update": nbytes0},
        "hbm_gbs": head["gbs"],
        "roofline": {"bound": "hbm", "achieved": head["gbs"], "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": head["frac_of_peak"],
                     "traffic": traffic},
        "cpu_baseline": cpu,
        "detail": detail,
        "kernel_digest": kernel_digest(),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
