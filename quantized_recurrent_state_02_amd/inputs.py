"""Seeded synthetic inputs for the compressed-state decode workloads.

This module only draws random numbers and shapes them; it holds none of the
recurrence or codec arithmetic, imports numpy (and torch, lazily, for the
device-side draws of large workloads), and is the one module that both the
HIP path's tests/benchmark and the CPU oracle consume.

Every tensor comes from ``numpy.random.default_rng(SeedSequence([cfg,
tensor_id, step]))`` (PCG64), is drawn and transformed in float64 and cast to
float32 once.  Tensor ids: 0 initial state, 1 q, 2 k, 3 v, 4 alpha or g,
5 beta, 6 protected-channel choice, 7 smoothing scales c, 8 slot ids.

Workloads (decode shapes follow the pages' serving measurements: 32 heads,
d_k = d_v = 128, batches up to 256, and a 1-layer decode benchmark):
  0  GDN, n=1,   H=4,  64 steps, c = 1
  1  GDN, n=256, H=32, 256 steps, c log-uniform in [0.5, 2]
  2  KDA, n=256, H=32, 256 steps, c log-uniform in [0.5, 2]
  3  prefill, 8 sequences x 32 heads, 4096 tokens, chunk 64, GDN gating, c = 1
  4  paged: 4096 slots (GDN slots [0, 2048), KDA slots [2048, 4096)),
     1024 active (512 of each type), H=32, 1024 steps, heavy-tailed states
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

DK = 128
DV = 128
KHI = 16

T_STATE, T_Q, T_K, T_V, T_GATE, T_BETA, T_CHOICE, T_SMOOTH, T_SLOTS = range(9)


def rng(cfg: int, tensor_id: int, step: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg, tensor_id, step]))


@dataclass(frozen=True)
class Workload:
    cfg: int
    kind: str            # "gdn", "kda", "prefill" or "paged"
    n: int               # requests per step (active requests for "paged")
    heads: int
    steps: int           # decode steps, or tokens for prefill
    num_slots: int
    smooth: bool
    chunk: int = 0


WORKLOADS = {
    0: Workload(0, "gdn", 1, 4, 64, 1, False),
    1: Workload(1, "gdn", 256, 32, 256, 256, True),
    2: Workload(2, "kda", 256, 32, 256, 256, True),
    3: Workload(3, "prefill", 8, 32, 4096, 8, False, chunk=64),
    4: Workload(4, "paged", 1024, 32, 1024, 4096, True),
}


def _softplus(x):
    return np.logaddexp(0.0, x)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _l2_normalise(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def protected_perm(cfg: int, heads: int) -> np.ndarray:
    """Per-head key-row permutation, int32 [H][128].

    The 16 protected channels of a head are the first 16 entries of a seeded
    random permutation (no calibration); stored row order lists them
    ascending, then the other 112 ascending (a stable partition).
    """
    r = rng(cfg, T_CHOICE)
    out = np.empty((heads, DK), dtype=np.int32)
    for h in range(heads):
        chosen = np.sort(r.permutation(DK)[:KHI])
        rest = np.setdiff1d(np.arange(DK), chosen)
        out[h] = np.concatenate([chosen, rest])
    return out


def smoothing(cfg: int, heads: int, enabled: bool) -> np.ndarray:
    """Per-head value-column smoothing scales c > 0, float32 [H][128]:
    exp(U(ln 0.5, ln 2)) when enabled, else ones."""
    if not enabled:
        return np.ones((heads, DV), dtype=np.float32)
    r = rng(cfg, T_SMOOTH)
    return np.exp(r.uniform(np.log(0.5), np.log(2.0), size=(heads, DV))).astype(np.float32)


def initial_state(cfg: int, n: int, heads: int, perm: np.ndarray | None = None,
                  heavy_tailed: bool = False, first: int = 0) -> np.ndarray:
    """Model-space initial states, float32 [n][H][128][128].

    Default: N(0, 0.1) with 2 seeded outlier rows and 2 outlier columns per
    head multiplied by 20 (intersections by 400).
    heavy_tailed: 0.1 * Student-t(3) with 4 outlier rows x20 placed in the
    head's first four protected (FP16) channels ``perm[h][0:4]``.
    ``first`` offsets the request index so a subset [first, first+n) of a
    larger batch can be drawn identically (one generator per request).
    """
    out = np.empty((n, heads, DK, DV), dtype=np.float32)
    for b in range(n):
        r = rng(cfg, T_STATE, first + b)
        if heavy_tailed:
            S = 0.1 * r.standard_t(3.0, size=(heads, DK, DV))
            for h in range(heads):
                S[h, perm[h, :4], :] *= 20.0
        else:
            S = r.normal(0.0, 0.1, size=(heads, DK, DV))
            for h in range(heads):
                rows = r.choice(DK, 2, replace=False)
                cols = r.choice(DV, 2, replace=False)
                S[h, rows, :] *= 20.0
                S[h, :, cols] *= 20.0
        out[b] = S.astype(np.float32)
    return out


def step_inputs(cfg: int, step: int, n: int, heads: int, kind: str):
    """Per-step decode operands in model key order.

    q, k: N(0,1) then l2-normalised per head; v: N(0,1);
    beta = sigmoid(N(0,1)); GDN alpha = exp(-softplus(N(0,1) + 3)) per head;
    KDA g = -softplus(N(0,1) + 2) per key channel.
    Returns dict with float32 q, k, v [n][H][128], beta [n][H] and either
    alpha [n][H] ("gdn") or g [n][H][128] ("kda").
    """
    shp = (n, heads, DK)
    q = _l2_normalise(rng(cfg, T_Q, step).standard_normal(shp))
    k = _l2_normalise(rng(cfg, T_K, step).standard_normal(shp))
    v = rng(cfg, T_V, step).standard_normal((n, heads, DV))
    beta = _sigmoid(rng(cfg, T_BETA, step).standard_normal((n, heads)))
    out = dict(q=q.astype(np.float32), k=k.astype(np.float32), v=v.astype(np.float32),
               beta=beta.astype(np.float32))
    if kind == "gdn":
        a = np.exp(-_softplus(rng(cfg, T_GATE, step).standard_normal((n, heads)) + 3.0))
        out["alpha"] = a.astype(np.float32)
    elif kind == "kda":
        g = -_softplus(rng(cfg, T_GATE, step).standard_normal(shp) + 2.0)
        out["g"] = g.astype(np.float32)
    else:
        raise ValueError(kind)
    return out


def prefill_inputs(cfg: int, n: int, heads: int, tokens: int, first: int = 0):
    """Prefill operands [n][T][H][128] (q, k l2-normalised), alpha and beta
    [n][T][H], GDN gating.  One generator per sequence (``first`` offsets the
    sequence index so any subset draws identically)."""
    q = np.empty((n, tokens, heads, DK), dtype=np.float32)
    k = np.empty_like(q)
    v = np.empty((n, tokens, heads, DV), dtype=np.float32)
    alpha = np.empty((n, tokens, heads), dtype=np.float32)
    beta = np.empty_like(alpha)
    for b in range(n):
        s = first + b
        q[b] = _l2_normalise(rng(cfg, T_Q, s).standard_normal((tokens, heads, DK)))
        k[b] = _l2_normalise(rng(cfg, T_K, s).standard_normal((tokens, heads, DK)))
        v[b] = rng(cfg, T_V, s).standard_normal((tokens, heads, DV))
        alpha[b] = np.exp(-_softplus(rng(cfg, T_GATE, s).standard_normal((tokens, heads)) + 3.0))
        beta[b] = _sigmoid(rng(cfg, T_BETA, s).standard_normal((tokens, heads)))
    return dict(q=q, k=k, v=v, alpha=alpha, beta=beta)


def paged_slots(cfg: int = 4, num_slots: int = 4096, active: int = 1024):
    """Distinct random active slot ids for the paged workload: half drawn
    from the GDN-typed range [0, num_slots/2), half from the KDA-typed range
    [num_slots/2, num_slots).  Returns (gdn_slots, kda_slots) int32."""
    r = rng(cfg, T_SLOTS)
    half = num_slots // 2
    g = np.sort(r.choice(half, active // 2, replace=False)).astype(np.int32)
    k = (np.sort(r.choice(half, active // 2, replace=False)) + half).astype(np.int32)
    r.shuffle(g)
    r.shuffle(k)
    return g, k


# ---------------------------------------------------------------------------
# Device-side draws of the same recipes (large workloads).  Each tensor uses a
# torch generator on the device seeded from SeedSequence([cfg, tensor_id,
# step]); values are drawn in float64, transformed, and cast to float32 once.
# A caller that checks against the oracle copies the drawn arrays to the host.
# ---------------------------------------------------------------------------

def _torch_gen(cfg: int, tensor_id: int, step: int, device):
    import torch

    seed = int(np.random.SeedSequence([cfg, tensor_id, step]).generate_state(1, np.uint64)[0])
    g = torch.Generator(device=device)
    g.manual_seed(seed & ((1 << 63) - 1))
    return g


def initial_state_device(cfg: int, n: int, heads: int, perm: np.ndarray, first: int = 0,
                         device="cuda"):
    """Heavy-tailed model-space initial states on the device, float32
    [n][H][128][128]: 0.1 * Student-t(3) (drawn as Z / sqrt(chi2_3 / 3), the
    chi-square as a sum of three squared normals), with the head's first four
    protected channels perm[h][0:4] multiplied by 20.  One generator per
    request index first + b."""
    import torch

    out = torch.empty((n, heads, DK, DV), dtype=torch.float32, device=device)
    rows = torch.as_tensor(np.asarray(perm)[:, :4].astype(np.int64), device=device)
    for b in range(n):
        g = _torch_gen(cfg, T_STATE, first + b, device)
        z = torch.randn((heads, DK, DV), generator=g, dtype=torch.float64, device=device)
        c2 = torch.randn((3, heads, DK, DV), generator=g, dtype=torch.float64,
                         device=device).square().sum(0)
        S = 0.1 * z / torch.sqrt(c2 / 3.0)
        S[torch.arange(heads, device=device)[:, None], rows, :] *= 20.0
        out[b] = S.to(torch.float32)
    return out


def step_inputs_device(cfg: int, step: int, n: int, heads: int, kind: str, device="cuda"):
    """Per-step decode operands on the device, the recipe of step_inputs."""
    import torch

    def normal(tid, shape):
        return torch.randn(shape, generator=_torch_gen(cfg, tid, step, device),
                           dtype=torch.float64, device=device)

    shp = (n, heads, DK)
    q = normal(T_Q, shp)
    k = normal(T_K, shp)
    q = q / q.norm(dim=-1, keepdim=True)
    k = k / k.norm(dim=-1, keepdim=True)
    out = dict(q=q.float(), k=k.float(), v=normal(T_V, (n, heads, DV)).float(),
               beta=torch.sigmoid(normal(T_BETA, (n, heads))).float())
    if kind == "gdn":
        out["alpha"] = torch.exp(-torch.nn.functional.softplus(normal(T_GATE, (n, heads)) + 3.0)).float()
    elif kind == "kda":
        out["g"] = (-torch.nn.functional.softplus(normal(T_GATE, shp) + 2.0)).float()
    else:
        raise ValueError(kind)
    return out
