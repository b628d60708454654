"""Helpers shared by the GPU parity tests: run the HIP path and the oracle on
the same seeded inputs and compare them.

Tolerances (derived from the arithmetic; the oracle is FP32 with sequential
sums, the GPU FP32 with FMAs and a tree of partial sums):

* Encoding identical FP32 inputs: codes, scales and FP16 bits are identical.
* One decode step from states that already differ by D (GPU - oracle,
  dequantized, stored space): the pre-requantization values differ by at most
      dx[i,j] = lam_i |D_ij| + |k_i| beta sum_m |k_m| lam_m |D_mj| + eps_ij
  with eps_ij = 2^-20 (lam_i |That_ij| + |k_i| beta (|v'_j| + 130 sum_m |k_m|
  lam_m |That_mj|)) covering FP32 rounding of either side.  Requantization
  moves each side by at most half its step (s/2 on INT8 rows, half an FP16 ulp
  on FP16 rows), so after the step
      |D'_ij| <= dx_ij + max(s_gpu, s_orc)        (INT8 rows)
      |D'_ij| <= dx_ij + ulp16(max(|a|, |b|))     (FP16 rows).
  The readout differs by at most c_j sum_i |q_i| dx_ij plus 2^-20 c_j 130
  sum_i |q_i| |T_ij|.
* The bar of one quantization step per stored element after N steps is
  checked on the final state: strictly on INT8 rows; on FP16 rows one FP16
  ulp plus the coupling of the last step's INT8 differences through the
  rank-1 write (see north_star_step_ok).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from quantized_recurrent_state_02_amd import binding, inputs

DK = DV = 128


def ulp16(x):
    """Spacing of FP16 numbers at |x| (subnormal spacing below 2^-14)."""
    a = np.maximum(np.abs(x), 2.0 ** -14)
    e = np.floor(np.log2(a))
    return 2.0 ** (e - 10)


def split_gpu(pool: binding.StatePool, slots) -> tuple:
    """Packed bytes of all heads of the given slots -> (hi, lo, sc)."""
    H = pool.num_heads
    raw = pool.units().view(pool.num_slots, H, pool.unit_bytes)[
        torch.as_tensor(np.asarray(slots), dtype=torch.long, device=pool.mem.device)]
    raw = raw.reshape(-1, pool.unit_bytes).cpu().numpy()
    if pool.fmt == binding.FMT_U8H16:
        return binding.split_units_u8h(raw)
    return binding.split_units(raw)


def oracle_units(opool, slots):
    H = opool.num_heads
    idx = (np.asarray(slots)[:, None] * H + np.arange(H)[None, :]).ravel()
    if isinstance(opool, oracle.OracleU8Pool):
        return opool.hi[idx], opool.lo[idx], opool.meta[idx]
    return opool.hi[idx], opool.lo[idx], opool.sc[idx]


def dequant_units(hi, lo, sc):
    """Dequantized stored-space states from split units (numpy, FP32 ops
    identical to the format definition: f32(fp16) and s * code)."""
    U = hi.shape[0]
    T = np.empty((U, DK, DV), dtype=np.float32)
    T[:, :16] = hi.view(np.float16).astype(np.float32)
    T[:, 16:] = np.repeat(sc, 32, axis=2) * lo.astype(np.float32)
    return T


def assert_units_equal(g, o, what=""):
    gh, gl, gs = g
    oh, ol, os_ = o
    assert np.array_equal(gh, oh), f"{what}: FP16 rows differ at {np.argwhere(gh != oh)[:4]}"
    assert np.array_equal(gl, ol), f"{what}: codes differ at {np.argwhere(gl != ol)[:4]}"
    assert np.array_equal(gs.view(np.uint8), os_.view(np.uint8)), f"{what}: scales differ"


class StepBound:
    """Per-step derived tolerance for compressed decode (see module doc)."""

    def __init__(self, perm, c, kind):
        self.perm = perm
        self.c = c.astype(np.float64)
        self.kind = kind

    def operands(self, d, b, h, gate):
        p = self.perm[h]
        k = d["k"][b, h].astype(np.float64)[p]
        q = d["q"][b, h].astype(np.float64)[p]
        if self.kind == "gdn":
            lam = np.full(DK, float(gate[b, h]))
        else:
            lam = np.exp(gate[b, h].astype(np.float64))[p]
        vp = d["v"][b, h].astype(np.float64) / self.c[h]
        return k, q, lam, vp, float(d["beta"][b, h])

    def pre_bound(self, D, That, k, lam, vp, beta):
        """Bound on |x_gpu - x_orc| before requantization, [DK][DV]."""
        aD = np.abs(D)
        prop = lam[:, None] * aD + np.abs(k)[:, None] * beta * (np.abs(k) * lam) @ aD
        mag = np.abs(k) * lam @ np.abs(That)
        eps = 2.0 ** -20 * (lam[:, None] * np.abs(That)
                            + np.abs(k)[:, None] * beta * (np.abs(vp) + 130 * mag)[None, :])
        return prop + eps


def north_star_step_ok(Tg, To, sg, so, coupling=None):
    """One quantization step per stored element.

    INT8 rows: the two codes differ by at most one step.  With scales s_g and
    s_o (equal unless the group maxima differ by rounding) and |code| <= 127,
    that is |T_gpu - T_orc| <= max(s_g, s_o) + 127 |s_g - s_o|, plus half an
    FP32 ulp per side for the rounding of s * code.
    FP16 rows: one FP16 ulp of the larger magnitude, plus ``coupling`` (the
    pre-requantization difference bound of the last step, [..., 16, 128]):
    INT8 codes of two correct implementations may differ by one step, and
    every such difference reaches all rows through the rank-1 write
    k' (beta delta)^T, so an FP16 row cannot be held to one ulp alone.
    Returns (ok_lo, ok_hi, ok_hi_one_ulp, |difference|).
    """
    d = np.abs(Tg.astype(np.float64) - To.astype(np.float64))
    sg64, so64 = sg.astype(np.float64), so.astype(np.float64)
    step = np.repeat(np.maximum(sg64, so64) + 127.0 * np.abs(sg64 - so64), 32, axis=-1)
    # each dequantized value is s * code rounded to FP32: half an ulp per side
    rnd = 0.5 * (np.spacing(np.abs(Tg[..., 16:, :]).astype(np.float32)).astype(np.float64)
                 + np.spacing(np.abs(To[..., 16:, :]).astype(np.float32)).astype(np.float64))
    ok_lo = d[..., 16:, :] <= step + rnd
    u16 = ulp16(np.maximum(np.abs(Tg[..., :16, :]), np.abs(To[..., :16, :])))
    ok_hi_ulp = d[..., :16, :] <= u16
    ok_hi = ok_hi_ulp if coupling is None else d[..., :16, :] <= u16 + coupling
    return ok_lo, ok_hi, ok_hi_ulp, d


def describe_misses(ok_lo, Tg, To, sg, so, limit=4):
    """Text naming the INT8 elements that fail the one-step check."""
    out = []
    for u, i, j in np.argwhere(~ok_lo)[:limit]:
        g = j // 32
        out.append(f"unit {u} int8 row {i} col {j}: gpu {Tg[u, 16 + i, j]!r} orc {To[u, 16 + i, j]!r} "
                   f"s_gpu {sg[u, i, g]!r} s_orc {so[u, i, g]!r} "
                   f"codes {Tg[u, 16 + i, j] / sg[u, i, g] if sg[u, i, g] else 0:.3f} / "
                   f"{To[u, 16 + i, j] / so[u, i, g] if so[u, i, g] else 0:.3f}")
    return "; ".join(out)


def to_dev(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device="cuda", dtype=dtype)
