"""CPU oracle for the compressed GDN/KDA recurrent-state decode update.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library (``quantized_recurrent_state_02_amd``) and imports
nothing from it.

The arithmetic lives in ``qrs_oracle.c`` (FP32 as the pages fix it, plus an
FP64 twin) and in ``model_f64.py`` (the model-space product form in FP64).
This module only marshals numpy arrays into the C library.

Sources: "DAMP: Decay-Aware Mixed-Precision Recurrent-State Quantization"
(arXiv 2608.27513, HTML) and the reading notes on its v2; the functions below
name the section or equation they follow.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

DK = 128
DV = 128
KHI = 16
KLO = DK - KHI
GRP = 32
NGRP = DV // GRP

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqrs_oracle.so")
_lib = None


def load():
    """Load (building first if needed) the oracle shared library."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _build

        _build.build_oracle()
    lib = ctypes.CDLL(LIB_PATH)
    p = ctypes.c_void_p
    i = ctypes.c_int
    i64 = ctypes.c_int64
    lib.orc_f32_to_f16.argtypes = [ctypes.c_float]
    lib.orc_f32_to_f16.restype = ctypes.c_uint16
    lib.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.orc_f16_to_f32.restype = ctypes.c_float
    lib.orc_f32_to_f16_array.argtypes = [p, p, i64]
    lib.orc_f16_to_f32_array.argtypes = [p, p, i64]
    lib.orc_quantize_group.argtypes = [p, i, p, p]
    lib.orc_store.argtypes = [p, p, p, i, p, p, p, i, p, i]
    lib.orc_dequant.argtypes = [p, p, p, i, p, p, p, i, p, i]
    lib.orc_i8_decode.argtypes = [p, p, p, i, p, p, p, i, i, p, p, p, p, p, p]
    lib.orc_f32_decode.argtypes = [p, i, p, p, p, i, i, p, p, p, p, p, p]
    lib.orc_f64_decode.argtypes = [p, i, p, p, p, i, i, p, p, p, p, p, p]
    lib.orc_i8_prefill.argtypes = [p, p, p, i, p, p, p, i, i, i, p, p, p, p, p, p, i]
    lib.orc_channel_error.argtypes = [p, i, i, p, p]
    lib.orc_hadamard32.argtypes = [p, p]
    lib.orc_quantize_group_u8.argtypes = [p, p, p, p]
    lib.orc_u8_store.argtypes = [p, p, p, i, p, p, p, i, p, i]
    lib.orc_u8_dequant.argtypes = [p, p, p, i, p, p, p, i, p, i]
    lib.orc_u8_decode.argtypes = [p, p, p, i, p, p, p, i, i, p, p, p, p, p, p]
    lib.orc_u8_prefill.argtypes = [p, p, p, i, p, p, p, i, i, i, p, p, p, p, p, p, i]
    lib.orc_unit_bytes.argtypes = []
    lib.orc_unit_bytes.restype = i64
    lib.orc_max_threads.argtypes = []
    lib.orc_max_threads.restype = i
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


# ---------------------------------------------------------------------------
# FP16 and group codec
# ---------------------------------------------------------------------------

def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """IEEE binary16 round-to-nearest-even of FP32 values, as uint16 bits."""
    x = _f32(x)
    out = np.empty(x.shape, dtype=np.uint16)
    load().orc_f32_to_f16_array(_ptr(x), _ptr(out), x.size)
    return out


def f16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    load().orc_f16_to_f32_array(_ptr(h), _ptr(out), h.size)
    return out


def quantize_group(x: np.ndarray):
    """Symmetric INT8 quantization of one group sharing one FP32 scale.

    DAMP v2 reading notes, section 2.2, Eqs.(5)-(6): s = max|x|/127 and
    code = round(x/s).  Returns (codes int8, scale float32).
    """
    x = _f32(x).ravel()
    code = np.empty(x.size, dtype=np.int8)
    s = np.empty(1, dtype=np.float32)
    load().orc_quantize_group(_ptr(x), x.size, _ptr(code), _ptr(s))
    return code, s[0]


def hadamard32(x: np.ndarray) -> np.ndarray:
    """Normalized block-32 Hadamard transform of the last axis (length 32) of
    x: y = H x / sqrt(32), H Sylvester order ([DAMP] HTML Appendix A.1,
    Table 3).  FP64 sums in index order, times RN64(2^-2.5), rounded to FP32."""
    x = _f32(x)
    flat = x.reshape(-1, GRP)
    out = np.empty_like(flat)
    lib = load()
    for r in range(flat.shape[0]):
        lib.orc_hadamard32(_ptr(flat[r]), _ptr(out[r]))
    return out.reshape(x.shape)


def quantize_group_u8(y: np.ndarray):
    """Asymmetric UINT8 codes of one transformed 32-value group with FP16
    scale and zero point (HTML section 3.2 Eq.(3), Appendix A.1).  Returns
    (codes uint8 [32], s16, z16) with s16, z16 the FP16 bit patterns."""
    y = _f32(y).ravel()
    assert y.size == GRP
    code = np.empty(GRP, dtype=np.uint8)
    sz = np.zeros(2, dtype=np.uint16)
    load().orc_quantize_group_u8(_ptr(y), _ptr(code), _ptr(sz[0:1]), _ptr(sz[1:2]))
    return code, sz[0], sz[1]


def max_threads() -> int:
    """OpenMP threads the oracle's loops over units use."""
    return int(load().orc_max_threads())


def unit_bytes() -> int:
    return int(load().orc_unit_bytes())


# ---------------------------------------------------------------------------
# Pools
# ---------------------------------------------------------------------------

class OraclePool:
    """Oracle representation of a packed state pool.

    Unit u = slot * num_heads + head holds stored key rows 0..15 as FP16 bits
    (``hi``), rows 16..127 as INT8 codes (``lo``) and one FP32 scale per 32
    values of each INT8 row (``sc``) -- the DAMP packed representation
    (arXiv HTML, Appendix A.5, Eq.(17)) with the v2 quantizer.
    ``perm[h][i]`` is the model key channel stored in row i; ``c[h][j]`` the
    value-column smoothing scale (v2 notes, section 2.7, Eq.(17) of v2).
    """

    def __init__(self, num_slots, num_heads, perm=None, c=None):
        self.num_slots = num_slots
        self.num_heads = num_heads
        U = num_slots * num_heads
        self.hi = np.zeros((U, KHI, DV), dtype=np.uint16)
        self.lo = np.zeros((U, KLO, DV), dtype=np.int8)
        self.sc = np.zeros((U, KLO, NGRP), dtype=np.float32)
        self.perm = _i32(perm if perm is not None else np.tile(np.arange(DK), (num_heads, 1)))
        self.c = _f32(c if c is not None else np.ones((num_heads, DV)))

    def copy(self):
        o = OraclePool.__new__(OraclePool)
        o.num_slots, o.num_heads = self.num_slots, self.num_heads
        o.hi, o.lo, o.sc = self.hi.copy(), self.lo.copy(), self.sc.copy()
        o.perm, o.c = self.perm.copy(), self.c.copy()
        return o

    def store(self, slots, S, space=0):
        """Encode states S [n][H][128][128]; space 0 = model, 1 = stored."""
        slots = _i32(slots)
        S = _f32(S)
        load().orc_store(_ptr(self.hi), _ptr(self.lo), _ptr(self.sc), self.num_heads,
                         _ptr(self.perm), _ptr(self.c), _ptr(slots), slots.size, _ptr(S), space)

    def dequant(self, slots, space=0):
        slots = _i32(slots)
        out = np.empty((slots.size, self.num_heads, DK, DV), dtype=np.float32)
        load().orc_dequant(_ptr(self.hi), _ptr(self.lo), _ptr(self.sc), self.num_heads,
                           _ptr(self.perm), _ptr(self.c), _ptr(slots), slots.size, _ptr(out),
                           space)
        return out

    def decode_step(self, slots, q, k, v, gate, beta, kind):
        """One compressed decode step (kind 0 = GDN with alpha [n][H],
        kind 1 = KDA with log-decay g [n][H][128], kind 2 = KDA with the decay
        factors exp(g) given [n][H][128]); returns o [n][H][128]."""
        slots = _i32(slots)
        q, k, v, gate, beta = (_f32(a) for a in (q, k, v, gate, beta))
        o = np.empty((slots.size, self.num_heads, DV), dtype=np.float32)
        load().orc_i8_decode(_ptr(self.hi), _ptr(self.lo), _ptr(self.sc), self.num_heads,
                             _ptr(self.perm), _ptr(self.c), _ptr(slots), slots.size, kind,
                             _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), _ptr(o))
        return o

    def prefill(self, slots, q, k, v, alpha, beta, chunk, init_from_pool):
        """Chunked prefill with GDN gating; q,k,v [n][T][H][128]."""
        slots = _i32(slots)
        q, k, v, alpha, beta = (_f32(a) for a in (q, k, v, alpha, beta))
        n, T = q.shape[0], q.shape[1]
        o = np.empty_like(q)
        load().orc_i8_prefill(_ptr(self.hi), _ptr(self.lo), _ptr(self.sc), self.num_heads,
                              _ptr(self.perm), _ptr(self.c), _ptr(slots), n, T, chunk,
                              _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(o),
                              int(init_from_pool))
        return o


class OracleDensePool:
    """Uncompressed state pool in stored coordinates, FP32 or FP64
    (compression disabled)."""

    def __init__(self, num_slots, num_heads, perm=None, c=None, dtype=np.float32):
        self.num_slots = num_slots
        self.num_heads = num_heads
        self.dtype = np.dtype(dtype)
        self.T = np.zeros((num_slots * num_heads, DK, DV), dtype=self.dtype)
        self.perm = _i32(perm if perm is not None else np.tile(np.arange(DK), (num_heads, 1)))
        self.c = _f32(c if c is not None else np.ones((num_heads, DV)))

    def set_model(self, slots, S):
        """Place model-space states S [n][H][128][128] (T = P_K S D_c^{-1})."""
        for b, s in enumerate(np.asarray(slots)):
            for h in range(self.num_heads):
                Tm = np.asarray(S[b, h], dtype=np.float64 if self.dtype == np.float64 else np.float32)
                Tm = Tm[self.perm[h], :] / self.c[h][None, :].astype(Tm.dtype)
                self.T[s * self.num_heads + h] = Tm

    def get_model(self, slots):
        out = np.empty((len(slots), self.num_heads, DK, DV), dtype=self.dtype)
        for b, s in enumerate(np.asarray(slots)):
            for h in range(self.num_heads):
                Tm = self.T[s * self.num_heads + h] * self.c[h][None, :].astype(self.dtype)
                out[b, h][self.perm[h], :] = Tm
        return out

    def decode_step(self, slots, q, k, v, gate, beta, kind):
        slots = _i32(slots)
        q, k, v, gate, beta = (_f32(a) for a in (q, k, v, gate, beta))
        o = np.empty((slots.size, self.num_heads, DV), dtype=self.dtype)
        fn = load().orc_f64_decode if self.dtype == np.float64 else load().orc_f32_decode
        fn(_ptr(self.T), self.num_heads, _ptr(self.perm), _ptr(self.c), _ptr(slots),
           slots.size, kind, _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), _ptr(o))
        return o


class OracleU8Pool:
    """Packed pool with the first revision's low tier: stored key rows 0..15
    as FP16 bits (``hi``), rows 16..127 as UINT8 codes of the normalized
    block-32 Hadamard transform of each 32-value group (``lo``) with an FP16
    scale and zero point per group (``meta`` [U][112][4][2]: s, z) -- the
    INT8+Hadamard format of [DAMP] HTML section 3.2 Eq.(3), Appendix A.1
    (Table 3) in the packed layout of Appendix A.5 Eq.(17).  Same
    coordinates, permutation and smoothing as OraclePool."""

    def __init__(self, num_slots, num_heads, perm=None, c=None):
        self.num_slots = num_slots
        self.num_heads = num_heads
        U = num_slots * num_heads
        self.hi = np.zeros((U, KHI, DV), dtype=np.uint16)
        self.lo = np.zeros((U, KLO, DV), dtype=np.uint8)
        self.meta = np.zeros((U, KLO, NGRP, 2), dtype=np.uint16)
        self.perm = _i32(perm if perm is not None else np.tile(np.arange(DK), (num_heads, 1)))
        self.c = _f32(c if c is not None else np.ones((num_heads, DV)))

    def store(self, slots, S, space=0):
        slots = _i32(slots)
        S = _f32(S)
        load().orc_u8_store(_ptr(self.hi), _ptr(self.lo), _ptr(self.meta), self.num_heads,
                            _ptr(self.perm), _ptr(self.c), _ptr(slots), slots.size, _ptr(S), space)

    def dequant(self, slots, space=0):
        slots = _i32(slots)
        out = np.empty((slots.size, self.num_heads, DK, DV), dtype=np.float32)
        load().orc_u8_dequant(_ptr(self.hi), _ptr(self.lo), _ptr(self.meta), self.num_heads,
                              _ptr(self.perm), _ptr(self.c), _ptr(slots), slots.size, _ptr(out),
                              space)
        return out

    def decode_step(self, slots, q, k, v, gate, beta, kind):
        slots = _i32(slots)
        q, k, v, gate, beta = (_f32(a) for a in (q, k, v, gate, beta))
        o = np.empty((slots.size, self.num_heads, DV), dtype=np.float32)
        load().orc_u8_decode(_ptr(self.hi), _ptr(self.lo), _ptr(self.meta), self.num_heads,
                             _ptr(self.perm), _ptr(self.c), _ptr(slots), slots.size, kind,
                             _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), _ptr(o))
        return o

    def prefill(self, slots, q, k, v, alpha, beta, chunk, init_from_pool):
        """Chunked prefill with GDN gating on this tier; q,k,v [n][T][H][128]."""
        slots = _i32(slots)
        q, k, v, alpha, beta = (_f32(a) for a in (q, k, v, alpha, beta))
        n, T = q.shape[0], q.shape[1]
        o = np.empty_like(q)
        load().orc_u8_prefill(_ptr(self.hi), _ptr(self.lo), _ptr(self.meta), self.num_heads,
                              _ptr(self.perm), _ptr(self.c), _ptr(slots), n, T, chunk,
                              _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(o),
                              int(init_from_pool))
        return o


def decay_f16(g: np.ndarray) -> np.ndarray:
    """KDA decay factors of a per-window record: exp(g) in FP64, rounded once
    to the nearest FP16 (ties to even), as FP32 values.  numpy's float64 ->
    float16 conversion rounds directly from the double (pinned in
    tests/test_oracle_window.py against exact rational rounding)."""
    return np.exp(np.asarray(g, dtype=np.float64)).astype(np.float16).astype(np.float32)


class OracleWindowPool:
    """Per-window quantization on the packed pool ("LeapQuant: Efficient Linear
    Attention with Accurate Recurrent State Quantization", section 3.2 and
    Figure 2; memory figures of section 4.3).

    The stored (quantized) state of a slot is held fixed for a window of
    ``window`` tokens.  Every token of the window is recorded as an FP16
    update: k and v rounded to FP16 and, for KDA, the decay factors exp(g)
    rounded to FP16 (exp taken in FP64, rounded once to the nearest FP16,
    ties to even); beta and GDN's alpha stay FP32.  Each output is that of
    the FP32 recurrence started from the dequantized window-start state and
    run through the window's records up to and including the current token,
    read out with the current q.  The token that completes the window stores
    the resulting FP32 state back into the pool (requantized), which starts
    the next window.  ``pos[b]`` is the index of this token in slot b's
    window; calls must visit positions 0, 1, ..., window - 1 in order.
    Window 1 is the per-step method of OraclePool with FP16-rounded k and v.
    """

    def __init__(self, num_slots, num_heads, perm=None, c=None, window=16):
        self.pool = OraclePool(num_slots, num_heads, perm, c)
        self.window = window
        self.num_heads = num_heads
        self.records = {}

    def store(self, slots, S, space=0):
        self.pool.store(slots, S, space)
        for s in np.asarray(slots).tolist():
            self.records[s] = []

    def step(self, slots, pos, q, k, v, gate, beta, kind):
        H = self.num_heads
        q, k, v, gate, beta = (_f32(a) for a in (q, k, v, gate, beta))
        out = np.empty((len(slots), H, DV), dtype=np.float32)
        for b, s in enumerate(np.asarray(slots).tolist()):
            recs = self.records.setdefault(s, [])
            assert len(recs) == int(pos[b]), "window positions must advance one token at a time"
            k16 = f16_bits_to_f32(f32_to_f16_bits(k[b]))
            v16 = f16_bits_to_f32(f32_to_f16_bits(v[b]))
            recs.append((k16, v16, decay_f16(gate[b]) if kind == 1 else gate[b].copy(),
                         beta[b].copy()))
            dense = OracleDensePool(1, H, self.pool.perm, self.pool.c)
            dense.T[:] = self.pool.dequant([s], space=1)[0]
            rkind = 2 if kind == 1 else kind    # KDA records hold the decay factors
            for kk, vv, gg, bb in recs:
                o = dense.decode_step([0], q[b:b + 1], kk[None], vv[None], gg[None], bb[None], rkind)
            out[b] = o[0]
            if len(recs) == self.window:
                self.pool.store([s], dense.T.reshape(1, H, DK, DV), space=1)
                self.records[s] = []
        return out
