"""Thin ctypes binding over libqrs (include/qrs.h).

Argument marshalling only: shapes, dtypes and devices are checked, torch
tensors are turned into device pointers and the current torch stream is
passed as the hipStream_t.  Every step of the computation runs in the HIP
library; there is no fallback.  Importing torch first makes the library bind
to the HIP runtime torch already loaded.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqrs.so")

FMT_FP32 = 0
FMT_I8F16 = 1
FMT_U8H16 = 2
SPACE_MODEL = 0
SPACE_STORED = 1
OK = 0
DECODE_SPLIT_AUTO, DECODE_SPLIT_WHOLE, DECODE_SPLIT_HALVES = 0, 1, 2
DK = DV = 128
KHI = 16
GRP = 32
UNIT_BYTES = {FMT_FP32: 65536, FMT_I8F16: 20224, FMT_U8H16: 20224}
HI_OFFSET, LO_OFFSET, SCALE_OFFSET = 0, 4096, 18432

EXPORTED = (
    "qrs_state_pool_bytes", "qrs_create_state_pool", "qrs_destroy_state_pool", "qrs_pool_info",
    "qrs_store_state", "qrs_dequant_state", "qrs_gdn_decode_step", "qrs_kda_decode_step",
    "qrs_decode_step_ex", "qrs_decode_step_pair", "qrs_window_buffer_bytes",
    "qrs_window_decode_step",
    "qrs_chunked_prefill", "qrs_channel_error", "qrs_persistence_window",
    "qrs_persistence_geometric", "qrs_channel_scores", "qrs_select_protected_channels",
    "qrs_set_decode_split", "qrs_status_string",
)

_lib = None


class QrsError(RuntimeError):
    pass


def load(path: str = LIB_PATH):
    """Load libqrs.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise QrsError(f"{path} is missing: build it with __graft_entry__.build() "
                       "(the HIP library is required; there is no fallback)")
    lib = ctypes.CDLL(path)
    p, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.qrs_state_pool_bytes.argtypes = [i] * 7
    lib.qrs_state_pool_bytes.restype = sz
    lib.qrs_create_state_pool.argtypes = [i] * 7 + [p, sz, p, p, p, ctypes.POINTER(p)]
    lib.qrs_create_state_pool.restype = i
    lib.qrs_destroy_state_pool.argtypes = [p]
    lib.qrs_destroy_state_pool.restype = i
    lib.qrs_pool_info.argtypes = [p] + [ctypes.POINTER(i)] * 3 + [ctypes.POINTER(sz)] * 3
    lib.qrs_pool_info.restype = i
    lib.qrs_store_state.argtypes = [p, p, i, p, i, p]
    lib.qrs_store_state.restype = i
    lib.qrs_dequant_state.argtypes = [p, p, i, p, i, p]
    lib.qrs_dequant_state.restype = i
    for name in ("qrs_gdn_decode_step", "qrs_kda_decode_step"):
        fn = getattr(lib, name)
        fn.argtypes = [p, p, i, p, p, p, p, p, p, p]
        fn.restype = i
    lib.qrs_set_decode_split.argtypes = [i]
    lib.qrs_set_decode_split.restype = i
    lib.qrs_decode_step_ex.argtypes = [p, i, i, p, i, i, i, p, p, p, p, p, p, p]
    lib.qrs_decode_step_ex.restype = i
    lib.qrs_decode_step_pair.argtypes = [p, p, i] + [p] * 6 + [p, i] + [p] * 6 + [p]
    lib.qrs_decode_step_pair.restype = i
    lib.qrs_window_buffer_bytes.argtypes = [i, i, i, i]
    lib.qrs_window_buffer_bytes.restype = sz
    lib.qrs_window_decode_step.argtypes = [p, i, i, p, sz, p, p, i, p, p, p, p, p, p, p]
    lib.qrs_window_decode_step.restype = i
    lib.qrs_chunked_prefill.argtypes = [p, p, i, i, i, i, p, p, p, p, p, p, i, p]
    lib.qrs_chunked_prefill.restype = i
    lib.qrs_channel_error.argtypes = [i, i, p, p, p, p]
    lib.qrs_channel_error.restype = i
    lib.qrs_persistence_window.argtypes = [i, i, i, p, i, p, p, i, p, p]
    lib.qrs_persistence_window.restype = i
    lib.qrs_persistence_geometric.argtypes = [i, i, i, p, i, p, p, p, ctypes.c_double, p, p]
    lib.qrs_persistence_geometric.restype = i
    lib.qrs_channel_scores.argtypes = [i, i, p, p, p, p, p, p]
    lib.qrs_channel_scores.restype = i
    lib.qrs_select_protected_channels.argtypes = [i, p, i, p]
    lib.qrs_select_protected_channels.restype = i
    lib.qrs_status_string.argtypes = [i]
    lib.qrs_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int, what: str):
    if status != OK:
        msg = load().qrs_status_string(status).decode()
        raise QrsError(f"{what}: {msg} ({status})")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, dtype, shape, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise QrsError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise QrsError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise QrsError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise QrsError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def set_decode_split(mode: int) -> int:
    """Choose the INT8-tier decode kernel (qrs_set_decode_split): one
    workgroup per unit, two per unit (value-column halves), or by grid size
    (the default).  Returns the previous mode."""
    prev = load().qrs_set_decode_split(int(mode))
    if prev < 0:
        raise QrsError(f"qrs_set_decode_split({mode}): invalid mode")
    return prev


def pool_bytes(fmt: int, num_slots: int, num_heads: int) -> int:
    khi, grp = (0, 0) if fmt == FMT_FP32 else (KHI, GRP)
    return int(load().qrs_state_pool_bytes(fmt, num_slots, num_heads, DK, DV, khi, grp))


class StatePool:
    """A packed state pool in device memory owned by a torch uint8 tensor."""

    def __init__(self, fmt: int, num_slots: int, num_heads: int, perm=None, smooth=None,
                 device="cuda"):
        lib = load()
        self.fmt, self.num_slots, self.num_heads = fmt, num_slots, num_heads
        nbytes = pool_bytes(fmt, num_slots, num_heads)
        if nbytes == 0:
            raise QrsError("unsupported pool shape")
        self.mem = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self._perm = None if perm is None else np.ascontiguousarray(perm, dtype=np.int32)
        self._smooth = None if smooth is None else np.ascontiguousarray(smooth, dtype=np.float32)
        for arr, shape, name in ((self._perm, (num_heads, DK), "perm"),
                                 (self._smooth, (num_heads, DV), "smooth")):
            if arr is not None and arr.shape != shape:
                raise QrsError(f"{name} must have shape {shape}")
        handle = ctypes.c_void_p()
        khi, grp = (0, 0) if fmt == FMT_FP32 else (KHI, GRP)
        st = lib.qrs_create_state_pool(
            fmt, num_slots, num_heads, DK, DV, khi, grp, ctypes.c_void_p(self.mem.data_ptr()),
            nbytes,
            None if self._perm is None else self._perm.ctypes.data_as(ctypes.c_void_p),
            None if self._smooth is None else self._smooth.ctypes.data_as(ctypes.c_void_p),
            _stream(), ctypes.byref(handle))
        _check(st, "qrs_create_state_pool")
        self.handle = handle
        self.unit_bytes = UNIT_BYTES[fmt]

    def close(self):
        if getattr(self, "handle", None):
            load().qrs_destroy_state_pool(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- raw views (for checks and export) --
    def units(self) -> torch.Tensor:
        """The state region as uint8 [num_slots * H][unit_bytes] (a view)."""
        n = self.num_slots * self.num_heads * self.unit_bytes
        return self.mem[:n].view(self.num_slots * self.num_heads, self.unit_bytes)

    def store(self, slots: torch.Tensor, S: torch.Tensor, space: int = SPACE_MODEL):
        n = slots.numel()
        st = load().qrs_store_state(self.handle, _dev(slots, torch.int32, (n,), "slots"), n,
                                    _dev(S, torch.float32, (n, self.num_heads, DK, DV), "S"),
                                    space, _stream())
        _check(st, "qrs_store_state")

    def dequant(self, slots: torch.Tensor, space: int = SPACE_MODEL, out=None) -> torch.Tensor:
        n = slots.numel()
        if out is None:
            out = torch.empty((n, self.num_heads, DK, DV), dtype=torch.float32,
                              device=self.mem.device)
        st = load().qrs_dequant_state(self.handle, _dev(slots, torch.int32, (n,), "slots"), n,
                                      _dev(out, torch.float32, (n, self.num_heads, DK, DV), "out"),
                                      space, _stream())
        _check(st, "qrs_dequant_state")
        return out

    def _step(self, fn, name, slots, q, k, v, gate, gate_shape, beta, out):
        n, H = slots.numel(), self.num_heads
        if out is None:
            out = torch.empty((n, H, DV), dtype=torch.float32, device=self.mem.device)
        st = fn(self.handle, _dev(slots, torch.int32, (n,), "slots"), n,
                _dev(q, torch.float32, (n, H, DK), "q"), _dev(k, torch.float32, (n, H, DK), "k"),
                _dev(v, torch.float32, (n, H, DV), "v"), _dev(gate, torch.float32, gate_shape, "gate"),
                _dev(beta, torch.float32, (n, H), "beta"),
                _dev(out, torch.float32, (n, H, DV), "o"), _stream())
        _check(st, name)
        return out

    def gdn_step(self, slots, q, k, v, alpha, beta, out=None):
        n = slots.numel()
        return self._step(load().qrs_gdn_decode_step, "qrs_gdn_decode_step", slots, q, k, v,
                          alpha, (n, self.num_heads), beta, out)

    def prefill(self, slots, q, k, v, alpha, beta, chunk=64, init_from_pool=True, out=None):
        """Chunked prefill (GDN gating): q, k, v [n][T][H][128] float32 or
        bfloat16 (one dtype), alpha, beta float32 [n][T][H]; returns o float32
        [n][T][H][128]."""
        n = slots.numel()
        if q.dim() != 4:
            raise QrsError("q must be [n][T][H][128]")
        T, H = q.shape[1], self.num_heads
        dt = q.dtype
        if dt not in (torch.float32, torch.bfloat16):
            raise QrsError("q, k, v must be float32 or bfloat16")
        if out is None:
            out = torch.empty((n, T, H, DV), dtype=torch.float32, device=self.mem.device)
        st = load().qrs_chunked_prefill(
            self.handle, _dev(slots, torch.int32, (n,), "slots"), n, T, int(chunk),
            0 if dt == torch.float32 else 1,
            _dev(q, dt, (n, T, H, DK), "q"), _dev(k, dt, (n, T, H, DK), "k"),
            _dev(v, dt, (n, T, H, DV), "v"), _dev(alpha, torch.float32, (n, T, H), "alpha"),
            _dev(beta, torch.float32, (n, T, H), "beta"),
            _dev(out, torch.float32, (n, T, H, DV), "o"), int(bool(init_from_pool)), _stream())
        _check(st, "qrs_chunked_prefill")
        return out

    def step_ex(self, kind, slots, q, k, v, gate, beta, heads=None, out=None):
        """qrs_decode_step_ex: kind "gdn" or "kda"; q, k, v (and out) float32 or
        bfloat16 [n][H][128]; heads = (begin, count) or None for all."""
        n, H = slots.numel(), self.num_heads
        h0, hc = (0, H) if heads is None else (int(heads[0]), int(heads[1]))
        dt = q.dtype
        if dt not in (torch.float32, torch.bfloat16):
            raise QrsError("q, k, v must be float32 or bfloat16")
        if out is None:
            out = torch.full((n, H, DV), float("nan"), dtype=dt, device=self.mem.device)
        kid = {"gdn": 0, "kda": 1}[kind]
        gshape = (n, H) if kid == 0 else (n, H, DK)
        st = load().qrs_decode_step_ex(
            self.handle, kid, 0 if dt == torch.float32 else 1, _dev(slots, torch.int32, (n,), "slots"),
            n, h0, hc, _dev(q, dt, (n, H, DK), "q"), _dev(k, dt, (n, H, DK), "k"),
            _dev(v, dt, (n, H, DV), "v"), _dev(gate, torch.float32, gshape, "gate"),
            _dev(beta, torch.float32, (n, H), "beta"), _dev(out, dt, (n, H, DV), "o"), _stream())
        _check(st, "qrs_decode_step_ex")
        return out

    def window_buffer(self, kind: str, window: int) -> torch.Tensor:
        """A zeroed device update buffer for window_step (uint8)."""
        nb = int(load().qrs_window_buffer_bytes({"gdn": 0, "kda": 1}[kind], self.num_slots,
                                                self.num_heads, int(window)))
        if nb == 0:
            raise QrsError("invalid window buffer shape")
        return torch.zeros(nb, dtype=torch.uint8, device=self.mem.device)

    def window_step(self, kind, window, buffer, slots, pos, q, k, v, gate, beta, out=None):
        """qrs_window_decode_step: one token per slot at window positions pos
        (int32 [n]); q, k, v float32 [n][H][128]."""
        n, H = slots.numel(), self.num_heads
        kid = {"gdn": 0, "kda": 1}[kind]
        if out is None:
            out = torch.empty((n, H, DV), dtype=torch.float32, device=self.mem.device)
        if not (isinstance(buffer, torch.Tensor) and buffer.is_cuda and buffer.dtype == torch.uint8):
            raise QrsError("buffer must be a device uint8 tensor")
        gshape = (n, H) if kid == 0 else (n, H, DK)
        st = load().qrs_window_decode_step(
            self.handle, kid, int(window), ctypes.c_void_p(buffer.data_ptr()), buffer.numel(),
            _dev(slots, torch.int32, (n,), "slots"), _dev(pos, torch.int32, (n,), "pos"), n,
            _dev(q, torch.float32, (n, H, DK), "q"), _dev(k, torch.float32, (n, H, DK), "k"),
            _dev(v, torch.float32, (n, H, DV), "v"), _dev(gate, torch.float32, gshape, "gate"),
            _dev(beta, torch.float32, (n, H), "beta"), _dev(out, torch.float32, (n, H, DV), "o"),
            _stream())
        _check(st, "qrs_window_decode_step")
        return out

    def kda_step(self, slots, q, k, v, g, beta, out=None):
        n = slots.numel()
        return self._step(load().qrs_kda_decode_step, "qrs_kda_decode_step", slots, q, k, v, g,
                          (n, self.num_heads, DK), beta, out)

    def pair_step(self, gdn, kda, out_gdn=None, out_kda=None):
        """qrs_decode_step_pair: a GDN step and a KDA step on disjoint slots
        in one call.  gdn = (slots, q, k, v, alpha, beta), kda = (slots, q, k,
        v, g, beta), float32 [n][H][128] operands as for gdn_step / kda_step.
        Returns (o_gdn, o_kda)."""
        H = self.num_heads
        args, outs = [], []
        for grp, out, gshape_of, name in ((gdn, out_gdn, lambda n: (n, H), "gdn"),
                                          (kda, out_kda, lambda n: (n, H, DK), "kda")):
            slots, q, k, v, gate, beta = grp
            n = slots.numel()
            if out is None:
                out = torch.empty((n, H, DV), dtype=torch.float32, device=self.mem.device)
            if n == 0:
                args += [None, 0] + [None] * 6
            else:
                args += [_dev(slots, torch.int32, (n,), f"{name} slots"), n,
                         _dev(q, torch.float32, (n, H, DK), f"{name} q"),
                         _dev(k, torch.float32, (n, H, DK), f"{name} k"),
                         _dev(v, torch.float32, (n, H, DV), f"{name} v"),
                         _dev(gate, torch.float32, gshape_of(n), f"{name} gate"),
                         _dev(beta, torch.float32, (n, H), f"{name} beta"),
                         _dev(out, torch.float32, (n, H, DV), f"{name} o")]
            outs.append(out)
        st = load().qrs_decode_step_pair(self.handle, *args, _stream())
        _check(st, "qrs_decode_step_pair")
        return outs[0], outs[1]


def split_units(raw: np.ndarray):
    """Split packed I8F16 unit bytes [U][20224] into (hi uint16 [U][16][128],
    lo int8 [U][112][128], sc float32 [U][112][4]) per the layout in qrs.h."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    U = raw.shape[0]
    hi = raw[:, HI_OFFSET:LO_OFFSET].copy().view(np.uint16).reshape(U, KHI, DV)
    lo = raw[:, LO_OFFSET:SCALE_OFFSET].copy().view(np.int8).reshape(U, DK - KHI, DV)
    sc = raw[:, SCALE_OFFSET:].copy().view(np.float32).reshape(U, DK - KHI, DV // GRP)
    return hi, lo, sc


def split_units_u8h(raw: np.ndarray):
    """Split packed U8H16 unit bytes [U][20224] into (hi uint16 [U][16][128],
    codes uint8 [U][112][128], meta uint16 [U][112][4][2] = FP16 (s, z))."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    U = raw.shape[0]
    hi = raw[:, HI_OFFSET:LO_OFFSET].copy().view(np.uint16).reshape(U, KHI, DV)
    lo = raw[:, LO_OFFSET:SCALE_OFFSET].copy().reshape(U, DK - KHI, DV)
    meta = raw[:, SCALE_OFFSET:].copy().view(np.uint16).reshape(U, DK - KHI, DV // GRP, 2)
    return hi, lo, meta


# ---------------------------------------------------------------------------
# key-channel selection (argument marshalling for the qrs_channel_* calls)
# ---------------------------------------------------------------------------

def _opt(t, dtype, shape, name):
    return None if t is None else _dev(t, dtype, shape, name)


def channel_error(S: torch.Tensor, smooth: torch.Tensor | None = None, out=None) -> torch.Tensor:
    """qrs_channel_error: e [n][H][128] (float64) for calibration states
    S [n][H][128][128] (float32, model coordinates) and smoothing c [H][128]."""
    n, H = S.shape[0], S.shape[1]
    if out is None:
        out = torch.empty((n, H, DK), dtype=torch.float64, device=S.device)
    st = load().qrs_channel_error(n, H, _dev(S, torch.float32, (n, H, DK, DV), "S"),
                                  _opt(smooth, torch.float32, (H, DV), "smooth"),
                                  _dev(out, torch.float64, (n, H, DK), "e"), _stream())
    _check(st, "qrs_channel_error")
    return out


def persistence_window(a: torch.Tensor, sample_seq: torch.Tensor, sample_t: torch.Tensor,
                       horizon: int = 256, out=None) -> torch.Tensor:
    """qrs_persistence_window: W [n][H][128] (float64) from decays
    a [n_seq][T][H][128] (float32) at the sampled writes (int32 [n] each)."""
    n_seq, T, H = a.shape[0], a.shape[1], a.shape[2]
    n = sample_seq.numel()
    if out is None:
        out = torch.empty((n, H, DK), dtype=torch.float64, device=a.device)
    st = load().qrs_persistence_window(
        n_seq, T, H, _dev(a, torch.float32, (n_seq, T, H, DK), "a"), n,
        _dev(sample_seq, torch.int32, (n,), "sample_seq"),
        _dev(sample_t, torch.int32, (n,), "sample_t"), int(horizon),
        _dev(out, torch.float64, (n, H, DK), "W"), _stream())
    _check(st, "qrs_persistence_window")
    return out


def persistence_geometric(a: torch.Tensor, sample_seq: torch.Tensor, sample_t: torch.Tensor,
                          weight: torch.Tensor, tau: float = 1e-4, out=None) -> torch.Tensor:
    """qrs_persistence_geometric: P [H][128] (float64)."""
    n_seq, T, H = a.shape[0], a.shape[1], a.shape[2]
    n = sample_seq.numel()
    if out is None:
        out = torch.empty((H, DK), dtype=torch.float64, device=a.device)
    st = load().qrs_persistence_geometric(
        n_seq, T, H, _dev(a, torch.float32, (n_seq, T, H, DK), "a"), n,
        _dev(sample_seq, torch.int32, (n,), "sample_seq"),
        _dev(sample_t, torch.int32, (n,), "sample_t"),
        _dev(weight, torch.float64, (n,), "weight"), float(tau),
        _dev(out, torch.float64, (H, DK), "P"), _stream())
    _check(st, "qrs_persistence_geometric")
    return out


def channel_scores(e: torch.Tensor, weight: torch.Tensor, W: torch.Tensor | None = None,
                   P: torch.Tensor | None = None, out=None) -> torch.Tensor:
    """qrs_channel_scores: C [H][128] (float64); exactly one of W, P."""
    n, H = e.shape[0], e.shape[1]
    if out is None:
        out = torch.empty((H, DK), dtype=torch.float64, device=e.device)
    st = load().qrs_channel_scores(n, H, _dev(e, torch.float64, (n, H, DK), "e"),
                                   _opt(W, torch.float64, (n, H, DK), "W"),
                                   _opt(P, torch.float64, (H, DK), "P"),
                                   _dev(weight, torch.float64, (n,), "weight"),
                                   _dev(out, torch.float64, (H, DK), "C"), _stream())
    _check(st, "qrs_channel_scores")
    return out


def select_protected_channels(score, k_hi: int = KHI) -> np.ndarray:
    """qrs_select_protected_channels: perm int32 [H][128] (host) from scores
    [H][128]; the first k_hi entries of each head are its protected channels."""
    sc = np.ascontiguousarray(score.cpu().numpy() if isinstance(score, torch.Tensor) else score,
                              dtype=np.float64)
    H = sc.shape[0]
    perm = np.empty((H, DK), np.int32)
    st = load().qrs_select_protected_channels(H, sc.ctypes.data_as(ctypes.c_void_p), int(k_hi),
                                              perm.ctypes.data_as(ctypes.c_void_p))
    _check(st, "qrs_select_protected_channels")
    return perm
