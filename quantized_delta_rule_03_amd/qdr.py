"""Thin Python binding of libqdr (C ABI in include/qdr.h).

Argument marshalling only: every step of the decode path runs in the HIP kernels of
``libqdr.so``. PyTorch supplies device memory (``torch.empty``) and the current HIP
stream. There is no fallback: if the library is missing or a call fails, an
exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqdr.so")

QDR_OK = 0
QDR_EINVAL = -1
QDR_EUNSUPPORTED = -2
QDR_EALIGN = -3
QDR_EHIP = -4
GDN = 0
KDA = 1
RULE_STEP, RULE_KEYROW, RULE_TENSOR = 0, 1, 2  # scale rules (QDR_RULE_*)

SYMBOLS = ("qdr_assign_bits", "qdr_state_bytes", "qdr_init_state", "qdr_quantize_state",
           "qdr_decode_step", "qdr_decode_window", "qdr_decode_window_static", "qdr_decode_chunk",
           "qdr_dequantize_state",
           "qdr_damp_select", "qdr_damp_bytes", "qdr_damp_init", "qdr_damp_quantize", "qdr_damp_step",
           "qdr_damp_dequantize", "qdr_comp_quantize", "qdr_comp_chunk", "qdr_comp_window",
           "qdr_comp_dequantize", "qdr_probe_copy", "qdr_probe_clock", "qdr_probe_clock_trace",
           "qdr_probe_wall_rate",
           "qdr_probe_last_error", "qdr_last_error")


class QdrError(RuntimeError):
    def __init__(self, code: int, where: str, text: str):
        super().__init__(f"{where} failed with {code}: {text}")
        self.code = code


class DampDesc(ctypes.Structure):
    _fields_ = [("n_req", ctypes.c_int32), ("n_head", ctypes.c_int32),
                ("gate", ctypes.c_int32), ("sel", ctypes.c_void_p)]


class Desc(ctypes.Structure):
    _fields_ = [("n_req", ctypes.c_int32), ("n_head", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("gate", ctypes.c_int32),
                ("bits", ctypes.c_void_p), ("window", ctypes.c_int32), ("rule", ctypes.c_int32)]


_lib = None


def lib():
    """Load libqdr.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "quantized_delta_rule_03_amd/build.py (or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        P, i32 = ctypes.c_void_p, ctypes.c_int32
        D = ctypes.POINTER(Desc)
        DD = ctypes.POINTER(DampDesc)
        u64 = ctypes.c_uint64
        sz = ctypes.POINTER(ctypes.c_size_t)
        sigs = {
            "qdr_assign_bits": [i32, i32, i32, P, P],
            "qdr_state_bytes": [D, sz, sz, sz, sz],
            "qdr_init_state": [D, P, P, P, P, P],
            "qdr_quantize_state": [D, P, P, P, P, P, P],
            "qdr_decode_step": [D, P, P, P, P, P, P, P, P, P, P, P],
            "qdr_decode_window": [D, P, P, P, P, P, i32, P, P, P, P, P, P, P],
            "qdr_decode_window_static": [D, P, P, P, P, i32, P, P, P, P, P, P, P],
            "qdr_decode_chunk": [D, P, P, P, P, i32, P, P, P, P, P, P, P],
            "qdr_damp_select": [i32, i32, P, P],
            "qdr_damp_bytes": [DD, sz, sz, sz, sz],
            "qdr_damp_init": [DD, P, P, P, P, P],
            "qdr_damp_quantize": [DD, P, P, P, P, P, u64, u64, P],
            "qdr_damp_step": [DD, P, P, P, P, P, P, P, P, P, P, u64, u64, P],
            "qdr_damp_dequantize": [DD, P, P, P, P, P, P],
            "qdr_dequantize_state": [D, P, P, P, P, P, P],
            "qdr_comp_quantize": [D, P, P, P, P, i32, P, P, P, P],
            "qdr_comp_chunk": [D, P, P, P, P, i32, P, P, i32, P, P, P, P, P, P, P],
            "qdr_comp_window": [D, P, P, P, P, i32, P, P, P, i32, P, P, P, P, P, P, P],
            "qdr_comp_dequantize": [D, P, P, P, P, i32, P, P, P, P],
            "qdr_probe_copy": [P, P, ctypes.c_size_t, P],
            "qdr_probe_clock": [P, i32, i32, P],
            "qdr_probe_clock_trace": [P, i32, i32, P],
            "qdr_probe_wall_rate": [ctypes.POINTER(ctypes.c_double)],
        }
        for name, args in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.qdr_last_error.argtypes = []
        L.qdr_last_error.restype = ctypes.c_char_p
        L.qdr_probe_last_error.argtypes = []
        L.qdr_probe_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def last_error() -> str:
    return lib().qdr_last_error().decode()


def _check(rc: int, where: str):
    if rc != QDR_OK:
        raise QdrError(rc, where, last_error())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream or None


def assign_bits(gate: int, halflife: np.ndarray, dk: int = 128) -> np.ndarray:
    """Lifetime quartile bit map (host): GDN halflife [n_head], KDA [n_head, dk]."""
    hl = np.ascontiguousarray(halflife, np.float64)
    n_head = hl.shape[0]
    out = np.zeros((n_head, dk), np.uint8)
    _check(lib().qdr_assign_bits(gate, n_head, dk, hl.ctypes.data, out.ctypes.data),
           "qdr_assign_bits")
    return out


@dataclass
class Layout:
    """Descriptor plus the sizes libqdr reports for it."""
    n_req: int
    n_head: int
    gate: int
    bits: np.ndarray
    window: int = 0
    rule: int = RULE_STEP
    packed_bytes: int = 0
    scale_bytes: int = 0
    meta_bytes: int = 0
    window_bytes: int = 0
    _desc: Desc = field(default=None, repr=False)

    def __post_init__(self):
        self.bits = np.ascontiguousarray(self.bits, np.uint8).reshape(self.n_head, 128)
        self._desc = Desc(self.n_req, self.n_head, 128, 128, self.gate,
                          self.bits.ctypes.data, self.window, self.rule)
        s = [ctypes.c_size_t() for _ in range(4)]
        _check(lib().qdr_state_bytes(ctypes.byref(self._desc), *[ctypes.byref(x) for x in s]),
               "qdr_state_bytes")
        self.packed_bytes, self.scale_bytes, self.meta_bytes, self.window_bytes = (
            int(x.value) for x in s)

    @property
    def desc(self):
        return ctypes.byref(self._desc)

    @property
    def req_bytes(self):
        return self.packed_bytes // self.n_req if self.n_req else 0


def init_state(L: Layout, packed, row_scale, col_scale, meta, stream=None):
    _check(lib().qdr_init_state(L.desc, _ptr(packed), _ptr(row_scale), _ptr(col_scale),
                                _ptr(meta), _stream(stream)), "qdr_init_state")


def quantize_state(L: Layout, meta, S, packed, row_scale, col_scale, stream=None):
    _check(lib().qdr_quantize_state(L.desc, _ptr(meta), _ptr(S), _ptr(packed), _ptr(row_scale),
                                    _ptr(col_scale), _stream(stream)), "qdr_quantize_state")


def decode_step(L: Layout, meta, packed, row_scale, col_scale, q, k, v, a, b, o, stream=None):
    _check(lib().qdr_decode_step(L.desc, _ptr(meta), _ptr(packed), _ptr(row_scale),
                                 _ptr(col_scale), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                                 _ptr(o), _stream(stream)), "qdr_decode_step")


def decode_window(L: Layout, meta, packed, row_scale, col_scale, window_buf, t, q, k, v, a, b, o,
                  stream=None):
    _check(lib().qdr_decode_window(L.desc, _ptr(meta), _ptr(packed), _ptr(row_scale),
                                   _ptr(col_scale), _ptr(window_buf), int(t), _ptr(q), _ptr(k),
                                   _ptr(v), _ptr(a), _ptr(b), _ptr(o), _stream(stream)),
           "qdr_decode_window")


def decode_window_static(L: Layout, meta, packed, row_scale, col_scale, t, q, k, v, a, b, o,
                         stream=None):
    _check(lib().qdr_decode_window_static(L.desc, _ptr(meta), _ptr(packed), _ptr(row_scale),
                                          _ptr(col_scale), int(t), _ptr(q), _ptr(k), _ptr(v),
                                          _ptr(a), _ptr(b), _ptr(o), _stream(stream)),
           "qdr_decode_window_static")


def decode_chunk(L: Layout, meta, packed, row_scale, col_scale, T, q, k, v, a, b, o, stream=None):
    _check(lib().qdr_decode_chunk(L.desc, _ptr(meta), _ptr(packed), _ptr(row_scale),
                                  _ptr(col_scale), int(T), _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                                  _ptr(b), _ptr(o), _stream(stream)), "qdr_decode_chunk")


def dequantize_state(L: Layout, meta, packed, row_scale, col_scale, S_out, stream=None):
    _check(lib().qdr_dequantize_state(L.desc, _ptr(meta), _ptr(packed), _ptr(row_scale),
                                      _ptr(col_scale), _ptr(S_out), _stream(stream)),
           "qdr_dequantize_state")


TOK_EMPTY = 0xFFFF  # empty compensator-token slot
COMP_MAX = 64


def comp_quantize(L: Layout, meta, packed, row_scale, col_scale, m, tok_idx, tok_val, S,
                  stream=None):
    _check(lib().qdr_comp_quantize(L.desc, _ptr(meta), _ptr(packed), _ptr(row_scale),
                                   _ptr(col_scale), int(m), _ptr(tok_idx), _ptr(tok_val), _ptr(S),
                                   _stream(stream)), "qdr_comp_quantize")


def comp_chunk(L: Layout, meta, packed, row_scale, col_scale, m, tok_idx, tok_val, T, q, k, v,
               a, b, o, stream=None):
    _check(lib().qdr_comp_chunk(L.desc, _ptr(meta), _ptr(packed), _ptr(row_scale),
                                _ptr(col_scale), int(m), _ptr(tok_idx), _ptr(tok_val), int(T),
                                _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(o),
                                _stream(stream)), "qdr_comp_chunk")


def comp_window(L: Layout, meta, packed, row_scale, col_scale, m, tok_idx, tok_val, window_buf,
                t, q, k, v, a, b, o, stream=None):
    _check(lib().qdr_comp_window(L.desc, _ptr(meta), _ptr(packed), _ptr(row_scale),
                                 _ptr(col_scale), int(m), _ptr(tok_idx), _ptr(tok_val),
                                 _ptr(window_buf), int(t), _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                                 _ptr(b), _ptr(o), _stream(stream)), "qdr_comp_window")


def comp_dequantize(L: Layout, meta, packed, row_scale, col_scale, m, tok_idx, tok_val, S_out,
                    stream=None):
    _check(lib().qdr_comp_dequantize(L.desc, _ptr(meta), _ptr(packed), _ptr(row_scale),
                                     _ptr(col_scale), int(m), _ptr(tok_idx), _ptr(tok_val),
                                     _ptr(S_out), _stream(stream)), "qdr_comp_dequantize")


class StatePool:
    """Caller-owned device buffers of one layer's quantized state (torch allocations)."""

    def __init__(self, n_req: int, n_head: int, gate: int, bits: np.ndarray, window: int = 0,
                 device="cuda", rule: int = RULE_STEP):
        import torch

        self.layout = Layout(n_req, n_head, gate, bits, window, rule)
        L = self.layout
        self.device = torch.device(device)
        self.packed = torch.empty(max(L.packed_bytes, 16), dtype=torch.uint8, device=device)
        shape = (n_req, n_head, 128)
        self.row_scale = torch.empty(shape, dtype=torch.float32, device=device)
        self.col_scale = torch.empty(shape, dtype=torch.float32, device=device)
        self.meta = torch.empty(L.meta_bytes, dtype=torch.uint8, device=device)
        self.window_buf = (torch.empty(L.window_bytes, dtype=torch.uint8, device=device)
                           if L.window_bytes else None)
        init_state(L, self.packed, self.row_scale, self.col_scale, self.meta)

    def quantize(self, S, stream=None):
        quantize_state(self.layout, self.meta, S, self.packed, self.row_scale, self.col_scale,
                       stream)

    def step(self, q, k, v, a, b, o, stream=None):
        decode_step(self.layout, self.meta, self.packed, self.row_scale, self.col_scale,
                    q, k, v, a, b, o, stream)

    def window_token(self, t, q, k, v, a, b, o, stream=None):
        decode_window(self.layout, self.meta, self.packed, self.row_scale, self.col_scale,
                      self.window_buf, t, q, k, v, a, b, o, stream)

    def chunk(self, q, k, v, a, b, o, stream=None):
        """T tokens at once; inputs token-major [T, n_req, n_head, ...] (T = b.shape[0])."""
        decode_chunk(self.layout, self.meta, self.packed, self.row_scale, self.col_scale,
                     int(b.shape[0]), q, k, v, a, b, o, stream)

    def dequantize(self, S_out=None, stream=None):
        import torch

        if S_out is None:
            S_out = torch.empty((self.layout.n_req, self.layout.n_head, 128, 128),
                                dtype=torch.float32, device=self.device)
        dequantize_state(self.layout, self.meta, self.packed, self.row_scale, self.col_scale,
                         S_out, stream)
        return S_out

    def load_host(self, packed: np.ndarray, row_scale: np.ndarray, col_scale: np.ndarray):
        """Copy a host packed state (same layout) into the device buffers."""
        import torch

        n = self.layout.packed_bytes
        self.packed[:n].copy_(torch.from_numpy(np.ascontiguousarray(packed).reshape(-1)))
        self.row_scale.copy_(torch.from_numpy(np.ascontiguousarray(row_scale)))
        self.col_scale.copy_(torch.from_numpy(np.ascontiguousarray(col_scale)))

    def to_host(self):
        n = self.layout.packed_bytes
        return (self.packed[:n].cpu().numpy().reshape(self.layout.n_req, -1),
                self.row_scale.cpu().numpy(), self.col_scale.cpu().numpy())

    # compensator tokens: tok_idx (uint16 bits in an int16 tensor) and tok_val,
    # [n_req, n_head, m]; empty slots until the first comp_quantize / comp_chunk
    def comp_enable(self, m: int):
        import torch

        L = self.layout
        self.m = int(m)
        shape = (L.n_req, L.n_head, max(self.m, 1))
        self.tok_idx = torch.full(shape, -1, dtype=torch.int16, device=self.device)
        self.tok_val = torch.zeros(shape, dtype=torch.float32, device=self.device)

    def comp_quantize(self, S, m: int, stream=None):
        self.comp_enable(m)
        comp_quantize(self.layout, self.meta, self.packed, self.row_scale, self.col_scale,
                      self.m, self.tok_idx, self.tok_val, S, stream)

    def comp_chunk(self, q, k, v, a, b, o, stream=None):
        comp_chunk(self.layout, self.meta, self.packed, self.row_scale, self.col_scale, self.m,
                   self.tok_idx, self.tok_val, int(b.shape[0]), q, k, v, a, b, o, stream)

    def comp_window_token(self, t, q, k, v, a, b, o, stream=None):
        comp_window(self.layout, self.meta, self.packed, self.row_scale, self.col_scale, self.m,
                    self.tok_idx, self.tok_val, self.window_buf, t, q, k, v, a, b, o, stream)

    def comp_dequantize(self, S_out=None, stream=None):
        import torch

        if S_out is None:
            S_out = torch.empty((self.layout.n_req, self.layout.n_head, 128, 128),
                                dtype=torch.float32, device=self.device)
        comp_dequantize(self.layout, self.meta, self.packed, self.row_scale, self.col_scale,
                        self.m, self.tok_idx, self.tok_val, S_out, stream)
        return S_out

    def comp_load_host(self, tok_idx: np.ndarray, tok_val: np.ndarray):
        import torch

        self.comp_enable(tok_idx.shape[-1])
        if self.m:
            idx = np.ascontiguousarray(tok_idx, np.uint16).view(np.int16)
            self.tok_idx.copy_(torch.from_numpy(idx))
            self.tok_val.copy_(torch.from_numpy(np.ascontiguousarray(tok_val, np.float32)))

    def comp_to_host(self):
        m = self.m
        return (self.tok_idx.cpu().numpy().view(np.uint16)[..., :m],
                self.tok_val.cpu().numpy()[..., :m])


def damp_select(gate: int, halflife: np.ndarray, n_head: int) -> np.ndarray:
    """Binary16 channels of the DAMP-style variant (qdr_damp_select)."""
    hl = np.ascontiguousarray(halflife, np.float64)
    out = np.zeros((n_head, 128), np.uint8)
    _check(lib().qdr_damp_select(int(gate), int(n_head), hl.ctypes.data, out.ctypes.data),
           "qdr_damp_select")
    return out


class DampState:
    """Device buffers of the DAMP-style storage variant (torch allocations): half
    [n_unit][128][16] (binary16 bits as int16), codes [n_unit][128][112] int8, R
    [n_unit][112], meta [n_head][128]."""

    def __init__(self, n_req: int, n_head: int, gate: int, sel: np.ndarray, seed: int = 0,
                 device="cuda"):
        import torch

        self.n_req, self.n_head, self.gate, self.seed = n_req, n_head, gate, int(seed)
        self.sel = np.ascontiguousarray(sel, np.uint8).reshape(n_head, 128)
        self._desc = DampDesc(n_req, n_head, gate, self.sel.ctypes.data)
        s = [ctypes.c_size_t() for _ in range(4)]
        _check(lib().qdr_damp_bytes(ctypes.byref(self._desc), *[ctypes.byref(x) for x in s]),
               "qdr_damp_bytes")
        n_unit = n_req * n_head
        self.device = torch.device(device)
        self.half = torch.empty((n_unit, 128, 16), dtype=torch.int16, device=device)
        self.codes = torch.empty((n_unit, 128, 112), dtype=torch.int8, device=device)
        self.R = torch.empty((n_unit, 112), dtype=torch.float32, device=device)
        self.meta = torch.empty(max(int(s[3].value), 16), dtype=torch.uint8, device=device)
        _check(lib().qdr_damp_init(ctypes.byref(self._desc), _ptr(self.meta), _ptr(self.half),
                                   _ptr(self.codes), _ptr(self.R), _stream(None)),
               "qdr_damp_init")

    def quantize(self, S, step: int = 0, stream=None):
        _check(lib().qdr_damp_quantize(ctypes.byref(self._desc), _ptr(self.meta), _ptr(S),
                                       _ptr(self.half), _ptr(self.codes), _ptr(self.R),
                                       self.seed, int(step), _stream(stream)),
               "qdr_damp_quantize")

    def step(self, q, k, v, a, b, o, step: int, stream=None):
        _check(lib().qdr_damp_step(ctypes.byref(self._desc), _ptr(self.meta), _ptr(self.half),
                                   _ptr(self.codes), _ptr(self.R), _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(a), _ptr(b), _ptr(o), self.seed, int(step),
                                   _stream(stream)), "qdr_damp_step")

    def dequantize(self, stream=None):
        import torch

        S = torch.empty((self.n_req, self.n_head, 128, 128), dtype=torch.float32,
                        device=self.device)
        _check(lib().qdr_damp_dequantize(ctypes.byref(self._desc), _ptr(self.meta),
                                         _ptr(self.half), _ptr(self.codes), _ptr(self.R),
                                         _ptr(S), _stream(stream)), "qdr_damp_dequantize")
        return S

    def load_host(self, half: np.ndarray, codes: np.ndarray, R: np.ndarray):
        import torch

        self.half.copy_(torch.from_numpy(np.ascontiguousarray(half).view(np.int16)))
        self.codes.copy_(torch.from_numpy(np.ascontiguousarray(codes)))
        self.R.copy_(torch.from_numpy(np.ascontiguousarray(R)))

    def to_host(self):
        return (self.half.cpu().numpy().view(np.uint16), self.codes.cpu().numpy(),
                self.R.cpu().numpy())


# ---- measurement helpers --------------------------------------------------------------

def probe_copy(src, dst, stream=None):
    """Streaming copy of src into dst (same byte size, device tensors) on the probe kernel."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("probe_copy: src and dst differ in size")
    rc = lib().qdr_probe_copy(_ptr(src), _ptr(dst), n, _stream(stream))
    if rc != QDR_OK:
        raise QdrError(rc, "qdr_probe_copy", lib().qdr_probe_last_error().decode())


def probe_clock(out, iters: int, stream=None):
    """Clock probe: out is a device int64 tensor [n_block, 4]."""
    rc = lib().qdr_probe_clock(_ptr(out), int(out.shape[0]), int(iters), _stream(stream))
    if rc != QDR_OK:
        raise QdrError(rc, "qdr_probe_clock", lib().qdr_probe_last_error().decode())


def probe_clock_trace(out, period: int, stream=None):
    """Clock trace: out is a device int64 tensor [n_sample, 2]; one sample every `period`
    ticks of the constant-rate counter."""
    rc = lib().qdr_probe_clock_trace(_ptr(out), int(out.shape[0]), int(period), _stream(stream))
    if rc:
        raise QdrError(rc, "qdr_probe_clock_trace", lib().qdr_probe_last_error().decode())


def probe_wall_rate() -> float:
    hz = ctypes.c_double()
    rc = lib().qdr_probe_wall_rate(ctypes.byref(hz))
    if rc != QDR_OK:
        raise QdrError(rc, "qdr_probe_wall_rate", lib().qdr_probe_last_error().decode())
    return float(hz.value)
