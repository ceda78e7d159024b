"""Plain scalar CPU oracle for the quantized Delta-rule decode step.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product library
(``quantized_delta_rule_03_amd``) never imports it, and the two share no code.

The arithmetic lives in ``qdr_oracle.c`` (scalar C, fp32 state arithmetic with
fp64 dot products, built with ``-ffp-contract=off``); this module only builds and
loads it and marshals numpy arrays. See ``qdr_oracle.h`` for the contract and the
page citations.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qdr_oracle.c")
_LIB = os.path.join(_HERE, "libqdr_oracle.so")

GDN = 0
KDA = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no SIMD intrinsics, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = [
            "gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
            "-fPIC", "-shared", "-o", tmp, _SRC, "-lm",
        ]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f32 = ctypes.c_int, ctypes.c_long, ctypes.c_float
        u64 = ctypes.c_uint64
        sig = {
            "oref_assign_bits": (i32, [i32, i32, i32, P, P]),
            "oref_layout": (i64, [i32, i32, P, P, P]),
            "oref_pack": (i32, [i32, i32, P, P, P]),
            "oref_unpack": (i32, [i32, i32, P, P, P]),
            "oref_quantize": (None, [i32, i32, P, P, P, P, P]),
            "oref_quantize_rule": (None, [i32, i32, P, P, P, P, P, i32]),
            "oref_dequantize": (None, [i32, i32, P, P, P, P]),
            "oref_step": (None, [i32, i32, i32, P, P, P, P, P, P, P, P, f32, P, P]),
            "oref_step_rule": (None, [i32, i32, i32, P, P, P, P, P, P, P, P, f32, P, P, i32]),
            "oref_window": (None, [i32, i32, i32, P, P, P, P, i32, P, P, P, P, P, P, P]),
            "oref_recur_fp64": (None, [i32, i32, i32, P, P, P, P, P, f32, P]),
            "oref_request_bytes": (i64, [i32, i32, i32, P]),
            "oref_quantize_pool": (i32, [i32, i32, i32, i32, P, P, P, P, P]),
            "oref_quantize_pool_rule": (i32, [i32, i32, i32, i32, P, P, P, P, P, i32]),
            "oref_dequantize_pool": (i32, [i32, i32, i32, i32, P, P, P, P, P]),
            "oref_step_pool": (i32, [i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P, P,
                                     i64, i64]),
            "oref_step_pool_rule": (i32, [i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P,
                                          P, i64, i64, i32]),
            "oref_window_pool": (i32, [i32, i32, i32, i32, i32, P, P, P, P, i32, P, P, P, P,
                                       P, P, i64, i64]),
            "oref_comp_select": (None, [i32, i32, i32, P, P, P]),
            "oref_comp_quantize": (None, [i32, i32, P, P, i32, P, P, P, P, P]),
            "oref_comp_dequantize": (None, [i32, i32, P, P, P, i32, P, P, P]),
            "oref_comp_window": (None, [i32, i32, i32, P, P, P, P, i32, P, P, i32, P, P, P, P,
                                        P, P, P]),
            "oref_comp_quantize_pool": (i32, [i32, i32, i32, i32, P, P, i32, P, P, P, P, P]),
            "oref_comp_dequantize_pool": (i32, [i32, i32, i32, i32, P, P, P, P, i32, P, P, P]),
            "oref_comp_window_pool": (i32, [i32, i32, i32, i32, i32, P, P, P, P, i32, P, P, i32,
                                            P, P, P, P, P, P, i64, i64]),
            "oref_philox4x32_10": (None, [P, P, P]),
            "oref_philox4x32": (None, [P, P, ctypes.c_int, P]),
            "oref_f32_to_f16": (ctypes.c_uint16, [f32]),
            "oref_f16_to_f32": (f32, [ctypes.c_uint16]),
            "oref_damp_perm": (i32, [i32, P, P]),
            "oref_damp_quantize_pool": (i32, [i32, i32, i32, P, P, P, P, P, u64, u64]),
            "oref_damp_dequantize_pool": (i32, [i32, i32, i32, P, P, P, P, P]),
            "oref_damp_step_pool": (i32, [i32, i32, i32, i32, P, P, P, P, P, P, P, P, P, P,
                                          u64, u64, i64, i64]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(arr):
    return None if arr is None else arr.ctypes.data


def _c(arr, dtype):
    a = np.ascontiguousarray(arr, dtype=dtype)
    return a


# ---------------------------------------------------------------------------
# per-unit logical interface
# ---------------------------------------------------------------------------

def assign_bits(gate: int, halflife: np.ndarray, dk: int) -> np.ndarray:
    """Lifetime quartile bit map; GDN halflife [n_head], KDA halflife [n_head, dk]."""
    hl = _c(halflife, np.float64)
    n_head = hl.shape[0]
    out = np.zeros((n_head, dk), np.uint8)
    if lib().oref_assign_bits(gate, n_head, dk, _p(hl), _p(out)) != 0:
        raise ValueError("oref_assign_bits failed")
    return out


def layout(bits: np.ndarray, dv: int = 128):
    """(tile_bytes, perm[dk], seg_bits[dk/32]) for one head's bit map."""
    b = _c(bits, np.uint8)
    dk = b.shape[0]
    perm = np.zeros(dk, np.uint8)
    seg = np.zeros(max(dk // 32, 1), np.uint8)
    n = lib().oref_layout(dv, dk, _p(b), _p(perm), _p(seg))
    if n < 0:
        raise ValueError("bit map not representable in the packed format")
    return int(n), perm, seg


def pack(codes: np.ndarray, bits: np.ndarray) -> np.ndarray:
    c = _c(codes, np.int8)
    b = _c(bits, np.uint8)
    dv, dk = c.shape
    n, _, _ = layout(b, dv)
    tile = np.zeros(n, np.uint8)
    if lib().oref_pack(dv, dk, _p(b), _p(c), _p(tile)) != 0:
        raise ValueError("oref_pack failed")
    return tile


def unpack(tile: np.ndarray, bits: np.ndarray, dv: int = 128) -> np.ndarray:
    b = _c(bits, np.uint8)
    t = _c(tile, np.uint8)
    dk = b.shape[0]
    codes = np.zeros((dv, dk), np.int8)
    if lib().oref_unpack(dv, dk, _p(b), _p(t), _p(codes)) != 0:
        raise ValueError("oref_unpack failed")
    return codes


RULE_STEP, RULE_KEYROW, RULE_TENSOR = 0, 1, 2  # scale rules (see qdr_oracle.h)


def quantize(S: np.ndarray, bits: np.ndarray, rule: int = RULE_STEP):
    """fp32 state [dv, dk] -> (codes int8 [dv, dk], R [dk], c [dv])."""
    S = _c(S, np.float32)
    b = _c(bits, np.uint8)
    dv, dk = S.shape
    codes = np.zeros((dv, dk), np.int8)
    R = np.zeros(dk, np.float32)
    c = np.zeros(dv, np.float32)
    lib().oref_quantize_rule(dv, dk, _p(b), _p(S), _p(codes), _p(R), _p(c), int(rule))
    return codes, R, c


def dequantize(codes: np.ndarray, R: np.ndarray, c: np.ndarray) -> np.ndarray:
    codes = _c(codes, np.int8)
    R = _c(R, np.float32)
    c = _c(c, np.float32)
    dv, dk = codes.shape
    S = np.zeros((dv, dk), np.float32)
    lib().oref_dequantize(dv, dk, _p(codes), _p(R), _p(c), _p(S))
    return S


def step(codes, R, c, bits, gate, q, k, v, a, b, return_state=False, rule: int = RULE_STEP):
    """One decode step on one unit. Returns (codes, R, c, o[, S_new])."""
    codes = _c(codes, np.int8).copy()
    R = _c(R, np.float32).copy()
    c = _c(c, np.float32).copy()
    bb = _c(bits, np.uint8)
    dv, dk = codes.shape
    q, k = _c(q, np.float32), _c(k, np.float32)
    v = _c(v, np.float32)
    a = _c(np.atleast_1d(a), np.float32)
    o = np.zeros(dv, np.float32)
    S_new = np.zeros((dv, dk), np.float32) if return_state else None
    lib().oref_step_rule(dv, dk, gate, _p(bb), _p(codes), _p(R), _p(c), _p(q), _p(k), _p(v),
                         _p(a), float(b), _p(o), _p(S_new), int(rule))
    if return_state:
        return codes, R, c, o, S_new
    return codes, R, c, o


def window(codes, R, c, bits, gate, q, k, v, a, b, return_state=False):
    """One window (W = len(b) tokens) on one unit. Returns (codes, R, c, o[W, dv][, S])."""
    codes = _c(codes, np.int8).copy()
    R = _c(R, np.float32).copy()
    c = _c(c, np.float32).copy()
    bb = _c(bits, np.uint8)
    dv, dk = codes.shape
    q, k, v = _c(q, np.float32), _c(k, np.float32), _c(v, np.float32)
    a = _c(a, np.float32)
    b = _c(b, np.float32)
    W = b.shape[0]
    o = np.zeros((W, dv), np.float32)
    S_end = np.zeros((dv, dk), np.float32) if return_state else None
    lib().oref_window(dv, dk, gate, _p(bb), _p(codes), _p(R), _p(c), W, _p(q), _p(k),
                      _p(v), _p(a), _p(b), _p(o), _p(S_end))
    if return_state:
        return codes, R, c, o, S_end
    return codes, R, c, o


def recur_fp64(S: np.ndarray, gate, q, k, v, a, b):
    """One unquantized fp64 step, in place on S (float64 [dv, dk]); returns o."""
    assert S.dtype == np.float64 and S.flags.c_contiguous
    dv, dk = S.shape
    o = np.zeros(dv, np.float32)
    lib().oref_recur_fp64(dv, dk, gate, _p(S), _p(_c(q, np.float32)), _p(_c(k, np.float32)),
                          _p(_c(v, np.float32)), _p(_c(np.atleast_1d(a), np.float32)),
                          float(b), _p(o))
    return o


# ---------------------------------------------------------------------------
# compensator tokens (see qdr_oracle.h): m fp32 entries per unit, largest |S| first
# ---------------------------------------------------------------------------

TOK_EMPTY = 0xFFFF


def comp_select(S: np.ndarray, m: int):
    """Tokens of one unit's fp32 state: (tok_idx uint16 [m], tok_val [m], residual)."""
    R = _c(S, np.float32).copy()
    dv, dk = R.shape
    idx = np.zeros(m, np.uint16)
    val = np.zeros(m, np.float32)
    lib().oref_comp_select(dv, dk, int(m), _p(R), _p(idx), _p(val))
    return idx, val, R


def comp_quantize(S: np.ndarray, bits: np.ndarray, m: int):
    """(codes, R, c, tok_idx, tok_val) of one unit: tokens, then the residual quantized."""
    S = _c(S, np.float32)
    b = _c(bits, np.uint8)
    dv, dk = S.shape
    codes = np.zeros((dv, dk), np.int8)
    R = np.zeros(dk, np.float32)
    c = np.zeros(dv, np.float32)
    idx = np.zeros(m, np.uint16)
    val = np.zeros(m, np.float32)
    lib().oref_comp_quantize(dv, dk, _p(b), _p(S), int(m), _p(codes), _p(R), _p(c), _p(idx),
                             _p(val))
    return codes, R, c, idx, val


def comp_dequantize(codes, R, c, tok_idx, tok_val) -> np.ndarray:
    codes = _c(codes, np.int8)
    R, c = _c(R, np.float32), _c(c, np.float32)
    idx, val = _c(tok_idx, np.uint16), _c(tok_val, np.float32)
    dv, dk = codes.shape
    S = np.zeros((dv, dk), np.float32)
    lib().oref_comp_dequantize(dv, dk, _p(codes), _p(R), _p(c), idx.shape[0], _p(idx), _p(val),
                               _p(S))
    return S


def comp_window(codes, R, c, tok_idx, tok_val, bits, gate, q, k, v, a, b, return_state=False):
    """One window with compensator tokens on one unit.
    Returns (codes, R, c, tok_idx, tok_val, o[W, dv][, S_end])."""
    codes = _c(codes, np.int8).copy()
    R = _c(R, np.float32).copy()
    c = _c(c, np.float32).copy()
    idx = _c(tok_idx, np.uint16).copy()
    val = _c(tok_val, np.float32).copy()
    bb = _c(bits, np.uint8)
    dv, dk = codes.shape
    q, k, v = _c(q, np.float32), _c(k, np.float32), _c(v, np.float32)
    a, b = _c(a, np.float32), _c(b, np.float32)
    W = b.shape[0]
    o = np.zeros((W, dv), np.float32)
    S_end = np.zeros((dv, dk), np.float32) if return_state else None
    lib().oref_comp_window(dv, dk, gate, _p(bb), _p(codes), _p(R), _p(c), idx.shape[0],
                           _p(idx), _p(val), W, _p(q), _p(k), _p(v), _p(a), _p(b), _p(o),
                           _p(S_end))
    out = (codes, R, c, idx, val, o)
    return out + (S_end,) if return_state else out


# ---------------------------------------------------------------------------
# pool interface (the packed layout the product library uses)
# ---------------------------------------------------------------------------

class Pool:
    """Host copy of a packed state pool: packed[n_req, req_bytes], scales, bit map."""

    def __init__(self, n_req, n_head, bits, dv=128, dk=128, rule=RULE_STEP):
        self.n_req, self.n_head, self.dv, self.dk = n_req, n_head, dv, dk
        self.rule = int(rule)
        self.bits = _c(bits, np.uint8).reshape(n_head, dk)
        rb = lib().oref_request_bytes(n_head, dv, dk, _p(self.bits))
        if rb < 0:
            raise ValueError("bit map not representable")
        self.req_bytes = int(rb)
        self.packed = np.zeros((n_req, self.req_bytes), np.uint8)
        self.row_scale = np.zeros((n_req, n_head, dk), np.float32)
        self.col_scale = np.zeros((n_req, n_head, dv), np.float32)

    def copy(self):
        p = Pool.__new__(Pool)
        p.__dict__.update(self.__dict__)
        p.packed = self.packed.copy()
        p.row_scale = self.row_scale.copy()
        p.col_scale = self.col_scale.copy()
        if hasattr(self, "tok_idx"):
            p.tok_idx = self.tok_idx.copy()
            p.tok_val = self.tok_val.copy()
        return p

    # compensator tokens: tok_idx / tok_val [n_req, n_head, m]
    def comp_init(self, m: int):
        self.tok_idx = np.full((self.n_req, self.n_head, m), TOK_EMPTY, np.uint16)
        self.tok_val = np.zeros((self.n_req, self.n_head, m), np.float32)

    def comp_quantize(self, S: np.ndarray, m: int):
        S = _c(S, np.float32)
        assert S.shape == (self.n_req, self.n_head, self.dv, self.dk)
        self.comp_init(m)
        rc = lib().oref_comp_quantize_pool(self.n_req, self.n_head, self.dv, self.dk,
                                           _p(self.bits), _p(S), int(m), _p(self.packed),
                                           _p(self.row_scale), _p(self.col_scale),
                                           _p(self.tok_idx), _p(self.tok_val))
        if rc:
            raise RuntimeError("oref_comp_quantize_pool failed")

    def comp_dequantize(self) -> np.ndarray:
        S = np.zeros((self.n_req, self.n_head, self.dv, self.dk), np.float32)
        rc = lib().oref_comp_dequantize_pool(self.n_req, self.n_head, self.dv, self.dk,
                                             _p(self.bits), _p(self.packed), _p(self.row_scale),
                                             _p(self.col_scale), self.tok_idx.shape[-1],
                                             _p(self.tok_idx), _p(self.tok_val), _p(S))
        if rc:
            raise RuntimeError("oref_comp_dequantize_pool failed")
        return S

    def comp_window(self, gate, q, k, v, a, b, u0=0, u1=None):
        """window() with the pool's compensator tokens; returns o [W, n_req, n_head, dv]."""
        n_unit = self.n_req * self.n_head
        u1 = n_unit if u1 is None else u1
        q, k, v = _c(q, np.float32), _c(k, np.float32), _c(v, np.float32)
        a, b = _c(a, np.float32), _c(b, np.float32)
        W = b.shape[0]
        o = np.zeros((W, self.n_req, self.n_head, self.dv), np.float32)
        rc = lib().oref_comp_window_pool(self.n_req, self.n_head, self.dv, self.dk, gate,
                                         _p(self.bits), _p(self.packed), _p(self.row_scale),
                                         _p(self.col_scale), self.tok_idx.shape[-1],
                                         _p(self.tok_idx), _p(self.tok_val), W, _p(q), _p(k),
                                         _p(v), _p(a), _p(b), _p(o), u0, u1)
        if rc:
            raise RuntimeError("oref_comp_window_pool failed")
        return o

    def quantize(self, S: np.ndarray):
        S = _c(S, np.float32)
        assert S.shape == (self.n_req, self.n_head, self.dv, self.dk)
        rc = lib().oref_quantize_pool_rule(self.n_req, self.n_head, self.dv, self.dk,
                                           _p(self.bits), _p(S), _p(self.packed),
                                           _p(self.row_scale), _p(self.col_scale), self.rule)
        if rc:
            raise RuntimeError("oref_quantize_pool failed")

    def dequantize(self) -> np.ndarray:
        S = np.zeros((self.n_req, self.n_head, self.dv, self.dk), np.float32)
        rc = lib().oref_dequantize_pool(self.n_req, self.n_head, self.dv, self.dk,
                                        _p(self.bits), _p(self.packed), _p(self.row_scale),
                                        _p(self.col_scale), _p(S))
        if rc:
            raise RuntimeError("oref_dequantize_pool failed")
        return S

    def step(self, gate, q, k, v, a, b, u0=0, u1=None):
        """One decode step on units [u0, u1) in place; returns o [n_req, n_head, dv]."""
        n_unit = self.n_req * self.n_head
        u1 = n_unit if u1 is None else u1
        o = np.zeros((self.n_req, self.n_head, self.dv), np.float32)
        q, k, v = _c(q, np.float32), _c(k, np.float32), _c(v, np.float32)
        a, b = _c(a, np.float32), _c(b, np.float32)
        rc = lib().oref_step_pool_rule(self.n_req, self.n_head, self.dv, self.dk, gate,
                                       _p(self.bits), _p(self.packed), _p(self.row_scale),
                                       _p(self.col_scale), _p(q), _p(k), _p(v), _p(a), _p(b),
                                       _p(o), u0, u1, self.rule)
        if rc:
            raise RuntimeError("oref_step_pool failed")
        return o

    def step_threads(self, gate, q, k, v, a, b, threads=8):
        """``step`` over all units, split into contiguous unit ranges on host threads
        (the C code releases the GIL; ranges are disjoint, so results are identical)."""
        from concurrent.futures import ThreadPoolExecutor

        n_unit = self.n_req * self.n_head
        q, k, v = _c(q, np.float32), _c(k, np.float32), _c(v, np.float32)
        a, b = _c(a, np.float32), _c(b, np.float32)
        o = np.zeros((self.n_req, self.n_head, self.dv), np.float32)
        cuts = np.linspace(0, n_unit, max(1, min(threads, n_unit)) + 1).astype(int)

        def run(i):
            return lib().oref_step_pool_rule(self.n_req, self.n_head, self.dv, self.dk, gate,
                                             _p(self.bits), _p(self.packed),
                                             _p(self.row_scale), _p(self.col_scale), _p(q),
                                             _p(k), _p(v), _p(a), _p(b), _p(o),
                                             int(cuts[i]), int(cuts[i + 1]), self.rule)

        with ThreadPoolExecutor(len(cuts) - 1) as ex:
            rcs = list(ex.map(run, range(len(cuts) - 1)))
        if any(rcs):
            raise RuntimeError("oref_step_pool failed")
        return o

    def window(self, gate, q, k, v, a, b, u0=0, u1=None):
        """One window over W tokens (inputs [W, n_req, n_head, ...]); returns o."""
        n_unit = self.n_req * self.n_head
        u1 = n_unit if u1 is None else u1
        q, k, v = _c(q, np.float32), _c(k, np.float32), _c(v, np.float32)
        a, b = _c(a, np.float32), _c(b, np.float32)
        W = b.shape[0]
        o = np.zeros((W, self.n_req, self.n_head, self.dv), np.float32)
        rc = lib().oref_window_pool(self.n_req, self.n_head, self.dv, self.dk, gate,
                                    _p(self.bits), _p(self.packed), _p(self.row_scale),
                                    _p(self.col_scale), W, _p(q), _p(k), _p(v), _p(a),
                                    _p(b), _p(o), u0, u1)
        if rc:
            raise RuntimeError("oref_window_pool failed")
        return o

    def window_threads(self, gate, q, k, v, a, b, threads=8):
        """``window`` over all units, split into contiguous unit ranges on host threads
        (disjoint ranges, so the results are those of ``window``)."""
        from concurrent.futures import ThreadPoolExecutor

        n_unit = self.n_req * self.n_head
        q, k, v = _c(q, np.float32), _c(k, np.float32), _c(v, np.float32)
        a, b = _c(a, np.float32), _c(b, np.float32)
        W = b.shape[0]
        o = np.zeros((W, self.n_req, self.n_head, self.dv), np.float32)
        cuts = np.linspace(0, n_unit, max(1, min(threads, n_unit)) + 1).astype(int)

        def run(i):
            return lib().oref_window_pool(self.n_req, self.n_head, self.dv, self.dk, gate,
                                          _p(self.bits), _p(self.packed), _p(self.row_scale),
                                          _p(self.col_scale), W, _p(q), _p(k), _p(v), _p(a),
                                          _p(b), _p(o), int(cuts[i]), int(cuts[i + 1]))

        with ThreadPoolExecutor(len(cuts) - 1) as ex:
            rcs = list(ex.map(run, range(len(cuts) - 1)))
        if any(rcs):
            raise RuntimeError("oref_window_pool failed")
        return o


# ---------------------------------------------------------------------------
# DAMP-style storage variant (see qdr_oracle.h)
# ---------------------------------------------------------------------------

DAMP_HALF = 16


DAMP_PHILOX_ROUNDS = 7


def philox4x32(ctr, key, rounds):
    """Philox4x32 block with `rounds` rounds: 4 counter words, 2 key words -> 4 words."""
    c = np.asarray(ctr, np.uint32).copy()
    k = np.asarray(key, np.uint32).copy()
    out = np.zeros(4, np.uint32)
    lib().oref_philox4x32(_p(c), _p(k), int(rounds), _p(out))
    return out


def philox4x32_10(ctr, key):
    """Philox4x32-10 block: 4 counter words, 2 key words -> 4 output words."""
    c = np.asarray(ctr, np.uint32).copy()
    k = np.asarray(key, np.uint32).copy()
    out = np.zeros(4, np.uint32)
    lib().oref_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def f32_to_f16_bits(x: float) -> int:
    return int(lib().oref_f32_to_f16(float(x)))


def f16_bits_to_f32(h: int) -> float:
    return float(lib().oref_f16_to_f32(int(h)))


def damp_perm(sel: np.ndarray) -> np.ndarray:
    """sel [n_head][128] flags (16 per head) -> perm [n_head][128] (physical -> logical)."""
    sel = _c(sel, np.uint8).reshape(-1, 128)
    perm = np.zeros_like(sel)
    for h in range(sel.shape[0]):
        if lib().oref_damp_perm(128, _p(sel[h]), _p(perm[h])) != 0:
            raise ValueError("each head needs exactly 16 selected channels")
    return perm


class DampPool:
    """Host DAMP-variant pool: half [n_unit][128][16] (binary16 bits), codes
    [n_unit][128][112], R [n_unit][112]; units r * n_head + h."""

    def __init__(self, n_req, n_head, sel, seed=0):
        self.n_req, self.n_head = n_req, n_head
        self.n_unit = n_req * n_head
        self.perm = damp_perm(sel)
        self.seed = int(seed)
        self.half = np.zeros((self.n_unit, 128, DAMP_HALF), np.uint16)
        self.codes = np.zeros((self.n_unit, 128, 128 - DAMP_HALF), np.int8)
        self.R = np.full((self.n_unit, 128 - DAMP_HALF), np.float32(1.0 / 127.0), np.float32)

    def copy(self):
        p = DampPool.__new__(DampPool)
        p.__dict__.update(self.__dict__)
        p.half, p.codes, p.R = self.half.copy(), self.codes.copy(), self.R.copy()
        return p

    def quantize(self, S: np.ndarray, step: int = 0):
        S = _c(S, np.float32).reshape(self.n_unit, 128, 128)
        lib().oref_damp_quantize_pool(self.n_unit, self.n_head, 128, _p(self.perm), _p(S),
                                      _p(self.half), _p(self.codes), _p(self.R), self.seed,
                                      int(step))

    def dequantize(self) -> np.ndarray:
        S = np.zeros((self.n_unit, 128, 128), np.float32)
        lib().oref_damp_dequantize_pool(self.n_unit, self.n_head, 128, _p(self.perm),
                                        _p(self.half), _p(self.codes), _p(self.R), _p(S))
        return S.reshape(self.n_req, self.n_head, 128, 128)

    def step(self, gate, q, k, v, a, b, step: int, u0: int = 0, u1=None):
        """One step on units [u0, u1) (default all); returns o for the whole pool."""
        q, k, v = _c(q, np.float32), _c(k, np.float32), _c(v, np.float32)
        a, b = _c(a, np.float32), _c(b, np.float32)
        o = np.zeros((self.n_req, self.n_head, 128), np.float32)
        lib().oref_damp_step_pool(self.n_unit, self.n_head, 128, gate, _p(self.perm),
                                  _p(self.half), _p(self.codes), _p(self.R), _p(q), _p(k),
                                  _p(v), _p(a), _p(b), _p(o), self.seed, int(step), int(u0),
                                  self.n_unit if u1 is None else int(u1))
        return o
