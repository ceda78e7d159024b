"""C-ABI checks that need no GPU: the library loads, exports every symbol the header
declares, and its host-side logic (validation, sizes, bit map) behaves as documented."""
import ctypes
import os
import re

import numpy as np
import pytest

from quantized_delta_rule_03_amd import qdr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_symbols():
    text = open(os.path.join(ROOT, "include", "qdr.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qdr_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = qdr.lib()
    syms = header_symbols()
    assert set(syms) == set(qdr.SYMBOLS), syms
    for s in syms:
        assert hasattr(L, s), s


def test_assign_bits_matches_oracle(oref):
    rng = np.random.default_rng(1)
    tau = np.exp(rng.uniform(0, np.log(4096), 32))
    assert np.array_equal(qdr.assign_bits(qdr.GDN, tau), oref.assign_bits(0, tau, 128))
    tau2 = np.exp(rng.uniform(0, np.log(8192), (8, 128)))
    assert np.array_equal(qdr.assign_bits(qdr.KDA, tau2), oref.assign_bits(1, tau2, 128))
    ties = np.ones(12)
    assert np.array_equal(qdr.assign_bits(qdr.GDN, ties), oref.assign_bits(0, ties, 128))


@pytest.mark.parametrize("gate", [0, 1])
def test_state_bytes_matches_oracle_layout(oref, gate):
    rng = np.random.default_rng(2)
    if gate == 0:
        bits = qdr.assign_bits(0, np.exp(rng.uniform(0, 8, 32)))
    else:
        bits = qdr.assign_bits(1, np.exp(rng.uniform(0, 9, (32, 128))))
    L = qdr.Layout(7, 32, gate, bits, window=64)
    pool = oref.Pool(7, 32, bits)
    assert L.packed_bytes == 7 * pool.req_bytes
    assert L.scale_bytes == 7 * 32 * 128 * 4
    assert L.meta_bytes == 64 + 32 * 272 + 64
    assert L.window_bytes == 7 * 32 * (64 * 2 * 128 * 4 + 2 * 128 * 4)


def _desc(n_req=2, n_head=4, dk=128, dv=128, gate=0, bits=None, window=0, rule=0):
    if bits is None:
        bits = np.full((n_head, 128), 8, np.uint8)
    d = qdr.Desc(n_req, n_head, dk, dv, gate, bits.ctypes.data if bits is not False else None,
                 window, rule)
    return d, bits


def _state_bytes(d):
    s = [ctypes.c_size_t() for _ in range(4)]
    return qdr.lib().qdr_state_bytes(ctypes.byref(d), *[ctypes.byref(x) for x in s])


@pytest.mark.parametrize("kw,code", [
    (dict(dk=64), qdr.QDR_EUNSUPPORTED),
    (dict(dv=256), qdr.QDR_EUNSUPPORTED),
    (dict(n_head=0), qdr.QDR_EINVAL),
    (dict(n_req=-1), qdr.QDR_EINVAL),
    (dict(gate=7), qdr.QDR_EINVAL),
    (dict(window=-3), qdr.QDR_EINVAL),
])
def test_descriptor_validation(kw, code):
    d, keep = _desc(**kw)
    assert _state_bytes(d) == code
    assert qdr.last_error() != ""


def test_bad_bit_maps():
    bits = np.full((4, 128), 8, np.uint8)
    bits[1, 5] = 5
    d, keep = _desc(bits=bits)
    assert _state_bytes(d) == qdr.QDR_EUNSUPPORTED
    assert "bits[1][5]" in qdr.last_error()
    bits = np.full((4, 128), 8, np.uint8)
    bits[2, :20] = 4
    d, keep = _desc(bits=bits)
    assert _state_bytes(d) == qdr.QDR_EUNSUPPORTED
    d = qdr.Desc(2, 4, 128, 128, 0, None, 0)
    assert _state_bytes(d) == qdr.QDR_EINVAL


def test_pointer_validation_before_any_launch():
    """Null and misaligned device pointers are rejected on the host (no GPU touched)."""
    d, keep = _desc()
    L = qdr.lib()
    P = 1 << 20  # aligned fake address, never dereferenced because validation fails first
    rc = L.qdr_decode_step(ctypes.byref(d), P, P, P, P, P, P, P, P, None, P, None)
    assert rc == qdr.QDR_EINVAL and "b is NULL" in qdr.last_error()
    rc = L.qdr_decode_step(ctypes.byref(d), P, P + 4, P, P, P, P, P, P, P, P, None)
    assert rc == qdr.QDR_EALIGN and "packed" in qdr.last_error()
    rc = L.qdr_quantize_state(ctypes.byref(d), None, P, P, P, P, None)
    assert rc == qdr.QDR_EINVAL and "meta" in qdr.last_error()
    rc = L.qdr_dequantize_state(ctypes.byref(d), P, P, P, P + 8, P, None)
    assert rc == qdr.QDR_EALIGN


def test_static_window_size_limit():
    """qdr_decode_window_static holds n_req * n_head * (1024 W + 1024) bytes in its 32 MiB
    array: 504 units at W = 64 fit (the call goes on to its pointer checks), 505 do not."""
    L = qdr.lib()
    P = 1 << 20
    d, keep = _desc(n_req=505, n_head=1, window=64)
    rc = L.qdr_decode_window_static(ctypes.byref(d), P, P, P, P, 0, P, P, P, P, P, P, None)
    assert rc == qdr.QDR_EUNSUPPORTED and "33612800 bytes" in qdr.last_error()
    d, keep = _desc(n_req=504, n_head=1, window=64)
    rc = L.qdr_decode_window_static(ctypes.byref(d), None, P, P, P, 0, P, P, P, P, P, P, None)
    assert rc == qdr.QDR_EINVAL and "meta" in qdr.last_error()


def test_window_position_validation():
    d, keep = _desc(window=0)
    L = qdr.lib()
    P = 1 << 20
    rc = L.qdr_decode_window(ctypes.byref(d), P, P, P, P, P, 0, P, P, P, P, P, P, None)
    assert rc == qdr.QDR_EUNSUPPORTED
    d, keep = _desc(window=64)
    rc = L.qdr_decode_window(ctypes.byref(d), P, P, P, P, P, 64, P, P, P, P, P, P, None)
    assert rc == qdr.QDR_EUNSUPPORTED and "t = 64" in qdr.last_error()
    rc = L.qdr_decode_window(ctypes.byref(d), P, P, P, P, P, -1, P, P, P, P, P, P, None)
    assert rc == qdr.QDR_EUNSUPPORTED
    d, keep = _desc(window=300)
    rc = L.qdr_decode_window(ctypes.byref(d), P, P, P, P, P, 3, P, P, P, P, P, P, None)
    assert rc == qdr.QDR_EUNSUPPORTED and "exceeds" in qdr.last_error()
    d, keep = _desc(window=64)
    rc = L.qdr_decode_window(ctypes.byref(d), P, P, P, P, None, 3, P, P, P, P, P, P, None)
    assert rc == qdr.QDR_EINVAL and "window_buf" in qdr.last_error()


def test_chunk_validation():
    d, keep = _desc()
    L = qdr.lib()
    P = 1 << 20
    rc = L.qdr_decode_chunk(ctypes.byref(d), P, P, P, P, -1, P, P, P, P, P, P, None)
    assert rc == qdr.QDR_EINVAL and "T = -1" in qdr.last_error()
    rc = L.qdr_decode_chunk(ctypes.byref(d), P, P, P, P, 16, P, P, P, P, P, None, None)
    assert rc == qdr.QDR_EINVAL and "o is NULL" in qdr.last_error()
    rc = L.qdr_decode_chunk(ctypes.byref(d), P, P, P, P, 16, P, P + 4, P, P, P, P, None)
    assert rc == qdr.QDR_EALIGN and "k" in qdr.last_error()


def test_comp_validation():
    """Compensator-token entry points: m range, rule, token buffers (no GPU work)."""
    d, keep = _desc()
    L = qdr.lib()
    P = 1 << 20
    for bad in (-1, qdr.COMP_MAX + 1):
        rc = L.qdr_comp_chunk(ctypes.byref(d), P, P, P, P, bad, P, P, 8, P, P, P, P, P, P, None)
        assert rc == qdr.QDR_EINVAL and f"m = {bad}" in qdr.last_error()
    rc = L.qdr_comp_quantize(ctypes.byref(d), P, P, P, P, 4, None, P, P, None)
    assert rc == qdr.QDR_EINVAL and "tok_idx is NULL" in qdr.last_error()
    rc = L.qdr_comp_dequantize(ctypes.byref(d), P, P, P, P, 4, P, P + 8, P, None)
    assert rc == qdr.QDR_EALIGN and "tok_val" in qdr.last_error()
    rc = L.qdr_comp_chunk(ctypes.byref(d), P, P, P, P, 4, P, P, -2, P, P, P, P, P, P, None)
    assert rc == qdr.QDR_EINVAL and "T = -2" in qdr.last_error()
    rc = L.qdr_comp_quantize(ctypes.byref(d), P, P, P, P, 4, P, P, None, None)
    assert rc == qdr.QDR_EINVAL and "S_in is NULL" in qdr.last_error()
    d, keep = _desc(rule=qdr.RULE_KEYROW)
    rc = L.qdr_comp_quantize(ctypes.byref(d), P, P, P, P, 4, P, P, P, None)
    assert rc == qdr.QDR_EUNSUPPORTED and "QDR_RULE_STEP" in qdr.last_error()
    d, keep = _desc(window=8)
    rc = L.qdr_comp_window(ctypes.byref(d), P, P, P, P, 4, P, P, P, 8, P, P, P, P, P, P, None)
    assert rc == qdr.QDR_EUNSUPPORTED and "t = 8" in qdr.last_error()
    rc = L.qdr_comp_window(ctypes.byref(d), P, P, P, P, 4, None, P, P, 0, P, P, P, P, P, P, None)
    assert rc == qdr.QDR_EINVAL and "tok_idx is NULL" in qdr.last_error()
    d, keep = _desc()
    rc = L.qdr_comp_window(ctypes.byref(d), P, P, P, P, 4, P, P, P, 0, P, P, P, P, P, P, None)
    assert rc == qdr.QDR_EUNSUPPORTED and "no window mode" in qdr.last_error()
    # nothing to do: zero requests or T = 0 with no buffers at all
    d, keep = _desc(n_req=0)
    assert L.qdr_comp_quantize(ctypes.byref(d), P, None, None, None, 4, None, None, None,
                               None) == qdr.QDR_OK
    d, keep = _desc()
    assert L.qdr_comp_chunk(ctypes.byref(d), P, None, None, None, 4, None, None, 0, None, None,
                            None, None, None, None, None) == qdr.QDR_OK


def test_rule_validation():
    L = qdr.lib()
    P = 1 << 20
    for bad in (-1, 3):
        d, keep = _desc(rule=bad)
        assert _state_bytes(d) == qdr.QDR_EINVAL and "rule" in qdr.last_error()
    d, keep = _desc(rule=qdr.RULE_TENSOR)
    assert _state_bytes(d) == qdr.QDR_OK
    d, keep = _desc(window=8, rule=qdr.RULE_KEYROW)
    rc = L.qdr_decode_window(ctypes.byref(d), P, P, P, P, P, 0, P, P, P, P, P, P, None)
    assert rc == qdr.QDR_EUNSUPPORTED and "QDR_RULE_STEP" in qdr.last_error()
    rc = L.qdr_decode_chunk(ctypes.byref(d), P, P, P, P, 4, P, P, P, P, P, P, None)
    assert rc == qdr.QDR_EUNSUPPORTED and "QDR_RULE_STEP" in qdr.last_error()


def test_damp_validation_and_sizes():
    L = qdr.lib()
    P = 1 << 20
    sel = np.zeros((4, 128), np.uint8)
    sel[:, :16] = 1
    d = qdr.DampDesc(2, 4, 1, sel.ctypes.data)
    s = [ctypes.c_size_t() for _ in range(4)]
    assert L.qdr_damp_bytes(ctypes.byref(d), *[ctypes.byref(x) for x in s]) == qdr.QDR_OK
    assert [x.value for x in s] == [8 * 128 * 16 * 2, 8 * 128 * 112, 8 * 112 * 4, 4 * 128]
    sel[2, 40] = 1
    assert L.qdr_damp_bytes(ctypes.byref(d), None, None, None, None) == qdr.QDR_EUNSUPPORTED
    assert "17" in qdr.last_error()
    d = qdr.DampDesc(2, 4, 1, None)
    assert L.qdr_damp_bytes(ctypes.byref(d), None, None, None, None) == qdr.QDR_EINVAL
    sel[2, 40] = 0
    d = qdr.DampDesc(2, 4, 1, sel.ctypes.data)
    rc = L.qdr_damp_step(ctypes.byref(d), P, P, P, P, P, P, P, P, None, P, 0, 0, None)
    assert rc == qdr.QDR_EINVAL and "b is NULL" in qdr.last_error()
    rc = L.qdr_damp_quantize(ctypes.byref(d), P, P + 4, P, P, P, 0, 0, None)
    assert rc == qdr.QDR_EALIGN


def test_damp_select_takes_the_longest_lived_channels():
    rng = np.random.default_rng(0)
    tau = np.exp(rng.uniform(0, 9, (3, 128)))
    tau[1, 5:40] = tau[1, 5]  # ties: lowest indices first
    sel = qdr.damp_select(1, tau, 3)
    for h in range(3):
        want = np.zeros(128, np.uint8)
        want[np.argsort(-tau[h], kind="stable")[:16]] = 1
        assert np.array_equal(sel[h], want)
    g = qdr.damp_select(0, np.ones(3), 3)
    assert np.all(g[:, :16] == 1) and np.all(g[:, 16:] == 0)


def test_errors_are_thread_local():
    import threading

    d, keep = _desc(dk=64)
    assert _state_bytes(d) == qdr.QDR_EUNSUPPORTED
    seen = {}

    def other():
        seen["text"] = qdr.last_error()

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["text"] == ""
    assert qdr.last_error() != ""


def test_bit_map_summaries_are_never_stale():
    """The ABI caches the summary of each validated bit map; a map edited in place (same
    pointer) must be validated afresh, both when it turns invalid and when it changes the
    sizes."""
    lib = qdr.lib()
    bits = np.full((4, 128), 8, np.uint8)
    d, _ = _desc(n_req=3, n_head=4, bits=bits)
    sz = [ctypes.c_size_t() for _ in range(4)]
    assert lib.qdr_state_bytes(ctypes.byref(d), *[ctypes.byref(x) for x in sz]) == 0
    assert sz[0].value == 3 * 4 * 16384
    bits[1, :] = 4  # same pointer, other widths: head 1 now takes 8 KB
    assert lib.qdr_state_bytes(ctypes.byref(d), *[ctypes.byref(x) for x in sz]) == 0
    assert sz[0].value == 3 * (3 * 16384 + 8192)
    bits[2, 5] = 5  # invalid width
    assert lib.qdr_state_bytes(ctypes.byref(d), *[ctypes.byref(x) for x in sz]) == qdr.QDR_EUNSUPPORTED
    bits[2, 5] = 8
    assert lib.qdr_state_bytes(ctypes.byref(d), *[ctypes.byref(x) for x in sz]) == 0
    # many distinct maps in turn (more than the cache holds), each sized correctly
    for k in range(20):
        b = np.full((2, 128), 8, np.uint8)
        b[k % 2, : 32 * (1 + k % 3)] = 4
        dk_, _ = _desc(n_req=1, n_head=2, bits=b)
        assert lib.qdr_state_bytes(ctypes.byref(dk_), *[ctypes.byref(x) for x in sz]) == 0
        assert sz[0].value == 16 * int(b.astype(np.int64).sum())
