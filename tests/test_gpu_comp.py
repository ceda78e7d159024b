"""GPU parity of the compensator tokens (qdr_comp_quantize / qdr_comp_chunk /
qdr_comp_window / qdr_comp_dequantize) against the oracle.

Quantize and dequantize take the same fp32 inputs on both sides, so they are compared
bit for bit (packed codes, scales, token indices and values), including the cases that
drive the kernel's two selection paths: few candidates ranked in LDS, and many equal
magnitudes (a constant-magnitude state) that take the exact bisection. A chunk (or a
window of per-token calls) runs fp32 arithmetic on the GPU and the fp64 window recurrence
in the oracle, so it is compared teacher-forced at the chunk and window bar: readouts rel-L2 <= 1e-4; the same token set
(or, at a near-tie of magnitudes, differences only among entries within 1e-5 of the cut)
with values to 1e-5; codes within 1 LSB on <= 1e-4 of entries; scales to 1e-5.
"""
import numpy as np
import pytest

import oracle
from parity_tools import (CODE_FLIP_FRAC, DRIFT_REL_L2, O_REL_L2, bits_for, compare_codes,
                          gpu_to_oracle, prewarmed_state, rel_l2, to_dev)
from quantized_delta_rule_03_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_delta_rule_03_amd import qdr

    qdr.lib()
    return torch


def spikes(S, seed, n=12, scale=40.0):
    """Isolated large entries in every unit (the outliers the tokens are for)."""
    rng = np.random.default_rng(seed)
    S = S.copy()
    flat = S.reshape(-1, 128 * 128)
    for u in range(flat.shape[0]):
        pos = rng.choice(128 * 128, n, replace=False)
        flat[u, pos] = scale * rng.uniform(0.5, 1.0, n) * np.where(rng.random(n) < 0.5, -1, 1)
    return S.astype(np.float32)


def gpu_pool(torch, w, n_req, n_head, bits):
    from quantized_delta_rule_03_amd import qdr

    return qdr.StatePool(n_req, n_head, w.gate, bits)


def check_quantize(torch, w, bits, S, m, name):
    n_req, n_head = S.shape[:2]
    gpu = gpu_pool(torch, w, n_req, n_head, bits)
    print(f"[comp quantize] {name}: n_req={n_req} n_head={n_head} m={m}", flush=True)
    gpu.comp_quantize(torch.from_numpy(S).cuda(), m)
    ref = oracle.Pool(n_req, n_head, bits)
    ref.comp_quantize(S, m)
    packed, R, c = gpu.to_host()
    idx, val = gpu.comp_to_host()
    assert np.array_equal(idx, ref.tok_idx), name
    assert np.array_equal(val.view(np.uint32), ref.tok_val.view(np.uint32)), name
    assert np.array_equal(packed, ref.packed), name
    assert np.array_equal(R.view(np.uint32), ref.row_scale.view(np.uint32)), name
    assert np.array_equal(c.view(np.uint32), ref.col_scale.view(np.uint32)), name
    D = gpu.comp_dequantize().cpu().numpy()
    assert np.array_equal(D.view(np.uint32), ref.comp_dequantize().view(np.uint32)), name
    return gpu, ref


def test_comp_quantize_and_dequantize_bit_exact(torch_cuda):
    w = wl.WORKLOADS[2]
    H = 8
    bits = bits_for(w, n_head=H)
    rng = np.random.default_rng(3)
    base = (0.1 * rng.standard_normal((2, H, 128, 128))).astype(np.float32)
    S = spikes(base, 4)
    for m in (1, 16, 64):
        check_quantize(torch_cuda, w, bits, S, m, f"spiky m={m}")
    check_quantize(torch_cuda, w, bits, S, 0, "m=0")
    check_quantize(torch_cuda, w, bits, np.ascontiguousarray(prewarmed_state(w, 1)[:, :H]), 16,
                   "prewarmed outlier rows/columns")


def test_comp_selection_edge_cases(torch_cuda):
    w = wl.WORKLOADS[1]
    H = 4
    bits = bits_for(w, n_head=H)
    rng = np.random.default_rng(5)
    S = np.zeros((1, H, 128, 128), np.float32)
    # unit 0: constant magnitude, random signs -> every entry ties (bisection path)
    S[0, 0] = np.where(rng.random((128, 128)) < 0.5, -1.0, 1.0)
    # unit 1: a plateau of equal small entries with five larger ones (bisection path;
    # the cut falls inside the plateau, lowest flat indices first)
    S[0, 1] = 0.25
    S[0, 1].flat[[9000, 17, 12345, 400, 16383]] = -3.0
    # unit 2: three nonzero entries and a negative zero (fewer than m: empty slots)
    S[0, 2].flat[[5, 700, 16000]] = [1.0, -2.0, 0.5]
    S[0, 2].flat[9] = -0.0
    # unit 3: spikes with an exact tie of magnitudes at the m-th place (LDS ranking)
    S[0, 3] = 0.05 * rng.standard_normal((128, 128))
    pos = rng.choice(128 * 128, 17, replace=False)
    S[0, 3].flat[pos[:15]] = 30.0 + np.arange(15)
    S[0, 3].flat[pos[15]] = 20.0
    S[0, 3].flat[pos[16]] = -20.0
    check_quantize(torch_cuda, w, bits, S, 16, "ties / plateau / sparse / exact tie")
    check_quantize(torch_cuda, w, bits, np.zeros_like(S), 16, "zero state")


def token_sets_agree(gi, gv, ri, rv, name):
    """Same tokens, or (near-tie at the cut) differences only within 1e-5 of the cut."""
    for u in range(gi.shape[0]):
        a = {int(i): float(v) for i, v in zip(gi[u], gv[u]) if i != oracle.TOK_EMPTY}
        b = {int(i): float(v) for i, v in zip(ri[u], rv[u]) if i != oracle.TOK_EMPTY}
        if a.keys() != b.keys():
            cut = min(abs(v) for v in b.values())
            for i in a.keys() ^ b.keys():
                x = a.get(i, b.get(i))
                assert abs(abs(x) - cut) <= 1e-5 * cut, (name, u, i, x, cut)
            return False
        va = np.array([a[i] for i in sorted(a)])
        vb = np.array([b[i] for i in sorted(b)])
        assert rel_l2(va, vb) <= 1e-5, (name, u)
    return True


def run_comp_chunks(torch, w, n_req, n_head, bits, m, T, n_chunks, S0, name):
    from quantized_delta_rule_03_amd import qdr

    gpu = qdr.StatePool(n_req, n_head, w.gate, bits)
    ref = oracle.Pool(n_req, n_head, bits)
    ref.comp_quantize(S0, m)
    gpu.load_host(ref.packed, ref.row_scale, ref.col_scale)
    gpu.comp_load_host(ref.tok_idx, ref.tok_val)
    worst_o, worst_flip, worst_lsb, ties = 0.0, 0.0, 0, 0
    for c in range(n_chunks):
        toks = []
        for t in range(T):
            inp = wl.step_inputs(w, c * T + t, n_req=n_req)
            toks.append({k: np.ascontiguousarray(v[:, :n_head]) for k, v in inp.items()})
        stack = {k: np.ascontiguousarray(np.stack([x[k] for x in toks])) for k in toks[0]}
        print(f"[{name}] chunk {c}: T={T} m={m} n_req={n_req} n_head={n_head}", flush=True)
        tf = gpu_to_oracle(gpu, bits)
        tf.tok_idx, tf.tok_val = [x.copy() for x in gpu.comp_to_host()]
        o_tf = tf.comp_window(w.gate, stack["q"], stack["k"], stack["v"], stack["a"],
                              stack["b"])
        ref.comp_window(w.gate, stack["q"], stack["k"], stack["v"], stack["a"], stack["b"])
        dev = to_dev(stack)
        o = torch.full((T, n_req, n_head, 128), float("nan"), dtype=torch.float32, device="cuda")
        gpu.comp_chunk(dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], o)
        og = o.cpu().numpy()
        assert np.isfinite(og).all(), name
        for t in range(T):
            worst_o = max(worst_o, rel_l2(og[t], o_tf[t]))
        gi, gv = gpu.comp_to_host()
        same = token_sets_agree(gi.reshape(-1, m), gv.reshape(-1, m),
                                tf.tok_idx.reshape(-1, m), tf.tok_val.reshape(-1, m), name)
        if not same:
            ties += 1
            continue
        g = gpu_to_oracle(gpu, bits)
        lsb, frac = compare_codes(g.packed, tf.packed, tf)
        worst_lsb, worst_flip = max(worst_lsb, lsb), max(worst_flip, frac)
        assert np.allclose(g.row_scale, tf.row_scale, rtol=1e-5, atol=0), name
        assert np.allclose(g.col_scale, tf.col_scale, rtol=1e-5, atol=0), name
    drift = rel_l2(gpu.comp_dequantize().cpu().numpy(), ref.comp_dequantize())
    print(f"[{name}] chunks={n_chunks} T={T} m={m} worst o rel-L2 tf={worst_o:.2e} "
          f"worst flips tf={worst_flip:.2e} (max {worst_lsb} LSB) near-tie chunks={ties} "
          f"drift={drift:.2e}", flush=True)
    assert worst_o <= O_REL_L2, name
    assert worst_lsb <= 1 and worst_flip <= CODE_FLIP_FRAC, name
    assert ties < n_chunks, name
    assert drift <= DRIFT_REL_L2, name


def test_comp_chunk_kda_8bit_prewarmed(torch_cuda):
    """Windowed serving shape (KDA, 8-bit, T = 64) on pre-warmed outlier states with
    spikes, 16 tokens per unit."""
    w = wl.WORKLOADS[4]
    n_req = 2
    S0 = spikes(prewarmed_state(w, n_req), 11)
    run_comp_chunks(torch_cuda, w, n_req, w.n_head, bits_for(w), 16, w.window, 2, S0,
                    "comp kda 8-bit T=64")


def test_comp_chunk_gdn_mixed_widths(torch_cuda):
    w = wl.WORKLOADS[1]
    H = 8
    rng = np.random.default_rng(12)
    S0 = spikes((0.1 * rng.standard_normal((1, H, 128, 128))).astype(np.float32), 13)
    run_comp_chunks(torch_cuda, w, 1, H, bits_for(w, n_head=H), 64, 40, 3, S0,
                    "comp gdn mixed T=40 m=64")


def test_comp_chunk_m0_is_the_plain_chunk(torch_cuda):
    from quantized_delta_rule_03_amd import qdr

    w = wl.WORKLOADS[2]
    H, T = 4, 33
    bits = bits_for(w, n_head=H)
    rng = np.random.default_rng(14)
    S0 = (0.1 * rng.standard_normal((1, H, 128, 128))).astype(np.float32)
    toks = [wl.step_inputs(w, t, n_req=1) for t in range(T)]
    stack = {k: np.ascontiguousarray(np.stack([x[k][:, :H] for x in toks])) for k in toks[0]}
    dev = to_dev(stack)
    outs = []
    for comp in (False, True):
        gpu = qdr.StatePool(1, H, w.gate, bits)
        gpu.quantize(torch_cuda.from_numpy(S0).cuda())
        o = torch_cuda.empty((T, 1, H, 128), dtype=torch_cuda.float32, device="cuda")
        if comp:
            gpu.comp_enable(0)
            gpu.comp_chunk(dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], o)
        else:
            gpu.chunk(dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], o)
        outs.append((o.cpu().numpy(), *gpu.to_host()))
    for x, y in zip(*outs):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


def run_comp_windows(torch, w, n_req, n_head, bits, m, W, n_windows, S0, name):
    """Window mode with tokens: W per-token calls (the last one folds), teacher-forced
    against the oracle's window with tokens from the GPU's state at each window start."""
    from quantized_delta_rule_03_amd import qdr

    gpu = qdr.StatePool(n_req, n_head, w.gate, bits, window=W)
    ref = oracle.Pool(n_req, n_head, bits)
    ref.comp_quantize(S0, m)
    gpu.load_host(ref.packed, ref.row_scale, ref.col_scale)
    gpu.comp_load_host(ref.tok_idx, ref.tok_val)
    worst_o, worst_flip, worst_lsb, ties = 0.0, 0.0, 0, 0
    o = torch.empty((n_req, n_head, 128), dtype=torch.float32, device="cuda")
    for c in range(n_windows):
        toks = []
        for t in range(W):
            inp = wl.step_inputs(w, c * W + t, n_req=n_req)
            toks.append({k: np.ascontiguousarray(v[:, :n_head]) for k, v in inp.items()})
        stack = {k: np.ascontiguousarray(np.stack([x[k] for x in toks])) for k in toks[0]}
        print(f"[{name}] window {c}: W={W} m={m} n_req={n_req} n_head={n_head}", flush=True)
        tf = gpu_to_oracle(gpu, bits)
        tf.tok_idx, tf.tok_val = [x.copy() for x in gpu.comp_to_host()]
        o_tf = tf.comp_window(w.gate, stack["q"], stack["k"], stack["v"], stack["a"],
                              stack["b"])
        ref.comp_window(w.gate, stack["q"], stack["k"], stack["v"], stack["a"], stack["b"])
        dev = to_dev(stack)
        for t in range(W):
            gpu.comp_window_token(t, dev["q"][t], dev["k"][t], dev["v"][t], dev["a"][t],
                                  dev["b"][t], o)
            og = o.cpu().numpy()
            assert np.isfinite(og).all(), name
            worst_o = max(worst_o, rel_l2(og, o_tf[t]))
        gi, gv = gpu.comp_to_host()
        same = token_sets_agree(gi.reshape(-1, m), gv.reshape(-1, m),
                                tf.tok_idx.reshape(-1, m), tf.tok_val.reshape(-1, m), name)
        if not same:
            ties += 1
            continue
        g = gpu_to_oracle(gpu, bits)
        lsb, frac = compare_codes(g.packed, tf.packed, tf)
        worst_lsb, worst_flip = max(worst_lsb, lsb), max(worst_flip, frac)
        assert np.allclose(g.row_scale, tf.row_scale, rtol=1e-5, atol=0), name
        assert np.allclose(g.col_scale, tf.col_scale, rtol=1e-5, atol=0), name
    drift = rel_l2(gpu.comp_dequantize().cpu().numpy(), ref.comp_dequantize())
    print(f"[{name}] windows={n_windows} W={W} m={m} worst o rel-L2 tf={worst_o:.2e} "
          f"worst flips tf={worst_flip:.2e} (max {worst_lsb} LSB) near-tie windows={ties} "
          f"drift={drift:.2e}", flush=True)
    assert worst_o <= O_REL_L2, name
    assert worst_lsb <= 1 and worst_flip <= CODE_FLIP_FRAC, name
    assert ties < n_windows, name
    assert drift <= DRIFT_REL_L2, name


def test_comp_window_kda_8bit_prewarmed(torch_cuda):
    w = wl.WORKLOADS[4]
    n_req = 2
    S0 = spikes(prewarmed_state(w, n_req), 15)
    run_comp_windows(torch_cuda, w, n_req, w.n_head, bits_for(w), 16, w.window, 2, S0,
                     "comp window kda 8-bit W=64")


def test_comp_window_gdn_mixed_widths(torch_cuda):
    w = wl.WORKLOADS[1]
    H = 8
    rng = np.random.default_rng(16)
    S0 = spikes((0.1 * rng.standard_normal((1, H, 128, 128))).astype(np.float32), 17)
    run_comp_windows(torch_cuda, w, 1, H, bits_for(w, n_head=H), 64, 16, 3, S0,
                     "comp window gdn mixed W=16 m=64")


def test_comp_window_m0_is_the_plain_window(torch_cuda):
    from quantized_delta_rule_03_amd import qdr

    w = wl.WORKLOADS[2]
    H, W = 4, 12
    bits = bits_for(w, n_head=H)
    rng = np.random.default_rng(18)
    S0 = (0.1 * rng.standard_normal((1, H, 128, 128))).astype(np.float32)
    toks = [to_dev({k: np.ascontiguousarray(v[:, :H]) for k, v in
                    wl.step_inputs(w, t, n_req=1).items()}) for t in range(W)]
    outs = []
    for comp in (False, True):
        gpu = qdr.StatePool(1, H, w.gate, bits, window=W)
        gpu.quantize(torch_cuda.from_numpy(S0).cuda())
        o = torch_cuda.empty((1, H, 128), dtype=torch_cuda.float32, device="cuda")
        if comp:
            gpu.comp_enable(0)
        got = []
        for t in range(W):
            x = toks[t]
            if comp:
                gpu.comp_window_token(t, x["q"], x["k"], x["v"], x["a"], x["b"], o)
            else:
                gpu.window_token(t, x["q"], x["k"], x["v"], x["a"], x["b"], o)
            got.append(o.cpu().numpy())
        outs.append((np.stack(got), *gpu.to_host()))
    for x, y in zip(*outs):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))
