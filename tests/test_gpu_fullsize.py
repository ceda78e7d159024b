"""Parity at the benchmark's full sizes and launch configurations, on sampled units (GPU).

The GPU runs the whole pool in the launches bench.py times; a few requests spread over the
pool (every head of each) are compared with the oracle, which computes only those units.
Units are independent, so this is parity for the sampled units at full scale (addressing,
grid and persistence over the whole pool included).

* chunk mode and chunk mode with 16 compensator tokens, 256 requests x 32 KDA heads,
  8-bit, one call of T = 64 tokens;
* window mode, the same shape, one window of W = 64 token calls and the fold;
* the DAMP-style variant, 1024 requests x 32 GDN heads, two steps from the initial state
  (the stochastic rounding is keyed by the unit index, which the sample keeps).

Inputs: full-size tensors drawn on the device by the seeded generator, with the sampled
requests' slices overwritten by the host generator's values for those requests (so the
oracle reads exactly what the GPU reads); the initial state is the oracle's quantization
of a seeded Gaussian state for the sampled requests.
"""
import numpy as np
import pytest

import oracle
from parity_tools import (CODE_FLIP_FRAC, O_REL_L2, bits_for, compare_codes, gpu_to_oracle,
                          rel_l2)
from quantized_delta_rule_03_amd import workloads as wl

pytestmark = pytest.mark.gpu

SAMPLE4 = [0, 97, 255]              # requests of the 256-request windowed shape
SAMPLE3 = [0, 1, 511, 1023]         # requests of the 1024-request serving shape


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_delta_rule_03_amd import qdr

    qdr.lib()
    return torch


def window_shape_inputs(torch, w, T, sample):
    """Token-major device inputs [T][n_req][n_head][...] and the sample's host copies."""
    dev = {k: [] for k in "qkvab"}
    host = {k: [] for k in "qkvab"}
    a_full = torch.from_numpy(wl.static_gate(w)).cuda()
    for t in range(T):
        d = wl.device_step_inputs(w, t, "cuda", seed=7)
        d["a"] = a_full.clone()
        for i, r in enumerate(sample):
            h = wl.step_inputs(w, t, n_req=1, r0=r)
            for k in "qkvab":
                d[k][r] = torch.from_numpy(np.ascontiguousarray(h[k][0])).cuda()
                if i == 0:
                    host[k].append([])
                host[k][t].append(h[k][0])
        for k in "qkvab":
            dev[k].append(d[k])
    dev = {k: torch.stack(v).contiguous() for k, v in dev.items()}
    host = {k: np.ascontiguousarray(np.stack([np.stack(x) for x in v])) for k, v in host.items()}
    return dev, host


def start_state(w, bits, sample, seed=31):
    rng = np.random.default_rng(seed)
    S0 = (0.1 * rng.standard_normal((len(sample), w.n_head, 128, 128))).astype(np.float32)
    ref = oracle.Pool(len(sample), w.n_head, bits)
    ref.quantize(S0)
    return S0, ref


def load_sample(gpu, ref, sample):
    """Full pool initialised, the sampled requests' slots set to the oracle's state."""
    packed, R, c = gpu.to_host()
    packed[sample] = ref.packed
    R[sample] = ref.row_scale
    c[sample] = ref.col_scale
    gpu.load_host(packed, R, c)


@pytest.mark.parametrize("m", [0, 16])
def test_chunk_full_size_sampled(torch_cuda, m):
    from quantized_delta_rule_03_amd import qdr

    torch = torch_cuda
    w = wl.WORKLOADS[4]
    T = w.window
    bits = bits_for(w)
    S0, ref = start_state(w, bits, SAMPLE4)
    if m:
        ref.comp_quantize(S0, m)
    dev, host = window_shape_inputs(torch, w, T, SAMPLE4)
    gpu = qdr.StatePool(w.n_req, w.n_head, w.gate, bits)
    load_sample(gpu, ref, SAMPLE4)
    if m:
        idx = np.full((w.n_req, w.n_head, m), oracle.TOK_EMPTY, np.uint16)
        val = np.zeros((w.n_req, w.n_head, m), np.float32)
        idx[SAMPLE4], val[SAMPLE4] = ref.tok_idx, ref.tok_val
        gpu.comp_load_host(idx, val)
    print(f"[full chunk m={m}] {w.n_req}x{w.n_head} units, T={T}, sample {SAMPLE4}", flush=True)
    o = torch.full((T, w.n_req, w.n_head, 128), float("nan"), device="cuda")
    if m:
        gpu.comp_chunk(dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], o)
        o_ref = ref.comp_window(w.gate, host["q"], host["k"], host["v"], host["a"], host["b"])
    else:
        gpu.chunk(dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], o)
        o_ref = ref.window(w.gate, host["q"], host["k"], host["v"], host["a"], host["b"])
    og = o.cpu().numpy()
    assert np.isfinite(og).all()
    worst = max(rel_l2(og[t][SAMPLE4], o_ref[t]) for t in range(T))
    g = gpu_to_oracle(gpu, bits)
    sub = oracle.Pool(len(SAMPLE4), w.n_head, bits)
    sub.packed[:], sub.row_scale[:], sub.col_scale[:] = (g.packed[SAMPLE4], g.row_scale[SAMPLE4],
                                                         g.col_scale[SAMPLE4])
    if m:
        gi, gv = gpu.comp_to_host()
        assert np.array_equal(gi[SAMPLE4], ref.tok_idx)
        assert rel_l2(gv[SAMPLE4], ref.tok_val) <= 1e-5
    lsb, frac = compare_codes(sub.packed, ref.packed, ref)
    print(f"[full chunk m={m}] worst o rel-L2 {worst:.2e}, codes max {lsb} LSB on "
          f"{frac:.2e}", flush=True)
    assert worst <= O_REL_L2
    assert lsb <= 1 and frac <= CODE_FLIP_FRAC
    np.testing.assert_allclose(sub.row_scale, ref.row_scale, rtol=1e-5)
    np.testing.assert_allclose(sub.col_scale, ref.col_scale, rtol=1e-5)


def test_window_full_size_sampled(torch_cuda):
    from quantized_delta_rule_03_amd import qdr

    torch = torch_cuda
    w = wl.WORKLOADS[4]
    W = w.window
    bits = bits_for(w)
    S0, ref = start_state(w, bits, SAMPLE4)
    dev, host = window_shape_inputs(torch, w, W, SAMPLE4)
    gpu = qdr.StatePool(w.n_req, w.n_head, w.gate, bits, window=W)
    load_sample(gpu, ref, SAMPLE4)
    print(f"[full window] {w.n_req}x{w.n_head} units, W={W}, sample {SAMPLE4}", flush=True)
    o = torch.empty((w.n_req, w.n_head, 128), device="cuda")
    og = []
    for t in range(W):
        gpu.window_token(t, dev["q"][t], dev["k"][t], dev["v"][t], dev["a"][t], dev["b"][t], o)
        og.append(o.cpu().numpy()[SAMPLE4])
    o_ref = ref.window(w.gate, host["q"], host["k"], host["v"], host["a"], host["b"])
    worst = max(rel_l2(og[t], o_ref[t]) for t in range(W))
    g = gpu_to_oracle(gpu, bits)
    lsb, frac = compare_codes(g.packed[SAMPLE4], ref.packed, ref)
    print(f"[full window] worst o rel-L2 {worst:.2e}, codes max {lsb} LSB on {frac:.2e}",
          flush=True)
    assert worst <= O_REL_L2
    assert lsb <= 1 and frac <= CODE_FLIP_FRAC
    np.testing.assert_allclose(g.row_scale[SAMPLE4], ref.row_scale, rtol=1e-5)
    np.testing.assert_allclose(g.col_scale[SAMPLE4], ref.col_scale, rtol=1e-5)


def test_damp_full_size_sampled(torch_cuda):
    from quantized_delta_rule_03_amd import qdr

    torch = torch_cuda
    w = wl.WORKLOADS[3]
    H = w.n_head
    sel = qdr.damp_select(w.gate, wl.halflives(w), H)
    gpu = qdr.DampState(w.n_req, H, w.gate, sel, seed=99)
    ref = oracle.DampPool(w.n_req, H, sel, seed=99)  # initial state: the zero state
    o = torch.empty((w.n_req, H, 128), device="cuda")
    units = [(r * H, (r + 1) * H) for r in SAMPLE3]
    print(f"[full damp] {w.n_req}x{H} units, sample {SAMPLE3}", flush=True)
    worst_o = 0.0
    for t in range(1, 3):
        inp = wl.step_inputs(w, t)
        dev = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in inp.items()}
        gpu.step(dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], o, step=t)
        o_ref = np.zeros_like(inp["v"])
        for u0, u1 in units:
            oo = ref.step(w.gate, inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], step=t,
                          u0=u0, u1=u1)
            o_ref[u0 // H] = oo[u0 // H]
        og = o.cpu().numpy()
        worst_o = max(worst_o, rel_l2(og[SAMPLE3], o_ref[SAMPLE3]))
    half, codes, R = gpu.to_host()
    n_flip = n_half = n_codes = 0
    exact = True
    for u0, u1 in units:
        d = np.abs(codes[u0:u1].astype(np.int32) - ref.codes[u0:u1].astype(np.int32))
        assert d.max() <= 1
        n_flip += int((d > 0).sum())
        n_codes += d.size
        n_half += int((half[u0:u1] != ref.half[u0:u1]).sum())
        np.testing.assert_allclose(R[u0:u1], ref.R[u0:u1], rtol=1e-6)
        exact = exact and not d.any() and np.array_equal(R[u0:u1].view(np.uint32),
                                                         ref.R[u0:u1].view(np.uint32))
    exact = exact and n_half == 0
    print(f"[full damp] worst o rel-L2 {worst_o:.2e}; codes differ on {n_flip / n_codes:.2e}, "
          f"binary16 values on {n_half} entries; bit-exact={exact}", flush=True)
    assert worst_o <= O_REL_L2
    assert n_flip / n_codes <= CODE_FLIP_FRAC
    assert n_half / n_codes <= CODE_FLIP_FRAC
