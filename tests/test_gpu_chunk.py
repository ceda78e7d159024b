"""GPU parity of chunk mode (qdr_decode_chunk) against the oracle's window reference.

qdr_decode_chunk takes T known tokens at once; its result is defined as that of one
window of W = T tokens: the oracle dequantizes the state, runs the exact recurrence in
fp64 over the T tokens (o_t = S_t q_t) and requantizes once at the end. The GPU carries
an fp32 state through sub-blocks of 16 tokens (matrix-core products with three-part bf16
operands, running gate products, a per-row triangular solve). Bar (as for the decode
step and window mode): every token's readout rel-L2 <= 1e-4; codes after each chunk,
teacher-forced (oracle started from the GPU's own state), within 1 LSB on <= 1e-4 of
entries, scales to 1e-5; free-running dequantized-state drift <= 1e-3.
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


def chunk_inputs(w, t0, T, n_req, n_head, gate_fn=None):
    toks = []
    for t in range(T):
        inp = wl.step_inputs(w, t0 + t, n_req=n_req)
        inp = {k: np.ascontiguousarray(v[:, :n_head]) for k, v in inp.items()}
        if gate_fn is not None:
            inp["a"] = gate_fn(t0 + t, inp["a"])
        toks.append(inp)
    return {k: np.ascontiguousarray(np.stack([x[k] for x in toks])) for k in toks[0]}


def run_chunks(torch, w, n_req, n_head, bits, T, n_chunks, S0, name, gate_fn=None):
    from quantized_delta_rule_03_amd import qdr

    gpu = qdr.StatePool(n_req, n_head, w.gate, bits)
    ref = oracle.Pool(n_req, n_head, bits)
    ref.quantize(S0)
    gpu.load_host(ref.packed, ref.row_scale, ref.col_scale)
    worst_o, worst_flip, worst_lsb, worst_o_free = 0.0, 0.0, 0, 0.0
    for c in range(n_chunks):
        stack = chunk_inputs(w, c * T, T, n_req, n_head, gate_fn)
        print(f"[{name}] chunk {c}: T={T} n_req={n_req} n_head={n_head}", flush=True)
        tf = gpu_to_oracle(gpu, bits)  # teacher-forced: the GPU's state at the chunk start
        o_tf = tf.window(w.gate, stack["q"], stack["k"], stack["v"], stack["a"], stack["b"])
        o_free = ref.window(w.gate, stack["q"], stack["k"], stack["v"], stack["a"], stack["b"])
        dev = to_dev(stack)
        o = torch.full((T, n_req, n_head, 128), float("nan"), dtype=torch.float32, device="cuda")
        gpu.chunk(dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], o)
        og = o.cpu().numpy()
        assert np.isfinite(og).all(), name
        for t in range(T):
            worst_o = max(worst_o, rel_l2(og[t], o_tf[t]))
            worst_o_free = max(worst_o_free, rel_l2(og[t], o_free[t]))
        g = gpu_to_oracle(gpu, bits)
        lsb, frac = compare_codes(g.packed, tf.packed, tf)
        worst_lsb, worst_flip = max(worst_lsb, lsb), max(worst_flip, frac)
        assert np.allclose(g.row_scale, tf.row_scale, rtol=1e-5, atol=0), name
        assert np.allclose(g.col_scale, tf.col_scale, rtol=1e-5, atol=0), name
    drift = rel_l2(gpu_to_oracle(gpu, bits).dequantize(), ref.dequantize())
    print(f"[{name}] chunks={n_chunks} T={T} worst o rel-L2 tf={worst_o:.2e} "
          f"free={worst_o_free:.2e} worst flips tf={worst_flip:.2e} (max {worst_lsb} LSB) "
          f"drift={drift:.2e}", flush=True)
    assert worst_o <= O_REL_L2, name
    assert worst_lsb <= 1 and worst_flip <= CODE_FLIP_FRAC, name
    assert drift <= DRIFT_REL_L2, name


def test_chunk_kda_8bit_prewarmed(torch_cuda):
    """Windowed serving shape (KDA, 8-bit, T = 64, pre-warmed outlier states) on a
    request subset: units are independent, so subset parity is parity for those units."""
    w = wl.WORKLOADS[4]
    n_req = 2
    bits = bits_for(w)
    S0 = prewarmed_state(w, n_req)
    run_chunks(torch_cuda, w, n_req, w.n_head, bits, w.window, 2, S0, "kda 8-bit T=64")


def test_chunk_gdn_mixed_widths(torch_cuda):
    w = wl.WORKLOADS[1]
    bits = bits_for(w)
    run_chunks(torch_cuda, w, 1, w.n_head, bits, 40, 3,
               np.zeros((1, w.n_head, 128, 128), np.float32), "gdn mixed T=40")


def test_chunk_kda_mixed_widths_prewarmed(torch_cuda):
    w = wl.WORKLOADS[2]
    bits = bits_for(w, n_head=8)
    S0 = prewarmed_state(w, 1)[:, :8]
    run_chunks(torch_cuda, w, 1, 8, bits, 64, 2, np.ascontiguousarray(S0), "kda mixed T=64")


@pytest.mark.parametrize("width", [4, 6])
def test_chunk_single_width_pools(torch_cuda, width):
    """Pools whose heads all have one width other than 8 (tile offsets then follow from
    the unit index alone), several requests and an odd head count."""
    w = wl.WORKLOADS[1]
    n_req, n_head = 3, 5
    bits = wl.uniform_bits(n_head, width)
    rng = np.random.default_rng(20 + width)
    S0 = (0.1 * rng.standard_normal((n_req, n_head, 128, 128))).astype(np.float32)
    run_chunks(torch_cuda, w, n_req, n_head, bits, 20, 2, S0, f"gdn {width}-bit T=20")


@pytest.mark.parametrize("T", [1, 15, 17, 100])
def test_chunk_lengths(torch_cuda, T):
    """One token, sub-block edges, and a chunk longer than the serving window."""
    w = wl.WORKLOADS[2]
    bits = bits_for(w, n_head=4)
    rng = np.random.default_rng(5)
    S0 = (0.1 * rng.standard_normal((1, 4, 128, 128))).astype(np.float32)
    run_chunks(torch_cuda, w, 1, 4, bits, T, 2, S0, f"kda mixed T={T}")


def test_chunk_extreme_gates(torch_cuda):
    """Gates of exactly 0 and 1 and tiny values (products far below the fp32 range over
    a sub-block): the decay factors are running products, so nothing overflows."""
    w = wl.WORKLOADS[2]
    bits = bits_for(w, n_head=4)
    rng = np.random.default_rng(9)
    S0 = (0.1 * rng.standard_normal((1, 4, 128, 128))).astype(np.float32)

    def gates(t, a):
        g = np.random.default_rng(1000 + t)
        x = a.copy()
        x[..., : 16] = 1e-30                      # tiny on some channels
        x[..., 16:24] = 0.0 if t % 5 == 0 else 1.0  # resets and no decay
        x[..., 24:32] = g.uniform(0.0, 1e-3, size=x[..., 24:32].shape).astype(np.float32)
        return x.astype(np.float32)

    run_chunks(torch_cuda, w, 1, 4, bits, 48, 2, S0, "kda extreme gates T=48", gates)


def test_chunk_zero_tokens_and_requests_are_noops(torch_cuda):
    from quantized_delta_rule_03_amd import qdr

    w = wl.WORKLOADS[4]
    gpu = qdr.StatePool(1, 4, w.gate, bits_for(w, n_head=4))
    before = gpu.to_host()
    e = torch_cuda.empty((0,), device="cuda")
    gpu.chunk(e, e, e, e, e, e)
    torch_cuda.cuda.synchronize()
    after = gpu.to_host()
    assert all(np.array_equal(x, y) for x, y in zip(before, after))
    gpu0 = qdr.StatePool(0, 4, w.gate, bits_for(w, n_head=4))
    b = torch_cuda.zeros((8, 0, 4), device="cuda")
    gpu0.chunk(e, e, e, e, b, e)
    torch_cuda.cuda.synchronize()
