"""The decode step and chunk mode under HIP graph capture (GPU).

Every entry point launches its kernels on the caller's stream and neither allocates nor
synchronizes nor clears memory, so a caller can capture a run of decode steps (or chunk
calls) once and replay it. Checked: several replays of a captured sequence, with eager
readbacks and synchronizations between them, give bit for bit the state and readouts of
the same calls made eagerly.
"""
import numpy as np
import pytest

import oracle
from parity_tools import bits_for, prewarmed_state, to_dev
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


def fresh_pool(torch, w, n_req, n_head, bits, S0):
    from quantized_delta_rule_03_amd import qdr

    ref = oracle.Pool(n_req, n_head, bits)
    ref.quantize(S0)
    gpu = qdr.StatePool(n_req, n_head, w.gate, bits)
    gpu.load_host(ref.packed, ref.row_scale, ref.col_scale)
    return gpu


def state_of(gpu):
    return [x.copy() for x in gpu.to_host()]


def test_captured_decode_steps_replay_like_eager_steps(torch_cuda):
    torch = torch_cuda
    w = wl.WORKLOADS[3]
    n_req, H, n_steps, replays = 4, w.n_head, 6, 3
    bits = bits_for(w)
    rng = np.random.default_rng(21)
    S0 = (0.1 * rng.standard_normal((n_req, H, 128, 128))).astype(np.float32)
    inputs = [to_dev(wl.step_inputs(w, t, n_req=n_req)) for t in range(n_steps)]
    eager = fresh_pool(torch, w, n_req, H, bits, S0)
    graph_pool = fresh_pool(torch, w, n_req, H, bits, S0)
    outs = [torch.empty((n_req, H, 128), dtype=torch.float32, device="cuda")
            for _ in range(n_steps)]
    # one eager call first (library set-up outside the capture), then the same on both
    graph_pool.step(**{k: inputs[0][k] for k in "qkvab"}, o=outs[0])
    eager.step(**{k: inputs[0][k] for k in "qkvab"}, o=outs[0])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(n_steps):
            graph_pool.step(**{k: inputs[t][k] for k in "qkvab"}, o=outs[t])
    print(f"[graph] captured {n_steps} decode steps, n_req={n_req} n_head={H}", flush=True)
    o_ref = torch.empty((n_req, H, 128), dtype=torch.float32, device="cuda")
    for r in range(replays):
        g.replay()
        torch.cuda.synchronize()
        got_o = [o.cpu().numpy() for o in outs]
        got = state_of(graph_pool)
        graph_pool.dequantize()  # eager work between replays
        for t in range(n_steps):
            eager.step(**{k: inputs[t][k] for k in "qkvab"}, o=o_ref)
            torch.cuda.synchronize()
            assert np.array_equal(o_ref.cpu().numpy().view(np.uint32),
                                  got_o[t].view(np.uint32)), (r, t)
        for x, y in zip(got, state_of(eager)):
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), r
        print(f"[graph] replay {r}: state and {n_steps} readouts bit-identical", flush=True)


def test_captured_chunks_replay_like_eager_chunks(torch_cuda):
    torch = torch_cuda
    w = wl.WORKLOADS[4]
    n_req, H, T, replays = 1, 8, 40, 3
    bits = bits_for(w, n_head=H)
    S0 = np.ascontiguousarray(prewarmed_state(w, n_req)[:, :H])
    toks = [wl.step_inputs(w, t, n_req=n_req) for t in range(T)]
    stack = to_dev({k: np.ascontiguousarray(np.stack([x[k][:, :H] for x in toks]))
                    for k in toks[0]})
    eager = fresh_pool(torch, w, n_req, H, bits, S0)
    graph_pool = fresh_pool(torch, w, n_req, H, bits, S0)
    o_g = torch.empty((T, n_req, H, 128), dtype=torch.float32, device="cuda")
    o_e = torch.empty_like(o_g)
    args = {k: stack[k] for k in "qkvab"}
    graph_pool.chunk(**args, o=o_g)
    eager.chunk(**args, o=o_e)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graph_pool.chunk(**args, o=o_g)
    print(f"[graph] captured one chunk call, T={T} n_head={H}", flush=True)
    for r in range(replays):
        g.replay()
        torch.cuda.synchronize()
        got_o = o_g.cpu().numpy()
        graph_pool.dequantize()
        eager.chunk(**args, o=o_e)
        torch.cuda.synchronize()
        assert np.array_equal(got_o.view(np.uint32), o_e.cpu().numpy().view(np.uint32)), r
        for x, y in zip(state_of(graph_pool), state_of(eager)):
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), r
        print(f"[graph] chunk replay {r}: state and readouts bit-identical", flush=True)
