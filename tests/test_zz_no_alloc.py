"""qdr_decode_window_static (window mode with the library's own static window buffer, for
callers that cannot allocate) against qdr_decode_window with a caller buffer: the same
kernels on the same inputs, so every readout, code and scale must agree bit for bit. Two
windows in a row, the second on a smaller pool, so the second reuses the static buffer
that the first one left behind; plus the size limit and a refused oversize pool (GPU)."""
import numpy as np
import pytest

from quantized_delta_rule_03_amd import qdr
from quantized_delta_rule_03_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qdr.lib()
    return torch


def run_window(torch, n_req, W, seed, static):
    w = wl.WORKLOADS[2]
    n_head = 8
    bits = np.ascontiguousarray(qdr.assign_bits(w.gate, wl.halflives(w)[:n_head]))
    pool = qdr.StatePool(n_req, n_head, w.gate, bits, window=0 if static else W)
    L = qdr.Layout(n_req, n_head, w.gate, bits, window=W)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    pool.quantize(0.3 * torch.randn((n_req, n_head, 128, 128), generator=g, device="cuda"))
    a = torch.from_numpy(wl.static_gate(w, n_req=n_req)[:, :n_head].copy()).cuda()
    outs = []
    o = torch.empty((n_req, n_head, 128), dtype=torch.float32, device="cuda")
    for t in range(W):
        x = {k: v[:, :n_head].contiguous()
             for k, v in wl.device_step_inputs(w, 100 * seed + t, "cuda", seed).items()}
        x = {k: v[:n_req].contiguous() for k, v in x.items()}
        if static:
            qdr.decode_window_static(L, pool.meta, pool.packed, pool.row_scale, pool.col_scale,
                                     t, x["q"], x["k"], x["v"], a, x["b"], o)
        else:
            qdr.decode_window(L, pool.meta, pool.packed, pool.row_scale, pool.col_scale,
                              pool.window_buf, t, x["q"], x["k"], x["v"], a, x["b"], o)
        outs.append(o.cpu().numpy())
    packed, R, c = pool.to_host()
    return np.stack(outs), packed, R, c


@pytest.mark.parametrize("calls", [[(6, 16, 1), (3, 16, 2)], [(4, 64, 3), (2, 8, 4)]])
def test_static_window_matches_caller_buffer(torch_cuda, calls):
    for n_req, W, seed in calls:  # the second window runs on a smaller pool
        o_s, p_s, R_s, c_s = run_window(torch_cuda, n_req, W, seed, static=True)
        o_c, p_c, R_c, c_c = run_window(torch_cuda, n_req, W, seed, static=False)
        print(f"[static window] n_req={n_req} W={W}: readouts, codes and scales bit-identical="
              f"{np.array_equal(o_s.view(np.uint32), o_c.view(np.uint32)) and np.array_equal(p_s, p_c)}",
              flush=True)
        assert np.array_equal(o_s.view(np.uint32), o_c.view(np.uint32))
        assert np.array_equal(p_s, p_c)
        assert np.array_equal(R_s.view(np.uint32), R_c.view(np.uint32))
        assert np.array_equal(c_s.view(np.uint32), c_c.view(np.uint32))


def test_static_window_refuses_an_oversize_pool(torch_cuda):
    bits = wl.uniform_bits(32, 8)
    L = qdr.Layout(16, 32, qdr.KDA, bits, window=64)  # 512 units x 66,048 B > 32 MiB
    meta = torch_cuda.empty(L.meta_bytes, dtype=torch_cuda.uint8, device="cuda")
    buf = torch_cuda.empty(16, dtype=torch_cuda.float32, device="cuda")
    with pytest.raises(qdr.QdrError) as e:
        qdr.decode_window_static(L, meta, buf, buf, buf, 0, buf, buf, buf, buf, buf, buf)
    assert e.value.code == qdr.QDR_EUNSUPPORTED
    assert "static" in str(e.value)
