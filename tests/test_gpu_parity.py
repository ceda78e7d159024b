"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded
inputs. Bar: codes within 1 LSB on <= 1e-4 of entries, o rel-L2 <= 1e-4 per step,
dequantized-state drift <= 1e-3 rel-L2 after 256 free-running steps. The arithmetic
contract is shared, so in practice everything is expected to match bit for bit; the
tests assert the bar and report exactness."""
import numpy as np
import pytest

import oracle
from parity_tools import (CODE_FLIP_FRAC, DRIFT_REL_L2, O_REL_L2, Trajectory, bits_for,
                          compare_codes, gpu_to_oracle, prewarmed_state, rel_l2, to_dev)
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


def make_pool(n_req, n_head, gate, bits, window=0):
    from quantized_delta_rule_03_amd import qdr

    return qdr.StatePool(n_req, n_head, gate, bits, window)


def report(name, traj):
    print(f"[{name}] steps={traj.steps} worst o rel-L2 tf={traj.worst_o_tf:.2e} "
          f"free={traj.worst_o_free:.2e} worst flips tf={traj.worst_flip_tf:.2e} "
          f"(max {traj.worst_lsb_tf} LSB)", flush=True)


# ---------------------------------------------------------------------------
# init / quantize / dequantize: bit-exact format and scale rule
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("gate", [0, 1])
def test_init_is_quantized_zero(torch_cuda, gate):
    rng = np.random.default_rng(0)
    if gate == 0:
        bits = oracle.assign_bits(0, np.exp(rng.uniform(0, 8, 8)), 128)
    else:
        bits = oracle.assign_bits(1, np.exp(rng.uniform(0, 9, (8, 128))), 128)
    gpu = make_pool(3, 8, gate, bits)
    torch_cuda.cuda.synchronize()
    ref = oracle.Pool(3, 8, bits)
    ref.quantize(np.zeros((3, 8, 128, 128), np.float32))
    packed, R, c = gpu.to_host()
    assert np.array_equal(packed, ref.packed)
    assert np.array_equal(R, ref.row_scale) and np.array_equal(c, ref.col_scale)


@pytest.mark.parametrize("gate,n_head", [(0, 8), (1, 4), (0, 3)])
def test_quantize_and_dequantize_bit_exact(torch_cuda, gate, n_head):
    rng = np.random.default_rng(1 + gate)
    if gate == 0:
        bits = oracle.assign_bits(0, np.exp(rng.uniform(0, 8, n_head)), 128)
        if n_head == 3:  # one head of each width
            bits = np.stack([np.full(128, b, np.uint8) for b in (4, 6, 8)])
    else:
        bits = oracle.assign_bits(1, np.exp(rng.uniform(0, 9, (n_head, 128))), 128)
    n_req = 5
    S = rng.standard_normal((n_req, n_head, 128, 128)).astype(np.float32)
    S[:, :, rng.uniform(size=128) < 0.02, :] *= 40.0
    S[:, :, :, rng.uniform(size=128) < 0.02] *= 40.0
    S[0, 0, 7, :] = 0.0  # zero value row
    S[1, 0, :, 9] = 0.0  # zero key row
    S[2, 0] = 0.0        # zero unit
    gpu = make_pool(n_req, n_head, gate, bits)
    gpu.quantize(torch_cuda.from_numpy(S).cuda())
    ref = oracle.Pool(n_req, n_head, bits)
    ref.quantize(S)
    packed, R, c = gpu.to_host()
    assert np.array_equal(R, ref.row_scale)
    assert np.array_equal(c, ref.col_scale)
    assert np.array_equal(packed, ref.packed)
    Sd = gpu.dequantize().cpu().numpy()
    assert np.array_equal(Sd, ref.dequantize())


# ---------------------------------------------------------------------------
# decode step, workload by workload
# ---------------------------------------------------------------------------

def run_workload(torch_cuda, wid, n_req, steps, S0=None, teacher_forced=True, name=None):
    w = wl.WORKLOADS[wid]
    bits = bits_for(w)
    gpu = make_pool(n_req, w.n_head, w.gate, bits)
    ref = oracle.Pool(n_req, w.n_head, bits)
    if S0 is None:
        ref.quantize(np.zeros((n_req, w.n_head, 128, 128), np.float32))
    else:
        ref.quantize(S0)
        gpu.load_host(ref.packed, ref.row_scale, ref.col_scale)
    g0 = gpu_to_oracle(gpu, bits)
    assert np.array_equal(g0.packed, ref.packed)
    traj = Trajectory(gpu, ref, w.gate)
    for t in range(steps):
        traj.step(wl.step_inputs(w, t, n_req=n_req), teacher_forced=teacher_forced)
    report(name or w.name, traj)
    return traj


def assert_bar(traj, drift=True):
    assert traj.worst_o_tf <= O_REL_L2
    assert traj.worst_lsb_tf <= 1 and traj.worst_flip_tf <= CODE_FLIP_FRAC
    assert traj.worst_o_free <= O_REL_L2
    if drift:
        d = traj.drift()
        lsb, frac = traj.free_codes()
        print(f"   free-running: drift rel-L2 {d:.2e}, code flips {frac:.2e} (max {lsb} LSB)")
        assert d <= DRIFT_REL_L2


def test_workload0_single_head_8bit(torch_cuda):
    """Single GDN head, 8-bit, zero start, 64 steps, per-step gate exp(-softplus(x))."""
    traj = run_workload(torch_cuda, 0, 1, 64)
    assert_bar(traj)


def test_workload1_gdn_mixed_subset(torch_cuda):
    """GDN, 32 heads with lifetime-quartile 8/6/4 bits, 256 steps (2 of 64 requests;
    units are independent, so these are exact parity for those units)."""
    traj = run_workload(torch_cuda, 1, 2, 256)
    assert_bar(traj)


def test_workload2_kda_prewarmed_subset(torch_cuda):
    """KDA per-channel gate, mixed bits per key channel, pre-warmed states with outlier
    rows and columns, 256 steps (1 of 256 requests)."""
    w = wl.WORKLOADS[2]
    S0 = prewarmed_state(w, 1)
    med = np.median(np.abs(S0), axis=(2, 3), keepdims=True)
    print(f"   pre-warm: fraction of entries > 10x unit median |S|: "
          f"{float((np.abs(S0) > 10 * med).mean()):.2e}")
    traj = run_workload(torch_cuda, 2, 1, 256, S0=S0)
    assert_bar(traj)


def test_workload3_full_size_sampled(torch_cuda):
    """Serving scale: 1024 requests x 32 heads in one launch per step (the benchmark's
    launch), 3 steps; six requests spread over the pool (192 units) checked against the
    oracle, plus the aggregate invariants of every unit."""
    torch = torch_cuda
    w = wl.WORKLOADS[3]
    bits = bits_for(w)
    gpu = make_pool(w.n_req, w.n_head, w.gate, bits)
    sample = [0, 173, 511, 512, 777, 1023]
    ref = oracle.Pool(len(sample), w.n_head, bits)
    ref.quantize(np.zeros((len(sample), w.n_head, 128, 128), np.float32))
    o = torch.empty((w.n_req, w.n_head, 128), dtype=torch.float32, device="cuda")
    worst_o = 0.0
    for t in range(3):
        inp = wl.step_inputs(w, t)
        dev = to_dev(inp)
        gpu.step(dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], o)
        sub = {k: v[sample] for k, v in inp.items()}
        o_ref = ref.step_threads(w.gate, sub["q"], sub["k"], sub["v"], sub["a"], sub["b"])
        o_gpu = o.cpu().numpy()[sample]
        worst_o = max(worst_o, rel_l2(o_gpu, o_ref))
        packed, R, c = gpu.to_host()
        lsb, frac = compare_codes(packed[sample], ref.packed, ref)
        assert lsb <= 1 and frac <= CODE_FLIP_FRAC
        np.testing.assert_allclose(R[sample], ref.row_scale, rtol=1e-6)
        np.testing.assert_allclose(c[sample], ref.col_scale, rtol=1e-6)
    print(f"[serving full size] worst o rel-L2 {worst_o:.2e}")
    assert worst_o <= O_REL_L2
    # every unit: the full code range is used in each non-zero key row (scale rule)
    Sd = gpu.dequantize()
    assert torch.isfinite(Sd).all()
    assert torch.isfinite(o).all()


# ---------------------------------------------------------------------------
# edge cases and determinism
# ---------------------------------------------------------------------------

def test_zero_requests_is_noop(torch_cuda):
    from quantized_delta_rule_03_amd import qdr

    bits = wl.uniform_bits(2, 6)
    L = qdr.Layout(0, 2, 0, bits)
    assert L.packed_bytes == 0
    torch = torch_cuda
    meta = torch.empty(L.meta_bytes, dtype=torch.uint8, device="cuda")
    qdr.init_state(L, None, None, None, meta)
    qdr.decode_step(L, meta, None, None, None, None, None, None, None, None, None)
    torch.cuda.synchronize()


def test_mixed_width_heads_and_special_inputs(torch_cuda):
    """A request with one head of each width plus KDA-style special inputs: b = 0 and
    a = 1 (state unchanged), k = 0 (pure decay), huge outliers."""
    torch = torch_cuda
    bits = np.stack([np.full(128, b, np.uint8) for b in (4, 6, 8)])
    rng = np.random.default_rng(9)
    n_req = 4
    S0 = rng.standard_normal((n_req, 3, 128, 128)).astype(np.float32)
    S0[1, :, 3, :] *= 1000.0
    gpu = make_pool(n_req, 3, 0, bits)
    ref = oracle.Pool(n_req, 3, bits)
    ref.quantize(S0)
    gpu.load_host(ref.packed, ref.row_scale, ref.col_scale)
    traj = Trajectory(gpu, ref, 0)
    for t in range(6):
        k = rng.standard_normal((n_req, 3, 128))
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        inp = {"q": rng.standard_normal((n_req, 3, 128)).astype(np.float32),
               "k": k.astype(np.float32),
               "v": rng.standard_normal((n_req, 3, 128)).astype(np.float32),
               "a": rng.uniform(0.5, 1, (n_req, 3)).astype(np.float32),
               "b": rng.uniform(0, 1, (n_req, 3)).astype(np.float32)}
        inp["a"][0] = 1.0
        inp["b"][0] = 0.0
        inp["k"][2] = 0.0
        before = gpu_to_oracle(gpu, bits)
        traj.step(inp)
        after = gpu_to_oracle(gpu, bits)
        lsb, frac = compare_codes(after.packed[:1], before.packed[:1], oracle.Pool(1, 3, bits))
        assert lsb == 0  # a = 1, b = 0: codes unchanged
    report("mixed heads / special inputs", traj)
    assert traj.worst_o_tf <= O_REL_L2 and traj.worst_lsb_tf <= 1
    assert traj.worst_flip_tf <= CODE_FLIP_FRAC


def test_gdn_heads_with_mixed_channel_widths(torch_cuda):
    """GDN gate on heads whose key channels have mixed widths (a per-channel bit map): the
    physical key order of such a head is not the logical one, so the step must read k, q
    through the head's position map, as quantize and dequantize do."""
    rng = np.random.default_rng(23)
    n_head, n_req = 4, 3
    bits = oracle.assign_bits(1, np.exp(rng.uniform(0, 9, (n_head, 128))), 128)
    S0 = rng.standard_normal((n_req, n_head, 128, 128)).astype(np.float32)
    gpu = make_pool(n_req, n_head, 0, bits)
    ref = oracle.Pool(n_req, n_head, bits)
    ref.quantize(S0)
    gpu.load_host(ref.packed, ref.row_scale, ref.col_scale)
    traj = Trajectory(gpu, ref, 0)
    for t in range(8):
        k = rng.standard_normal((n_req, n_head, 128))
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q = rng.standard_normal((n_req, n_head, 128))
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        inp = {"q": q.astype(np.float32), "k": k.astype(np.float32),
               "v": rng.standard_normal((n_req, n_head, 128)).astype(np.float32),
               "a": rng.uniform(0.5, 1, (n_req, n_head)).astype(np.float32),
               "b": rng.uniform(0, 1, (n_req, n_head)).astype(np.float32)}
        traj.step(inp)
    report("gdn, mixed channel widths", traj)
    assert_bar(traj)


def test_sparse_and_tiny_keys_and_queries(torch_cuda):
    """Keys and queries with whole zero segments, single nonzero positions and values down
    to fp32 subnormals next to normal ones in one segment: the per-segment fixed-point
    scale of the exact dot products must keep every term the fp32 results can see."""
    bits = np.stack([np.full(128, b, np.uint8) for b in (4, 6, 8)])
    rng = np.random.default_rng(17)
    n_req = 3
    S0 = rng.standard_normal((n_req, 3, 128, 128)).astype(np.float32)
    gpu = make_pool(n_req, 3, 0, bits)
    ref = oracle.Pool(n_req, 3, bits)
    ref.quantize(S0)
    gpu.load_host(ref.packed, ref.row_scale, ref.col_scale)
    traj = Trajectory(gpu, ref, 0)
    for t in range(6):
        k = rng.standard_normal((n_req, 3, 128)).astype(np.float32)
        q = rng.standard_normal((n_req, 3, 128)).astype(np.float32)
        # request 0: segments 0-1 zero; segment 2 mixes 1, 1e-30 and subnormals
        k[0, :, :64] = 0.0
        k[0, :, 64:70] = [1.0, 1e-30, 1e-40, -3e-39, 1e-20, -1.0]
        q[0, :, :32] = 0.0
        q[0, :, 32:36] = [1e-38, -1e-44, 5e-39, 1.0]
        # request 1: one nonzero key per segment, a query spanning 1e-20 .. 1e3
        k[1] = 0.0
        for pos, val in ((5, 0.5), (40, -1e-12), (77, 0.25), (120, 3e-8)):
            k[1, :, pos] = val
        q[1] = (q[1] * np.logspace(-20, 3, 128)).astype(np.float32)
        nrm = np.linalg.norm(k.astype(np.float64), axis=-1, keepdims=True)
        k = np.where(nrm > 0, k / np.maximum(nrm, 1e-300), k).astype(np.float32)
        inp = {"q": q, "k": k,
               "v": rng.standard_normal((n_req, 3, 128)).astype(np.float32),
               "a": rng.uniform(0.5, 1, (n_req, 3)).astype(np.float32),
               "b": rng.uniform(0, 1, (n_req, 3)).astype(np.float32)}
        traj.step(inp)
    report("sparse / tiny keys and queries", traj)
    assert traj.worst_o_tf <= O_REL_L2 and traj.worst_lsb_tf <= 1
    assert traj.worst_flip_tf <= CODE_FLIP_FRAC


def test_deterministic(torch_cuda):
    torch = torch_cuda
    w = wl.WORKLOADS[1]
    bits = bits_for(w)
    outs = []
    for rep in range(2):
        gpu = make_pool(4, w.n_head, w.gate, bits)
        o = torch.empty((4, w.n_head, 128), dtype=torch.float32, device="cuda")
        for t in range(5):
            dev = to_dev(wl.step_inputs(w, t, n_req=4))
            gpu.step(dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], o)
        outs.append((gpu.to_host(), o.cpu().numpy()))
    (p0, r0, c0), o0 = outs[0]
    (p1, r1, c1), o1 = outs[1]
    assert np.array_equal(p0, p1) and np.array_equal(r0, r1) and np.array_equal(c0, c1)
    assert np.array_equal(o0, o1)
