"""GPU parity of the DAMP-style storage variant (qdr_damp_*) against the oracle's DampPool.

The oracle takes the two dot products (u = S'k, o = S_new q) as one fp64 sum over the key
channels in logical order. The kernel sums the same exact fp64 products of u in its own
order, so u can differ in the last fp32 bit on rare rounding ties; it sums the readout o,
which feeds nothing back into the state, in fp32. Everything else (binary16
rounding, the per-row ranges, Philox4x32-7 stochastic rounding keyed by seed, unit and
step) is the same rule on both sides. The bar asserted is that of the main format (codes
within 1 LSB on <= 1e-4 of entries, o rel-L2 <= 1e-4, dequantized-state drift <= 1e-3);
bit-exactness is reported, not required.
"""
import numpy as np
import pytest

import oracle
from parity_tools import CODE_FLIP_FRAC, DRIFT_REL_L2, O_REL_L2, prewarmed_state, rel_l2, to_dev
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


def selection(w, n_head):
    from quantized_delta_rule_03_amd import qdr

    tau = wl.halflives(w)
    return qdr.damp_select(w.gate, tau[:n_head], n_head)


def to_oracle(gpu):
    p = oracle.DampPool(gpu.n_req, gpu.n_head, gpu.sel, seed=gpu.seed)
    p.half[:], p.codes[:], p.R[:] = gpu.to_host()
    return p


def compare(g, r):
    """(max |code diff|, fraction of codes that differ, binary16 bits equal, R equal)"""
    d = np.abs(g.codes.astype(np.int32) - r.codes.astype(np.int32))
    return int(d.max()), float((d > 0).mean()), np.array_equal(g.half, r.half), \
        np.array_equal(g.R, r.R)


def test_quantize_extreme_ranges_bit_exact(torch_cuda):
    """Key rows whose range leaves [2^-126, 2^126]: a subnormal range (1/A near 2^127) and
    a range near the fp32 maximum (1/A subnormal, so y can pass -1 and the clamp decides).
    Units with such a row take the clamped path, the others the unclamped one; both must
    match the oracle bit for bit."""
    from quantized_delta_rule_03_amd import qdr

    w = wl.WORKLOADS[2]
    n_req, H = 2, 4
    sel = selection(w, H)
    rng = np.random.default_rng(11)
    S = rng.standard_normal((n_req, H, 128, 128)).astype(np.float32)
    for h in (1, 3):
        int8_ch = np.flatnonzero(sel[h] == 0)
        tiny, huge = int8_ch[3], int8_ch[40]
        S[0, h, :, tiny] = (rng.uniform(-1.0, 1.0, 128) * 2.0 ** -127).astype(np.float32)
        S[0, h, 5, tiny] = np.float32(2.0 ** -127)
        S[0, h, 9, tiny] = 0.0
        # A = 2.4650119e38: fl(1/A) is subnormal and -A fl(1/A) rounds to -(1 + 2^-23),
        # so floor(127 y + u) reaches -128 for a zero random byte and is clamped
        big = np.float32(2.4650119e38)
        S[0, h, :, huge] = (rng.uniform(-1.0, 1.0, 128) * big).astype(np.float32)
        S[0, h, 20:120, huge] = -big
        S[0, h, 18, huge] = 0.0
    gpu = qdr.DampState(n_req, H, w.gate, sel, seed=9)
    ref = oracle.DampPool(n_req, H, sel, seed=9)
    for step in (3, 4, 5):
        gpu.quantize(torch_cuda.from_numpy(S).cuda(), step=step)
        ref.quantize(S, step=step)
        half, codes, R = gpu.to_host()
        assert np.array_equal(half, ref.half), step
        assert np.array_equal(codes, ref.codes), step
        assert np.array_equal(R, ref.R), step
        assert np.abs(codes.astype(np.int32)).max() <= 127


def test_init_and_quantize_bit_exact(torch_cuda):
    from quantized_delta_rule_03_amd import qdr

    w = wl.WORKLOADS[2]
    n_req, H = 2, 8
    sel = selection(w, H)
    gpu = qdr.DampState(n_req, H, w.gate, sel, seed=5)
    ref = oracle.DampPool(n_req, H, sel, seed=5)
    half, codes, R = gpu.to_host()
    assert np.all(half == 0) and np.all(codes == 0) and np.array_equal(R, ref.R)
    rng = np.random.default_rng(1)
    S = rng.standard_normal((n_req, H, 128, 128)).astype(np.float32)
    S[:, :, :, rng.uniform(size=128) < 0.03] *= 50.0
    S[0, 1, :, 7] = 0.0
    S[1, 2] = 0.0
    gpu.quantize(torch_cuda.from_numpy(S).cuda(), step=17)
    ref.quantize(S, step=17)
    half, codes, R = gpu.to_host()
    assert np.array_equal(half, ref.half)
    assert np.array_equal(codes, ref.codes)
    assert np.array_equal(R, ref.R)
    assert np.array_equal(gpu.dequantize().cpu().numpy(), ref.dequantize())


def run(torch_cuda, wid, n_req, n_head, steps, S0, name):
    from quantized_delta_rule_03_amd import qdr

    w = wl.WORKLOADS[wid]
    sel = selection(w, n_head)
    gpu = qdr.DampState(n_req, n_head, w.gate, sel, seed=1234)
    ref = oracle.DampPool(n_req, n_head, sel, seed=1234)
    ref.quantize(S0, step=0)
    gpu.load_host(ref.half, ref.codes, ref.R)
    o = torch_cuda.empty((n_req, n_head, 128), dtype=torch_cuda.float32, device="cuda")
    worst_o, worst_lsb, worst_flip, exact = 0.0, 0, 0.0, True
    for t in range(1, steps + 1):
        inp = wl.step_inputs(w, t, n_req=n_req)
        inp = {k: np.ascontiguousarray(v[:, :n_head]) for k, v in inp.items()}
        dev = to_dev(inp)
        tf = to_oracle(gpu)  # teacher-forced: the oracle steps from the GPU's state
        o_tf = tf.step(w.gate, inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], step=t)
        ref.step(w.gate, inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], step=t)
        gpu.step(dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], o, step=t)
        g = to_oracle(gpu)
        lsb, frac, heq, req = compare(g, tf)
        worst_o = max(worst_o, rel_l2(o.cpu().numpy(), o_tf))
        worst_lsb, worst_flip = max(worst_lsb, lsb), max(worst_flip, frac)
        exact = exact and lsb == 0 and heq and req
    drift = rel_l2(gpu.dequantize().cpu().numpy(), ref.dequantize())
    print(f"[{name}] steps={steps} worst o rel-L2 tf={worst_o:.2e} flips tf={worst_flip:.2e} "
          f"(max {worst_lsb} LSB) bit-exact={exact} drift={drift:.2e}", flush=True)
    assert worst_o <= O_REL_L2
    assert worst_lsb <= 1 and worst_flip <= CODE_FLIP_FRAC
    assert drift <= DRIFT_REL_L2


def test_step_kda_prewarmed(torch_cuda):
    w = wl.WORKLOADS[2]
    S0 = prewarmed_state(w, 1)[:, :8]
    run(torch_cuda, 2, 1, 8, 48, np.ascontiguousarray(S0), "damp kda prewarmed")


def test_step_gdn(torch_cuda):
    w = wl.WORKLOADS[1]
    rng = np.random.default_rng(3)
    S0 = (0.2 * rng.standard_normal((2, w.n_head, 128, 128))).astype(np.float32)
    run(torch_cuda, 1, 2, w.n_head, 48, S0, "damp gdn")


def test_zero_requests_is_noop(torch_cuda):
    from quantized_delta_rule_03_amd import qdr

    w = wl.WORKLOADS[2]
    gpu = qdr.DampState(0, 4, w.gate, selection(w, 4))
    e = torch_cuda.empty((0,), device="cuda")
    gpu.step(e, e, e, e, e, e, step=1)
    torch_cuda.cuda.synchronize()
