"""Error instrumentation of the scale rules (GPU) against an unquantized shadow state.

The dev.to page proposes logging per-row error norms against a high-precision reference
state over time, and compares uniform per-tensor INT8, per-row INT8 and finer-grained
precision. Here the GPU decode step runs the same seeded trajectory under four settings
(STEPQuant at the mixed 8/6/4-bit lifetime map, STEPQuant at 8 bits, per-key-row INT8,
per-tensor INT8) next to the oracle's unquantized fp64 recurrence (the shadow), on the
pre-warmed KDA states with 1% outlier key rows and value rows. Reported every 16 steps:
state error (rel-L2 against the shadow), readout error, and the share of the squared
error carried by the worst 5% of key rows. Asserted: the dynamic-range ordering at
8 bits (per-tensor > per-key-row > STEPQuant state error) at every checkpoint, and the
mixed 6-bit-nominal STEPQuant map ending below per-tensor INT8.
"""
import numpy as np
import pytest

import oracle
from parity_tools import bits_for, prewarmed_state, rel_l2, to_dev
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


def worst_share(err2: np.ndarray, frac=0.05):
    """Share of the total squared error in the worst `frac` of the entries of err2."""
    e = np.sort(err2.ravel())[::-1]
    k = max(1, int(round(frac * e.size)))
    return float(e[:k].sum() / max(e.sum(), 1e-300))


def test_rule_error_against_fp64_shadow(torch_cuda):
    from quantized_delta_rule_03_amd import qdr

    w = wl.WORKLOADS[2]
    n_req, H, steps = 1, w.n_head, 96
    S0 = prewarmed_state(w, n_req)
    b8 = wl.uniform_bits(H, 8)
    settings = [("STEP mixed 8/6/4", bits_for(w), qdr.RULE_STEP),
                ("STEP 8-bit", b8, qdr.RULE_STEP),
                ("KEYROW INT8", b8, qdr.RULE_KEYROW),
                ("TENSOR INT8", b8, qdr.RULE_TENSOR)]
    pools = []
    for name, bits, rule in settings:
        ref = oracle.Pool(n_req, H, bits, rule=rule)
        ref.quantize(S0)
        gpu = qdr.StatePool(n_req, H, w.gate, bits, rule=rule)
        gpu.load_host(ref.packed, ref.row_scale, ref.col_scale)
        pools.append(gpu)
    shadow = S0.astype(np.float64).copy()
    o = torch_cuda.empty((n_req, H, 128), dtype=torch_cuda.float32, device="cuda")
    hist = {name: [] for name, _, _ in settings}
    o_err = {name: 0.0 for name, _, _ in settings}
    for t in range(steps):
        inp = wl.step_inputs(w, t, n_req=n_req)
        dev = to_dev(inp)
        o_sh = np.zeros((n_req, H, 128), np.float32)
        for r in range(n_req):
            for h in range(H):
                o_sh[r, h] = oracle.recur_fp64(shadow[r, h], w.gate, inp["q"][r, h],
                                               inp["k"][r, h], inp["v"][r, h], inp["a"][r, h],
                                               inp["b"][r, h])
        for (name, _, _), gpu in zip(settings, pools):
            gpu.step(dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], o)
            o_err[name] = max(o_err[name], rel_l2(o.cpu().numpy(), o_sh))
        if (t + 1) % 16 == 0:
            for (name, _, _), gpu in zip(settings, pools):
                Sh = gpu.dequantize().cpu().numpy().astype(np.float64)
                d2 = (Sh - shadow) ** 2
                key_rows = d2.sum(axis=2)  # [r, h, key channel]: error per key row
                hist[name].append((t + 1, rel_l2(Sh, shadow), worst_share(key_rows)))
    print("\nstate error against the fp64 shadow (rel-L2) / share of squared error in the "
          "worst 5% of key rows:", flush=True)
    for name, _, _ in settings:
        line = "  ".join(f"t={t}: {e:.2e}/{s:.2f}" for t, e, s in hist[name])
        print(f"  {name:18s} {line}   worst readout rel-L2 {o_err[name]:.2e}", flush=True)
    for k in range(len(hist["STEP 8-bit"])):
        e_step = hist["STEP 8-bit"][k][1]
        e_row = hist["KEYROW INT8"][k][1]
        e_ten = hist["TENSOR INT8"][k][1]
        assert e_ten > e_row > e_step, (k, e_ten, e_row, e_step)
    assert hist["STEP mixed 8/6/4"][-1][1] < hist["TENSOR INT8"][-1][1]
