"""CPU pins of the oracle's comparison scale rules (no GPU).

The baselines are the dev.to page's "Uniform per-tensor INT8" and "Per-row (per-channel)
INT8" options (section listing the four quantization options), written in the same
(R_j, c_i) state format as the STEPQuant rule: KEYROW keeps one range per key row (the
first stage of the two-stage absmax) and c = 1; TENSOR keeps one range for the whole
state and c = 1. The pins tie them to the STEPQuant rule through the special cases where
the definitions coincide, and check the invariants each rule must satisfy on its own.
"""
import numpy as np
import pytest

import oracle

RULES = (oracle.RULE_STEP, oracle.RULE_KEYROW, oracle.RULE_TENSOR)
B8 = np.full(128, 8, np.uint8)


def mixed_bits():
    return np.array([8] * 32 + [6] * 64 + [4] * 32, np.uint8)


def qmax(bits):
    return (1 << (bits.astype(np.int32) - 1)) - 1


def rand_state(seed, outliers=False):
    rng = np.random.default_rng(seed)
    S = rng.standard_normal((128, 128))
    if outliers:  # 1% of key rows and value rows x 10
        S[:, rng.random(128) < 0.02] *= 10.0
        S[rng.random(128) < 0.02, :] *= 10.0
    return S.astype(np.float32)


def test_step_equals_keyrow_when_every_value_row_reaches_its_key_ranges():
    """S = s u^T with s_i = +-1: every value row attains each key row's range, so the
    STEPQuant value-column scales are all 1 and the rule reduces to per-key-row."""
    rng = np.random.default_rng(1)
    u = rng.standard_normal(128).astype(np.float32)
    s = np.where(rng.random(128) < 0.5, -1.0, 1.0).astype(np.float32)
    S = np.outer(s, u).astype(np.float32)
    for bits in (B8, mixed_bits()):
        c1, R1, k1 = oracle.quantize(S, bits, oracle.RULE_STEP)
        c2, R2, k2 = oracle.quantize(S, bits, oracle.RULE_KEYROW)
        assert np.array_equal(k1, np.ones(128, np.float32))
        assert np.array_equal(c1, c2) and np.array_equal(R1, R2) and np.array_equal(k1, k2)


def test_keyrow_equals_tensor_when_all_key_ranges_are_equal():
    S = rand_state(2)
    S = (S / np.abs(S).max(axis=0, keepdims=True)).astype(np.float32)  # every column max 1
    assert np.all(np.abs(S).max(axis=0) == 1.0)
    c1, R1, k1 = oracle.quantize(S, B8, oracle.RULE_KEYROW)
    c2, R2, k2 = oracle.quantize(S, B8, oracle.RULE_TENSOR)
    assert np.array_equal(c1, c2) and np.array_equal(R1, R2) and np.array_equal(k1, k2)


@pytest.mark.parametrize("bits", [B8, mixed_bits()], ids=["8bit", "mixed"])
def test_tensor_rule_invariants(bits):
    S = rand_state(3, outliers=True)
    codes, R, c = oracle.quantize(S, bits, oracle.RULE_TENSOR)
    assert np.all(c == 1.0)
    A = R * qmax(bits)  # one range for every key row
    assert np.allclose(A, A[0], rtol=2e-7)
    i, j = np.unravel_index(np.argmax(np.abs(S)), S.shape)
    assert abs(int(codes[i, j])) == qmax(bits)[j]


@pytest.mark.parametrize("bits", [B8, mixed_bits()], ids=["8bit", "mixed"])
def test_keyrow_rule_invariants(bits):
    S = rand_state(4, outliers=True)
    S[:, 7] = 0.0  # an all-zero key row
    codes, R, c = oracle.quantize(S, bits, oracle.RULE_KEYROW)
    assert np.all(c == 1.0)
    qm = qmax(bits)
    peak = np.abs(codes.astype(np.int32)).max(axis=0)
    nz = np.abs(S).max(axis=0) > 0
    assert np.array_equal(peak[nz], qm[nz])
    assert np.all(codes[:, 7] == 0) and R[7] == np.float32(1.0 / qm[7])


@pytest.mark.parametrize("rule", RULES)
def test_half_step_error_bound(rule):
    S = rand_state(5, outliers=True)
    bits = mixed_bits()
    codes, R, c = oracle.quantize(S, bits, rule)
    Sh = oracle.dequantize(codes, R, c).astype(np.float64)
    step = np.outer(c.astype(np.float64), R.astype(np.float64))
    err = np.abs(Sh - S.astype(np.float64))
    assert np.all(err <= 0.5 * step * (1 + 1e-5) + 1e-6 * np.abs(S))


@pytest.mark.parametrize("rule", RULES)
def test_requant_idempotence(rule):
    S = rand_state(6, outliers=True)
    bits = mixed_bits()
    codes, R, c = oracle.quantize(S, bits, rule)
    codes2, R2, c2 = oracle.quantize(oracle.dequantize(codes, R, c), bits, rule)
    assert np.array_equal(codes, codes2)
    assert np.allclose(R, R2, rtol=2e-7) and np.allclose(c, c2, rtol=2e-7)


@pytest.mark.parametrize("rule", RULES)
def test_zero_state_is_the_init_state(rule):
    bits = mixed_bits()
    codes, R, c = oracle.quantize(np.zeros((128, 128), np.float32), bits, rule)
    assert np.all(codes == 0) and np.all(c == 1.0)
    assert np.array_equal(R, (1.0 / qmax(bits)).astype(np.float32))


@pytest.mark.parametrize("rule", RULES)
def test_identity_step_keeps_the_codes(rule):
    """a = 1, b = 0: the update is the identity, so the step's requantization under the
    same rule must return the codes it started from."""
    S = rand_state(7, outliers=True)
    bits = mixed_bits()
    codes, R, c = oracle.quantize(S, bits, rule)
    rng = np.random.default_rng(8)
    k = rng.standard_normal(128).astype(np.float32)
    k /= np.linalg.norm(k)
    q = rng.standard_normal(128).astype(np.float32)
    v = rng.standard_normal(128).astype(np.float32)
    c2, R2, k2, o = oracle.step(codes, R, c, bits, 0, q, k, v, np.float32(1.0), 0.0, rule=rule)
    assert np.array_equal(c2, codes)


def test_dynamic_range_ordering_on_outlier_states():
    """The dynamic-range argument of the per-tensor option: with a few hot key rows and
    value rows, one range for the whole state leaves the rest of it few effective levels.
    At 8 bits the mean squared error orders TENSOR > KEYROW > STEP on such states."""
    errs = {r: 0.0 for r in RULES}
    for seed in range(4):
        S = rand_state(10 + seed, outliers=True)
        for r in RULES:
            codes, R, c = oracle.quantize(S, B8, r)
            d = oracle.dequantize(codes, R, c).astype(np.float64) - S
            errs[r] += float((d * d).mean())
    assert errs[oracle.RULE_TENSOR] > errs[oracle.RULE_KEYROW] > errs[oracle.RULE_STEP]
