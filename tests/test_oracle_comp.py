"""CPU pins of the oracle's compensator tokens (no GPU).

The LeapQuant abstract keeps the state's largest outliers as a few high-precision
compensator tokens that share the update path of the real tokens, and quantizes the
residual. The oracle's reading: a token is one state entry kept in fp32 (the rank-one
term x e_i e_j^T); the m tokens are the m nonzero entries of largest magnitude (equal
magnitudes: smaller flat index first); the residual has those entries set to 0.
Pins: the selection against a brute-force sort by numpy's lexsort; the exact split
S = residual + tokens; ties, empty slots, the zero state; m = 0 reducing to the plain
quantization and window; the window starting from the dequantized residual plus the
tokens; spikes kept exactly and the quantization error they would cause removed; a
per-key-channel power-of-two smoothing absorbed exactly by the two-stage fit.
"""
import numpy as np
import pytest

import oracle

MIXED = np.array([8] * 32 + [6] * 64 + [4] * 32, np.uint8)


def spiky_state(seed, n_spikes=12, scale=50.0, outlier_cols=True):
    rng = np.random.default_rng(seed)
    S = 0.1 * rng.standard_normal((128, 128))
    if outlier_cols:
        S[:, rng.random(128) < 0.03] *= 10.0
    pos = rng.choice(128 * 128, n_spikes, replace=False)
    S.flat[pos] = scale * np.where(rng.random(n_spikes) < 0.5, -1.0, 1.0) * rng.uniform(
        0.5, 1.0, n_spikes)
    return S.astype(np.float32), pos


def brute_force(S, m):
    flat = S.ravel()
    nz = np.flatnonzero(flat != 0)
    order = nz[np.lexsort((nz, -np.abs(flat[nz]).astype(np.float64)))]
    take = order[:m]
    idx = np.full(m, oracle.TOK_EMPTY, np.uint16)
    val = np.zeros(m, np.float32)
    idx[: take.size] = take
    val[: take.size] = flat[take]
    return idx, val


@pytest.mark.parametrize("m", [1, 8, 16, 64])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_selection_matches_brute_force_sort(m, seed):
    S, _ = spiky_state(seed)
    idx, val, res = oracle.comp_select(S, m)
    bi, bv = brute_force(S, m)
    assert np.array_equal(idx, bi) and np.array_equal(val.view(np.uint32), bv.view(np.uint32))


def test_exact_split_into_residual_and_tokens():
    S, _ = spiky_state(3)
    idx, val, res = oracle.comp_select(S, 16)
    back = res.copy()
    back.flat[idx.astype(np.int64)] += val
    assert np.array_equal(back.view(np.uint32), S.view(np.uint32))
    assert np.all(res.flat[idx.astype(np.int64)] == 0)
    assert np.abs(res).max() <= np.abs(val).min()
    assert np.all(np.diff(np.abs(val)) <= 0)  # listed largest first


def test_ties_take_the_smaller_flat_index():
    rng = np.random.default_rng(4)
    S = np.where(rng.random((128, 128)) < 0.5, -1.0, 1.0).astype(np.float32)
    idx, val, _ = oracle.comp_select(S, 16)
    assert np.array_equal(idx, np.arange(16, dtype=np.uint16))
    # two magnitudes; the cut falls inside the group of equal smaller ones
    S = np.full((128, 128), 0.25, np.float32)
    big = np.array([9000, 17, 12345, 400, 16383])
    S.flat[big] = -3.0
    idx, _, _ = oracle.comp_select(S, 8)
    assert list(idx) == sorted(big) + [0, 1, 2]


def test_fewer_nonzeros_than_slots_and_zero_state():
    S = np.zeros((128, 128), np.float32)
    S.flat[[5, 700, 16000]] = [1.0, -2.0, 0.5]
    S.flat[9] = -0.0  # negative zero is no outlier
    idx, val, res = oracle.comp_select(S, 8)
    assert list(idx[:3]) == [700, 5, 16000] and list(val[:3]) == [-2.0, 1.0, 0.5]
    assert np.all(idx[3:] == oracle.TOK_EMPTY) and np.all(val[3:] == 0)
    assert not np.any(res)
    idx, val, res = oracle.comp_select(np.zeros((128, 128), np.float32), 8)
    assert np.all(idx == oracle.TOK_EMPTY) and np.all(val == 0) and not np.any(res)


def test_m0_is_the_plain_quantization():
    S, _ = spiky_state(5)
    c1, R1, k1, idx, val = oracle.comp_quantize(S, MIXED, 0)
    c2, R2, k2 = oracle.quantize(S, MIXED)
    assert idx.size == 0 and np.array_equal(c1, c2)
    assert np.array_equal(R1, R2) and np.array_equal(k1, k2)


def test_key_channel_smoothing_is_absorbed_by_the_fit():
    """The residual's smoothing is read as the existing two-stage fit (no separate
    transform). What pins that reading: a per-key-channel diagonal smoothing S D (D a
    diagonal of powers of two, as a smoothing would apply per channel) leaves every code and
    value-column scale unchanged and multiplies each key-row range by its factor exactly,
    because the key-row stage divides those ranges out before any rounding; so does a
    global power-of-two factor."""
    S, _ = spiky_state(9)
    c0, R0, k0 = oracle.quantize(S, MIXED)
    e = np.random.default_rng(3).integers(-6, 7, size=128)
    D = np.ldexp(np.ones(128, np.float32), e).astype(np.float32)
    c1, R1, k1 = oracle.quantize(np.ascontiguousarray(S * D[None, :]), MIXED)
    assert np.array_equal(c1, c0) and np.array_equal(k1, k0)
    assert np.array_equal(R1, (R0 * D).astype(np.float32))
    c2, R2, k2 = oracle.quantize(np.ascontiguousarray(S * np.float32(2.0 ** -5)), MIXED)
    assert np.array_equal(c2, c0) and np.array_equal(k2, k0)
    assert np.array_equal(R2, (R0 * np.float32(2.0 ** -5)).astype(np.float32))


def test_spikes_are_kept_exactly_and_their_error_removed():
    """With at least as many tokens as spikes, the dequantized state holds every spike
    exactly, and the scales fit the remaining entries: the error falls well below that of
    the plain quantization, whose key-row and value-column ranges the spikes set."""
    S, pos = spiky_state(6, n_spikes=12, outlier_cols=False)
    codes, R, c, idx, val = oracle.comp_quantize(S, MIXED, 16)
    Sh = oracle.comp_dequantize(codes, R, c, idx, val)
    assert np.array_equal(Sh.flat[pos], S.flat[pos])
    e_tok = np.linalg.norm(Sh - S)
    e_plain = np.linalg.norm(oracle.dequantize(*oracle.quantize(S, MIXED)) - S)
    assert e_tok < 0.5 * e_plain, (e_tok, e_plain)
    # what is left is the quantization error of the residual alone
    _, _, res = oracle.comp_select(S, 16)
    e_res = np.linalg.norm(oracle.dequantize(*oracle.quantize(res, MIXED)) - res)
    assert e_tok == e_res


def unit_inputs(seed, W, gate):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((W, 128)).astype(np.float32)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    q = rng.standard_normal((W, 128)).astype(np.float32)
    v = rng.standard_normal((W, 128)).astype(np.float32)
    a = rng.uniform(0.9, 1.0, (W, 128) if gate else (W,)).astype(np.float32)
    b = rng.uniform(0.0, 1.0, W).astype(np.float32)
    return q, k, v, a, b


@pytest.mark.parametrize("gate", [oracle.GDN, oracle.KDA])
def test_window_starts_from_the_residual_plus_tokens(gate):
    S, _ = spiky_state(7)
    codes, R, c, idx, val = oracle.comp_quantize(S, MIXED, 16)
    q, k, v, a, b = unit_inputs(8, 10, gate)
    out = oracle.comp_window(codes, R, c, idx, val, MIXED, gate, q, k, v, a, b,
                             return_state=True)
    S0 = oracle.dequantize(codes, R, c)
    S0.flat[idx.astype(np.int64)] += val
    Sd = S0.astype(np.float64)
    for t in range(10):
        o_t = oracle.recur_fp64(Sd, gate, q[t], k[t], v[t], a[t], b[t])
        assert np.array_equal(o_t, out[5][t])
    S_end = Sd.astype(np.float32)
    assert np.array_equal(out[6], S_end)
    c2, R2, k2, i2, v2 = oracle.comp_quantize(S_end, MIXED, 16)
    assert np.array_equal(out[0], c2) and np.array_equal(out[3], i2)
    assert np.array_equal(out[1], R2) and np.array_equal(out[2], k2) and np.array_equal(out[4], v2)


@pytest.mark.parametrize("gate", [oracle.GDN, oracle.KDA])
def test_window_with_no_tokens_is_the_plain_window(gate):
    S, _ = spiky_state(9)
    codes, R, c = oracle.quantize(S, MIXED)
    q, k, v, a, b = unit_inputs(10, 7, gate)
    plain = oracle.window(codes, R, c, MIXED, gate, q, k, v, a, b)
    comp = oracle.comp_window(codes, R, c, np.zeros(0, np.uint16), np.zeros(0, np.float32),
                              MIXED, gate, q, k, v, a, b)
    for x, y in zip(plain[:3], comp[:3]):
        assert np.array_equal(x, y)
    assert np.array_equal(plain[3], comp[5])


def test_pool_drivers_follow_the_unit_functions():
    """Mixed widths reorder the key channels in the packed layout; the pool drivers keep
    token indices in logical order."""
    n_req, H, m = 2, 3, 8
    bits = np.stack([MIXED, np.roll(MIXED, 40), np.full(128, 6, np.uint8)])
    S = np.stack([np.stack([spiky_state(20 + 3 * r + h)[0] for h in range(H)])
                  for r in range(n_req)])
    pool = oracle.Pool(n_req, H, bits)
    pool.comp_quantize(S, m)
    D = pool.comp_dequantize()
    for r in range(n_req):
        for h in range(H):
            codes, R, c, idx, val = oracle.comp_quantize(S[r, h], bits[h], m)
            assert np.array_equal(pool.tok_idx[r, h], idx)
            assert np.array_equal(pool.tok_val[r, h], val)
            assert np.array_equal(D[r, h], oracle.comp_dequantize(codes, R, c, idx, val))
