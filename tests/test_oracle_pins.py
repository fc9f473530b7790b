"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: published
format values, library routines (torch's float8/bf16 casts, torch softmax),
exact integer arithmetic, brute force on tiny inputs, closed forms and the
page's layer list.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(12345)


def _finite_codes(n, rs=rng):
    c = rs.integers(0, 256, size=n).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3C  # avoid the NaN codes
    return c


# ------------------------------------------------------------------ E4M3 / bf16
def test_e4m3_matches_torch_float8_all_codes():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        v = oracle.e4m3(c)
        if np.isnan(ref[c]):
            assert np.isnan(v), c
        else:
            assert v == ref[c] and np.signbit(v) == np.signbit(ref[c]), (c, v, ref[c])


def test_e4m3_ocp_spot_values():
    n = 0
    for line in open(os.path.join(GOLDEN, "e4m3_ocp_spot.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        code, val = line.split()
        v = oracle.e4m3(int(code, 16))
        if val == "nan":
            assert np.isnan(v)
        else:
            assert v == float(val) and np.signbit(v) == val.startswith("-"), (code, v)
        n += 1
    assert n == 12


def test_bf16_decode_matches_torch():
    bits = rng.integers(0, 1 << 16, size=4000).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # finite only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16(int(b)) for b in bits])
    assert np.array_equal(got, ref)


def test_round_bf16_against_torch_and_ties():
    # values exactly representable in fp32: torch's fp32 -> bf16 cast is RNE
    x = (rng.standard_normal(3000) * 10.0 ** rng.integers(-5, 5, size=3000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.round_bf16(float(v)) for v in x], np.uint16)
    assert np.array_equal(got, ref)
    # exact ties go to the even significand
    assert oracle.round_bf16(1.0 + 2.0 ** -8) == 0x3F80  # tie between 1 and 1+2^-7 -> 1
    assert oracle.round_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82  # tie -> 1+2^-6 (even)
    assert oracle.round_bf16(-(1.0 + 2.0 ** -8 + 2.0 ** -30)) == 0xBF81  # just above a tie


# ------------------------------------------------------------------ E4M3 encoding / quantisation
def _finite_code_values():
    return [(c, oracle.e4m3(c)) for c in range(256) if (c & 0x7F) != 0x7F]


def test_encode_e4m3_round_trips_every_finite_code():
    for c, v in _finite_code_values():
        assert oracle.encode_e4m3(v) == c, (c, v)


def test_encode_e4m3_matches_torch_float8_cast():
    # torch's binary32 -> float8_e4m3fn cast rounds to nearest even; it does not
    # saturate, so only |x| <= 448 is compared (saturation is pinned below)
    x = (rng.standard_normal(6000) * 2.0 ** rng.integers(-12, 9, size=6000)).astype(np.float32)
    x = x[np.abs(x) <= 448]
    vals = sorted(v for c, v in _finite_code_values() if c < 0x80)
    mids = np.array([(a + b) / 2 for a, b in zip(vals, vals[1:])], np.float32)  # exact ties
    nxt = np.nextafter(mids, np.float32(np.inf))
    prv = np.nextafter(mids, np.float32(0))
    x = np.concatenate([x, mids, -mids, nxt, prv, -nxt])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.encode_e4m3(float(v)) for v in x], np.uint8)
    assert np.array_equal(got, ref)


def test_encode_e4m3_ties_saturation_and_signed_zero():
    vals = sorted(v for c, v in _finite_code_values() if c < 0x80)
    for c in range(0x7E):  # every adjacent pair: the tie goes to the even code
        m = (vals[c] + vals[c + 1]) / 2
        assert oracle.encode_e4m3(m) == (c if c % 2 == 0 else c + 1), c
        assert oracle.encode_e4m3(-m) == 0x80 | (c if c % 2 == 0 else c + 1), c
    for v in (448.0, 460.0, 464.0, 1e4, 1e30):
        assert oracle.encode_e4m3(v) == 0x7E and oracle.encode_e4m3(-v) == 0xFE
    assert oracle.encode_e4m3(0.0) == 0x00 and oracle.encode_e4m3(-0.0) == 0x80
    assert oracle.encode_e4m3(-2.0 ** -11) == 0x80  # rounds to zero, keeps the sign
    assert oracle.encode_e4m3(2.0 ** -10 * 1.0000001) == 0x01  # just past the first tie


@pytest.mark.parametrize("D", [128, 576])
def test_quantize_recovers_codes_times_power_of_two_scale(D):
    # x = dec(code) * 2^e with one entry at +-448 is exactly bf16, its amax is
    # 448 * 2^e, so the scale is exactly 2^e and every code must come back
    rs = np.random.default_rng(7 + D)
    codes = _finite_codes(6 * D, rs).reshape(6, D)
    exps = np.array([-20, -6, -1, 0, 3, 9])
    for r in range(6):
        codes[r, rs.integers(0, D)] = 0x7E if r % 2 == 0 else 0xFE
    x = np.array([[oracle.e4m3(int(c)) * 2.0 ** int(e) for c in row] for row, e in zip(codes, exps)])
    bits = _bf16_bits(x)
    assert np.array_equal(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy(), x)
    got_c, got_s = oracle.quantize_e4m3(bits)
    assert np.array_equal(got_s, (2.0 ** exps).astype(np.float32))
    # -0.0 codes decode to -0.0, which re-encodes as 0x80; 0x00 stays 0x00
    assert np.array_equal(got_c, codes)


def test_quantize_error_bound_and_zero_rows():
    rs = np.random.default_rng(99)
    x = (rs.standard_normal((40, 576)) * 10.0 ** rs.integers(-3, 3, size=(40, 1))).astype(np.float32)
    x[3] = 0.0
    x[4] = -0.0
    x[5, :] = 0.0
    x[5, 17] = -3.0  # one nonzero entry, negative
    bits = _bf16_bits(x)
    xb = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    codes, scales = oracle.quantize_e4m3(bits)
    assert scales[3] == 1.0 and scales[4] == 1.0
    assert np.all(codes[3] == 0x00) and np.all(codes[4] == 0x80)
    assert scales[5] == np.float32(3.0 / 448.0) and codes[5, 17] == 0xFE
    dec = np.vectorize(oracle.e4m3)(codes)
    for r in range(40):
        s = float(scales[r])
        if r not in (3, 4):
            assert s == np.float32(np.float32(np.abs(xb[r]).max()) / np.float32(448.0))
        y = xb[r] / s
        # nearest-code error: half a step, 2^-4 relative for normals, 2^-10 below 2^-6;
        # slack for the binary32 quotient
        bound = np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) * (1 + 2.0 ** -20)
        assert np.all(np.abs(dec[r] - y) <= bound), r
        assert np.all(np.signbit(dec[r]) == np.signbit(xb[r]))
        assert np.abs(dec[r]).max() == (448.0 if s != 1.0 or np.abs(xb[r]).max() else 0.0)


def test_quantize_rejects_non_finite_rows():
    bits = _bf16_bits(np.ones((2, 128), np.float32))
    bits[1, 5] = 0x7F80  # +inf
    with pytest.raises(ValueError):
        oracle.quantize_e4m3(bits)


def test_cache_append_writes_addressed_rows_only():
    rs = np.random.default_rng(5)
    B, T, L = 3, 4, 11
    pos = np.array([[7, 8, 9, 10], [-1, 0, 11, 3], [2, 5, 40, -7]], np.int32)
    k_codes = _finite_codes(B * T * 128, rs).reshape(B, T, 128)
    k_codes[..., 0] = 0x7E
    k_new = _bf16_bits(np.vectorize(oracle.e4m3)(k_codes) * 0.25)
    kv_new = _bf16_bits(rs.standard_normal((B, T, 576)))
    k8 = rs.integers(0, 256, size=(B, L, 128)).astype(np.uint8)
    ks = rs.standard_normal((B, L)).astype(np.float32)
    kvb = rs.integers(0, 1 << 16, size=(B, L, 576)).astype(np.uint16)
    o_k8, o_ks, o_kv, _ = oracle.cache_append(k_new, kv_new, pos, k8, ks, kvb, None)
    written = np.zeros((B, L), bool)
    for b in range(B):
        for t in range(T):
            p = pos[b, t]
            if 0 <= p < L:
                written[b, p] = True
                assert np.array_equal(o_k8[b, p], k_codes[b, t]) and o_ks[b, p] == 0.25
                assert np.array_equal(o_kv[b, p], kv_new[b, t])
    assert np.array_equal(o_k8[~written], k8[~written]) and np.array_equal(o_ks[~written], ks[~written])
    assert np.array_equal(o_kv[~written], kvb[~written])
    # FP8 latent cache: the rows are quantised like any other row
    kv8 = rs.integers(0, 256, size=(B, L, 576)).astype(np.uint8)
    kvs = np.zeros((B, L), np.float32)
    _, _, o_kv8, o_kvs = oracle.cache_append(None, kv_new, pos, None, None, kv8, kvs)
    c, s = oracle.quantize_e4m3(kv_new)
    for b in range(B):
        for t in range(T):
            p = pos[b, t]
            if 0 <= p < L:
                assert np.array_equal(o_kv8[b, p], c[b, t]) and o_kvs[b, p] == s[b, t]
    assert np.array_equal(o_kv8[~written], kv8[~written])
    with pytest.raises(ValueError):  # two tokens of one sequence at one position
        oracle.cache_append(None, kv_new, np.array([[1, 2, 1, 3]] * 3, np.int32), None, None,
                            kvb, None)


# ------------------------------------------------------------------ indexer
def _idx_inputs(B, T, L, rs):
    q8 = _finite_codes(B * T * 32 * 128, rs).reshape(B, T, 32, 128)
    k8 = _finite_codes(B * L * 128, rs).reshape(B, L, 128)
    qs = rs.uniform(0.001, 0.1, size=(B, T, 32)).astype(np.float32)
    w = rs.uniform(0, 1, size=(B, T, 32)).astype(np.float32)
    ks = rs.uniform(0.001, 0.1, size=(B, L)).astype(np.float32)
    return q8, qs, w, k8, ks


def _dec(codes):
    lut = np.array([oracle.e4m3(c) for c in range(256)])
    return lut[codes]


def test_idx_score_brute_force_numpy():
    rs = np.random.default_rng(7)
    B, T, L = 2, 3, 37
    q8, qs, w, k8, ks = _idx_inputs(B, T, L, rs)
    vis = np.array([[37, 20, 0], [1, 37, 50]], np.int32)
    got, got64 = oracle.idx_score(q8, qs, w, k8, ks, vis, want64=True)
    d = np.einsum("btjd,bsd->btjs", _dec(q8), _dec(k8))  # library contraction, float64
    ref = ks[:, None, :] * np.einsum("btj,btjs->bts", w.astype(np.float64) * qs, np.maximum(d, 0))
    for b in range(B):
        for t in range(T):
            v = min(max(vis[b, t], 0), L)
            assert np.all(np.isneginf(got[b, t, v:])) and np.all(np.isneginf(got64[b, t, v:]))
            np.testing.assert_allclose(got64[b, t, :v], ref[b, t, :v], rtol=1e-13, atol=0)
            np.testing.assert_array_equal(got[b, t, :v], got64[b, t, :v].astype(np.float32))


def test_idx_score_dot_is_exact():
    # one head, w = scales = 1: the double score equals relu(q.k) exactly; every E4M3
    # value is an integer multiple of 2^-9, so q.k * 2^18 is an exact integer
    rs = np.random.default_rng(8)
    L = 64
    q8, qs, w, k8, ks = _idx_inputs(1, 1, L, rs)
    w[:] = 0
    w[0, 0, 5] = 1
    qs[:] = 1
    ks[:] = 1
    _, got64 = oracle.idx_score(q8, qs, w, k8, ks, np.array([[L]], np.int32), want64=True)
    qi = [int(Fraction(oracle.e4m3(c)) * 512) for c in q8[0, 0, 5]]
    for s in range(L):
        ki = [int(Fraction(oracle.e4m3(c)) * 512) for c in k8[0, s]]
        exact = Fraction(sum(a * b for a, b in zip(qi, ki)), 1 << 18)
        assert Fraction(got64[0, 0, s]) == max(exact, Fraction(0)), s


def test_idx_score_closed_forms():
    L = 8
    q8 = np.full((1, 1, 32, 128), 0x44, np.uint8)  # 3.0
    k8 = np.full((1, L, 128), 0x30, np.uint8)  # 0.5
    k8[0, 3] = 0xB0  # -0.5 -> every head negative -> 0
    qs = np.linspace(0.5, 2.0, 32, dtype=np.float32).reshape(1, 1, 32)
    w = np.linspace(0.0, 1.0, 32, dtype=np.float32).reshape(1, 1, 32)
    ks = np.arange(1, L + 1, dtype=np.float32).reshape(1, L) * 0.25
    vis = np.array([[L]], np.int32)
    _, s64 = oracle.idx_score(q8, qs, w, k8, ks, vis, want64=True)
    d = 128 * 3.0 * 0.5
    for s in range(L):
        exp = 0.0 if s == 3 else float(ks[0, s]) * sum(float(w[0, 0, j]) * float(qs[0, 0, j]) * d
                                                      for j in range(32))
        assert s64[0, 0, s] == pytest.approx(exp, rel=1e-15, abs=0)
    # doubling every head weight doubles every score exactly
    s1 = oracle.idx_score(q8, qs, w, k8, ks, vis)
    s2 = oracle.idx_score(q8, qs, 2 * w, k8, ks, vis)
    np.testing.assert_array_equal(s2, 2 * s1)


def test_idx_score_query_opposite_key_is_zero():
    rs = np.random.default_rng(9)
    q8, qs, w, k8, ks = _idx_inputs(1, 1, 4, rs)
    q8[0, 0, :, :] = k8[0, 2, :] ^ 0x80  # every head = -key 2
    s = oracle.idx_score(q8, qs, w, k8, ks, np.array([[4]], np.int32))
    assert s[0, 0, 2] == 0.0 and not np.signbit(s[0, 0, 2])


def test_idx_score_vis_len_clamped():
    rs = np.random.default_rng(10)
    q8, qs, w, k8, ks = _idx_inputs(1, 2, 5, rs)
    s = oracle.idx_score(q8, qs, w, k8, ks, np.array([[-3, 99]], np.int32))
    assert np.all(np.isneginf(s[0, 0])) and np.all(np.isfinite(s[0, 1]))


# ------------------------------------------------------------------ top-k
def _brute_topk(scores, vis, k):
    order = sorted(range(vis), key=lambda s: (-float(scores[s]), s))
    sel = sorted(order[:k])
    return sel + [-1] * (k - len(sel))


@pytest.mark.parametrize("L,k", [(1, 1), (7, 4), (2047, 2048), (2048, 2048), (2049, 2048),
                                 (4096, 2048), (4096, 64), (300, 100)])
def test_topk_brute_force_with_ties(L, k):
    rs = np.random.default_rng(L * 31 + k)
    s = rs.integers(0, 50, size=(2, 2, L)).astype(np.float32) * 0.25  # many ties
    vis = np.array([[L, max(L // 2, 1)], [max(L - 1, 0), 0]], np.int32)
    got = oracle.topk(s, vis, k)
    for b in range(2):
        for t in range(2):
            assert list(got[b, t]) == _brute_topk(s[b, t], vis[b, t], k), (b, t)


def test_topk_properties():
    rs = np.random.default_rng(11)
    L, k = 5000, 2048
    s = rs.standard_normal((1, 1, L)).astype(np.float32)
    idx = oracle.topk(s, np.array([[L]], np.int32), k)[0, 0]
    assert len(set(idx)) == k and np.all(np.diff(idx) > 0)
    sel = np.zeros(L, bool)
    sel[idx] = True
    assert s[0, 0, sel].min() >= s[0, 0, ~sel].max()
    # scaling by a power of two changes nothing
    idx2 = oracle.topk(s * 8, np.array([[L]], np.int32), k)[0, 0]
    assert np.array_equal(idx, idx2)
    # all equal -> the first k positions
    eq = np.ones((1, 1, L), np.float32)
    assert np.array_equal(oracle.topk(eq, np.array([[L]], np.int32), k)[0, 0], np.arange(k))
    # fewer visible than k -> all of them then -1
    got = oracle.topk(s, np.array([[100]], np.int32), k)[0, 0]
    assert np.array_equal(got[:100], np.arange(100)) and np.all(got[100:] == -1)


def test_topk_signed_zero_is_a_tie_and_nan_rejected():
    s = np.array([[[-0.0, 0.0, -0.0, 1.0]]], np.float32)
    assert list(oracle.topk(s, np.array([[4]], np.int32), 2)[0, 0]) == [0, 3]
    s[0, 0, 1] = np.nan
    with pytest.raises(ValueError):
        oracle.topk(s, np.array([[4]], np.int32), 2)


# ------------------------------------------------------------------ attention
def _bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def _bits_to_f64(b):
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).double().numpy()


def _dense_ref(q, rows, sm):
    """dense softmax attention with torch (float64): q[64,576], rows[n,576]"""
    qt = torch.from_numpy(q)
    rt = torch.from_numpy(rows)
    z = sm * (qt @ rt.T)
    p = torch.softmax(z, dim=-1)
    return (p @ rt[:, :512]).numpy(), torch.logsumexp(z, dim=-1).numpy()


def test_sparse_mla_k_equals_L_matches_dense_softmax():
    rs = np.random.default_rng(12)
    B, T, L = 2, 2, 96
    q = _bf16_bits(rs.standard_normal((B, T, 64, 576)))
    kv = _bf16_bits(rs.standard_normal((B, L, 576)))
    idx = np.broadcast_to(np.arange(L, dtype=np.int32), (B, T, L)).copy()
    out, lse, out64 = oracle.sparse_mla(q, kv, None, idx, 1 / 24, want64=True)
    for b in range(B):
        for t in range(T):
            ref, rl = _dense_ref(_bits_to_f64(q[b, t]), _bits_to_f64(kv[b]), 1 / 24)
            np.testing.assert_allclose(out64[b, t], ref, rtol=1e-11, atol=1e-13)
            np.testing.assert_allclose(lse[b, t], rl, rtol=1e-6)
            # output rounding is RNE of the double result
            assert all(oracle.round_bf16(v) == o for v, o in
                       zip(out64[b, t].ravel()[:300], out[b, t].ravel()[:300]))


def test_sparse_mla_fp8_rows_match_dense_on_dequantised_values():
    rs = np.random.default_rng(13)
    L = 40
    q = _bf16_bits(rs.standard_normal((1, 1, 64, 576)))
    codes = _finite_codes(L * 576, rs).reshape(1, L, 576)
    sc = rs.uniform(0.001, 0.02, size=(1, L)).astype(np.float32)
    idx = np.arange(L, dtype=np.int32).reshape(1, 1, L)[:, :, ::-1].copy()
    out, lse, out64 = oracle.sparse_mla(q, codes, sc, idx, 1 / 24, want64=True)
    rows = _dec(codes[0]) * sc[0][:, None].astype(np.float64)
    ref, rl = _dense_ref(_bits_to_f64(q[0, 0]), rows, 1 / 24)
    np.testing.assert_allclose(out64[0, 0], ref, rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], rl, rtol=1e-6)


def test_sparse_mla_special_cases():
    rs = np.random.default_rng(14)
    L, k = 50, 8
    q = _bf16_bits(rs.standard_normal((1, 1, 64, 576)))
    kv = _bf16_bits(rs.standard_normal((1, L, 576)))
    # one valid index: out = the row's latent part, lse = its logit
    idx = np.full((1, 1, k), -1, np.int32)
    idx[0, 0, 3] = 17
    out, lse = oracle.sparse_mla(q, kv, None, idx, 1 / 24)
    for h in range(64):
        assert np.array_equal(out[0, 0, h], kv[0, 17, :512])
        z = np.dot(_bits_to_f64(q[0, 0, h]), _bits_to_f64(kv[0, 17])) / 24
        assert lse[0, 0, h] == pytest.approx(z, rel=1e-6, abs=1e-6)
    # no valid index: zeros and -inf
    idx[:] = -1
    out, lse = oracle.sparse_mla(q, kv, None, idx, 1 / 24)
    assert np.all(out == 0) and np.all(np.isneginf(lse))
    # q = 0: every selected row has weight 1/n -> the mean
    sel = np.array([1, 5, 9, 44, 2, 30, 31, 7], np.int32)
    zero_q = np.zeros_like(q)
    _, _, o64 = oracle.sparse_mla(zero_q, kv, None, sel.reshape(1, 1, k), 1 / 24, want64=True)
    mean = _bits_to_f64(kv[0, sel, :512]).mean(axis=0)
    np.testing.assert_allclose(o64[0, 0, 0], mean, rtol=1e-13, atol=1e-15)
    # permuting idx changes nothing (up to double rounding)
    _, _, a64 = oracle.sparse_mla(q, kv, None, sel.reshape(1, 1, k), 1 / 24, want64=True)
    _, _, b64 = oracle.sparse_mla(q, kv, None, sel[::-1].copy().reshape(1, 1, k), 1 / 24,
                                  want64=True)
    np.testing.assert_allclose(a64, b64, rtol=1e-12, atol=1e-15)
    # out-of-range positions are rejected
    with pytest.raises(ValueError):
        oracle.sparse_mla(q, kv, None, np.full((1, 1, k), L, np.int32), 1 / 24)


def test_sparse_mla_planted_peak_dominates():
    rs = np.random.default_rng(15)
    L = 64
    kvf = rs.standard_normal((1, L, 576))
    qf = rs.standard_normal((1, 1, 64, 576)) * 0.05
    # row 10 aligned with every head's query: logit about 20 above the rest
    kvf[0, 10] = qf[0, 0, 0] / np.linalg.norm(qf[0, 0, 0]) * (20 * 24 / np.linalg.norm(qf[0, 0, 0]))
    q, kv = _bf16_bits(qf), _bf16_bits(kvf)
    qf64 = _bits_to_f64(q)
    for h in range(64):
        qf64[0, 0, h] = qf64[0, 0, 0]
    q = _bf16_bits(qf64)
    idx = np.arange(L, dtype=np.int32).reshape(1, 1, L)
    _, _, o64 = oracle.sparse_mla(q, kv, None, idx, 1 / 24, want64=True)
    np.testing.assert_allclose(o64[0, 0, 0], _bits_to_f64(kv[0, 10, :512]), atol=2e-6 * 500)


# ------------------------------------------------------------------ IndexShare / MTP
def _golden_schedule():
    d = {}
    for line in open(os.path.join(GOLDEN, "indexshare_schedule.txt")):
        line = line.split("#")[0].strip()
        if line:
            key, val = line.split(":")
            d[key.strip()] = val.split()
    return d


def test_glm52_schedule_equals_page_list():
    g = _golden_schedule()
    n = int(g["n_layers"][0])
    full = [l for l in range(n) if oracle.is_full_layer(oracle.SCHED_GLM52, l)]
    assert full == [int(x) for x in g["full_layers"]]
    assert len(full) == int(g["n_full"][0]) and n - len(full) == int(g["n_shared"][0])
    assert round(100 * (n - len(full)) / n, 1) == float(g["shared_fraction_percent"][0])
    # one computing layer and three reusing layers per group of four
    assert [l for l in range(8) if oracle.is_full_layer(oracle.SCHED_GROUP4, l)] == [0, 4]
    assert all(oracle.is_full_layer(oracle.SCHED_ALL_FULL, l) for l in range(78))


def _small_layers(n, B, T, L, rs, kv_fp8=False, same_indexer=False):
    q8, qs, w, k8, ks = _idx_inputs(B, T, L, rs)
    layers = []
    for l in range(n):
        if not same_indexer:
            q8, qs, w, k8, ks = _idx_inputs(B, T, L, rs)
        ly = {"q8": q8, "q_scale": qs, "w": w, "k8": k8, "k_scale": ks,
              "q": _bf16_bits(rs.standard_normal((B, T, 64, 576)))}
        if kv_fp8:
            ly["kv"] = _finite_codes(B * L * 576, rs).reshape(B, L, 576)
            ly["kv_scale"] = rs.uniform(0.001, 0.01, size=(B, L)).astype(np.float32)
        else:
            ly["kv"] = _bf16_bits(rs.standard_normal((B, L, 576)))
        layers.append(ly)
    return layers


def test_indexshare_shared_layers_use_full_layer_selection():
    rs = np.random.default_rng(16)
    B, T, L, k = 1, 2, 300, 64
    layers = _small_layers(8, B, T, L, rs)
    vis = np.array([[300, 150]], np.int32)
    outs, lses, idx_out = oracle.indexshare(layers, oracle.SCHED_GROUP4, vis, k, 1 / 24)
    assert idx_out.shape[0] == 2
    for l in range(8):
        f = l // 4
        sc = oracle.idx_score(layers[4 * f]["q8"], layers[4 * f]["q_scale"], layers[4 * f]["w"],
                              layers[4 * f]["k8"], layers[4 * f]["k_scale"], vis)
        assert np.array_equal(idx_out[f], oracle.topk(sc, vis, k))
        o, s = oracle.sparse_mla(layers[l]["q"], layers[l]["kv"], None, idx_out[f], 1 / 24)
        assert np.array_equal(o, outs[l]) and np.array_equal(s, lses[l])
    # shared layers never read their own indexer inputs
    for l in (1, 2, 3, 5, 6, 7):
        for f in ("q8", "q_scale", "w", "k8", "k_scale"):
            layers[l][f] = None
    outs2, _, idx2 = oracle.indexshare(layers, oracle.SCHED_GROUP4, vis, k, 1 / 24)
    assert np.array_equal(idx2, idx_out) and all(np.array_equal(a, b) for a, b in zip(outs, outs2))


def test_indexshare_all_full_with_shared_inputs_gives_identical_selections():
    rs = np.random.default_rng(17)
    layers = _small_layers(4, 1, 1, 200, rs, same_indexer=True)
    vis = np.array([[200]], np.int32)
    _, _, idx_out = oracle.indexshare(layers, oracle.SCHED_ALL_FULL, vis, 32, 1 / 24)
    assert idx_out.shape[0] == 4 and all(np.array_equal(idx_out[0], idx_out[i]) for i in range(4))


def test_mtp_steps_reuse_step0_selection_and_kv():
    rs = np.random.default_rng(18)
    B, T, L, k = 2, 1, 256, 64
    layers = _small_layers(7, B, T, L, rs, kv_fp8=True)
    vis = np.full((B, T), L, np.int32)
    outs, lses, idx_out = oracle.indexshare(layers, 0, vis, k, 1 / 24, kv_fp8=True, mtp_steps=7)
    assert idx_out.shape[0] == 1
    for s in range(7):
        o, ls = oracle.sparse_mla(layers[s]["q"], layers[0]["kv"], layers[0]["kv_scale"],
                                  idx_out[0], 1 / 24)
        assert np.array_equal(o, outs[s]) and np.array_equal(ls, lses[s])
    # the same q at every step gives bit-identical outputs
    for s in range(7):
        layers[s]["q"] = layers[0]["q"]
    outs, _, _ = oracle.indexshare(layers, 0, vis, k, 1 / 24, kv_fp8=True, mtp_steps=7)
    assert all(np.array_equal(outs[0], outs[s]) for s in range(7))


# ------------------------------------------------------------------ context-parallel halves
def _shard_bounds(L, G, rs):
    cuts = np.sort(rs.choice(np.arange(1, L), size=G - 1, replace=False)) if G > 1 else []
    b = [0] + list(cuts) + [L]
    return list(zip(b[:-1], b[1:]))


@pytest.mark.parametrize("G", [1, 3, 8])
def test_topk_merge_of_shard_selections_equals_whole_row_selection(G):
    # the whole row's top-k lies inside the union of the shards' top-k's, and the
    # merge orders candidates as the whole-row selection does, so merging the
    # shards' selections must give oracle_topk of the whole row exactly; heavy
    # ties (scores from 7 values) make the position tie-break decide most slots
    rs = np.random.default_rng(300 + G)
    Q, L, k = 9, 700, 64
    scores = rs.choice(np.array([-2.5, -1.0, 0.0, 0.5, 1.0, 3.0, 7.25], np.float32), size=(Q, L))
    scores[0] = 1.0  # all equal
    vis = np.array([L, L, 5, 0, 64, 65, 300, 699, 1], np.int32)
    whole = oracle.topk(scores[:, None, :], vis[:, None], k)[:, 0]
    bounds = _shard_bounds(L, G, rs)
    cs, ci = [], []
    for lo, hi in bounds:
        lvis = np.clip(vis - lo, 0, hi - lo).astype(np.int32)
        local = oracle.topk(np.ascontiguousarray(scores[:, None, lo:hi]), lvis[:, None], k)[:, 0]
        c = oracle.topk_candidates(np.ascontiguousarray(scores[:, lo:hi]), local, lo)
        assert np.all((c[1] == -1) == (local == -1))
        cs.append(c[0])
        ci.append(c[1])
    merged = oracle.topk_merge(np.stack(cs), np.stack(ci), k)
    assert np.array_equal(merged, whole)
    # each shard's share of the whole selection, shifted back, is that selection
    back = []
    for lo, hi in bounds:
        loc = oracle.idx_localize(whole, lo, hi)
        for q in range(Q):
            row = loc[q]
            n = int((row >= 0).sum())
            assert np.all(row[n:] == -1) and np.all(np.diff(row[:n]) > 0)
            assert np.all(row[:n] < hi - lo)
        back.append(np.where(loc >= 0, loc + lo, -1))
    for q in range(Q):
        got = np.sort(np.concatenate([b[q][b[q] >= 0] for b in back]))
        assert np.array_equal(got, whole[q][whole[q] >= 0])


def test_topk_merge_edge_cases():
    cs = np.array([[[5.0, 1.0, -np.inf]], [[5.0, 9.0, 2.0]]], np.float32)  # [G=2][Q=1][3]
    ci = np.array([[[30, 2, -1]], [[7, 40, -1]]], np.int32)
    assert oracle.topk_merge(cs, ci, 2).tolist() == [[7, 40]]  # 9, then 5 at the lower position
    assert oracle.topk_merge(cs, ci, 3).tolist() == [[7, 30, 40]]
    assert oracle.topk_merge(cs, ci, 6).tolist() == [[2, 7, 30, 40, -1, -1]]  # empty slots never
    with pytest.raises(ValueError):  # one position offered twice
        oracle.topk_merge(cs, np.array([[[30, 2, -1]], [[30, 40, -1]]], np.int32), 2)
    with pytest.raises(ValueError):
        oracle.topk_merge(np.where(cs == 1.0, np.nan, cs).astype(np.float32), ci, 2)
    none = np.full((1, 1, 3), -1, np.int32)
    assert oracle.topk_merge(cs[:1], none, 2).tolist() == [[-1, -1]]


def _shard_attention(q, kv, idx, bounds, sm):
    po, pl = [], []
    for lo, hi in bounds:
        loc = oracle.idx_localize(idx, lo, hi)
        o, l = oracle.sparse_mla(q, np.ascontiguousarray(kv[:, lo:hi]), None, loc, sm)
        po.append(o)
        pl.append(l)
    return np.stack(po), np.stack(pl)


@pytest.mark.parametrize("G", [2, 5])
def test_lse_combine_of_shard_attention_equals_whole_attention(G):
    rs = np.random.default_rng(400 + G)
    B, T, L, k, sm = 2, 1, 96, 40, 1 / 24
    q = _bf16_bits(rs.standard_normal((B, T, 64, 576)) * 2)
    kv = _bf16_bits(rs.standard_normal((B, L, 576)))
    idx = np.stack([np.sort(rs.choice(L, size=k, replace=False)) for _ in range(B * T)]).reshape(
        B, T, k).astype(np.int32)
    idx[1, 0, -7:] = -1
    ref_o, ref_l, ref64 = oracle.sparse_mla(q, kv, None, idx, sm, want64=True)
    bounds = _shard_bounds(L, G, rs)
    po, pl = _shard_attention(q, kv, idx, bounds, sm)
    out, lse, out64 = oracle.lse_combine(po, pl, want64=True)
    # each shard output carries at most half a bf16 step (8 significant bits:
    # 2^-8 relative), so the weighted mean is within 2^-8 of the largest shard
    # value per element
    bound = 2.0 ** -8 * np.abs(_bits_to_f64(po)).max(axis=0) + 1e-12
    assert np.all(np.abs(out64 - ref64) <= bound)
    assert np.allclose(lse, ref_l, rtol=1e-6, atol=1e-6)
    assert np.array_equal(out, np.vectorize(oracle.round_bf16, otypes=[np.uint16])(out64))


def test_lse_combine_special_cases():
    rs = np.random.default_rng(7)
    po = _bf16_bits(rs.standard_normal((3, 2, 64, 512)))
    pl = rs.standard_normal((3, 2, 64)).astype(np.float32) * 4
    o1, l1 = oracle.lse_combine(po[:1], pl[:1])
    assert np.array_equal(o1, po[0]) and np.array_equal(l1, pl[0])  # one shard: identity
    pe = pl.copy()
    pe[1:] = -np.inf  # shards with no selected row weigh nothing
    o2, l2 = oracle.lse_combine(po, pe)
    assert np.array_equal(o2, po[0]) and np.array_equal(l2, pl[0])
    o3, l3 = oracle.lse_combine(po, np.full_like(pl, -np.inf))
    assert np.all(o3 == 0) and np.all(l3 == -np.inf)
    o4, l4 = oracle.lse_combine(np.stack([po[0], po[0]]), np.stack([pl[0], pl[0]]))
    assert np.array_equal(o4, po[0])  # two equal shards: the same mean, twice the mass
    assert np.allclose(l4, pl[0].astype(np.float64) + np.log(2.0), rtol=0, atol=1e-6)
    hi = pl.copy()
    hi[0] += 60.0  # one shard dominates: the others' weights fall below 2^-80
    o5, _ = oracle.lse_combine(po, hi)
    assert np.array_equal(o5, po[0])
