"""GPU parity of the HIP path (through the C ABI) against the CPU oracle, at
sizes the oracle finishes in seconds: several tiles, ragged tails, edge cases.
Expected values always come from the oracle run on host-generated inputs."""
import sys

import numpy as np
import pytest
import torch

import long_context_sparse_12_amd as lcs
import oracle
import synth
from synth import workloads as wl
from tests.parity import (DEV, bf16_to_f64, check_attention, check_scores, check_selection,
                          to_dev)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _zeros(nbytes):
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=DEV)


# ------------------------------------------------------------------ generator
def test_device_generator_matches_host():
    _say("case: generator device vs host")
    for tensor, R, D, perm, b0, nb, r0, nr in [(synth.T_IDX_KEY, 5000, 128, 100, 1, 2, 1000, 777),
                                               (synth.T_KV, 300, 576, 0, 0, 1, 0, 300),
                                               (synth.T_IDX_Q, 128, 128, 0, 3, 1, 0, 128)]:
        ch, sh = synth.host_fp8_rows(11, tensor, 3, R, D, perm, b0, nb, r0, nr)
        cd = torch.empty(nb * nr * D, dtype=torch.uint8, device=DEV)
        sd = torch.empty(nb * nr, dtype=torch.float32, device=DEV)
        synth.dev_fp8_rows(11, tensor, 3, R, D, perm, b0, nb, r0, nr, cd, sd)
        assert np.array_equal(cd.cpu().numpy(), ch.ravel())
        assert np.array_equal(sd.cpu().numpy().view(np.uint32), sh.ravel().view(np.uint32))
    bh = synth.host_bf16_rows(12, synth.T_ATT_Q, 2, 576, 1, 2, 5, 70)
    bd = torch.empty(2 * 70 * 576, dtype=torch.bfloat16, device=DEV)
    synth.dev_bf16_rows(12, synth.T_ATT_Q, 2, 576, 1, 2, 5, 70, bd)
    assert np.array_equal(bd.view(torch.int16).cpu().numpy().view(np.uint16), bh.ravel())
    uh = synth.host_uniform_rows(13, synth.T_IDX_W, 1, 32, 0, 3, 0, 9)
    ud = torch.empty(3 * 9 * 32, dtype=torch.float32, device=DEV)
    synth.dev_uniform_rows(13, synth.T_IDX_W, 1, 32, 0, 3, 0, 9, ud)
    assert np.array_equal(ud.cpu().numpy().view(np.uint32), uh.ravel().view(np.uint32))


# ------------------------------------------------------------------ indexer
@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 6, 7, 8, 16, 24, 37])
def test_idx_score_matches_oracle(T):
    """T < 16: the key-streaming kernel (up to 6 queries per pass, T = 7 and 8
    in two passes); T >= 16: the
    tiled prefill kernel (8-query chunks, 1024-key blocks; L = 8229 leaves a
    ragged last block and T = 37 a ragged last chunk)."""
    _say("case: idx_score T=%d" % T)
    B, L = 2, 8192 + 37
    w = wl.Workload("idx-parity", seed=40 + T, B=B, T=T, L=L, n_layers=1, plant_permyriad=100)
    inp = wl.host_indexer(w, 0)
    rs = np.random.default_rng(T)
    vis = rs.integers(L - 300, L + 1, size=(B, T)).astype(np.int32)
    vis[0, 0] = L
    if T > 1:
        vis[1, 1] = 100
    _, ref64 = oracle.idx_score(inp["q8"], inp["q_scale"], inp["w"], inp["k8"], inp["k_scale"],
                                vis, want64=True)
    scores = torch.empty((B, T, L), dtype=torch.float32, device=DEV)
    lcs.idx_score(to_dev(inp["q8"]), to_dev(inp["q_scale"]), to_dev(inp["w"]), to_dev(inp["k8"]),
                  to_dev(inp["k_scale"]), to_dev(vis), scores)
    rel = check_scores(scores.cpu().numpy(), ref64)
    _say("  max rel err %.3g" % rel)


@pytest.mark.parametrize("T", [2, 3, 4, 5, 6])
def test_idx_score_decode_many_tiles_per_wave(T):
    """The key-streaming kernel with 2-6 queries per pass over rows long enough
    that each wave scores 8 key tiles (2048 keys per workgroup), so both of its
    register buffers and, past 4 queries, the LDS-held head weights carry
    many tiles; B = 2 rows of 2^19 + 77 keys (a ragged last workgroup), one
    query cut at a visible length inside a checked window. Three windows of
    each row (start, middle, end) against the oracle."""
    B, L = 2, (1 << 19) + 77
    _say("case: idx_score decode many tiles T=%d L=%d" % (T, L))
    w = wl.Workload("idx-long", seed=60 + T, B=B, T=T, L=L, n_layers=1, plant_permyriad=100)
    rs = np.random.default_rng(100 + T)
    vis = rs.integers(L - 3000, L + 1, size=(B, T)).astype(np.int32)
    vis[0, 0] = L
    vis[1, T - 1] = (1 << 18) + 1000
    d = wl.dev_indexer(w, 0, DEV)
    scores = torch.empty((B, T, L), dtype=torch.float32, device=DEV)
    lcs.idx_score(d["q8"], d["q_scale"], d["w"], d["k8"], d["k_scale"], to_dev(vis), scores)
    torch.cuda.synchronize()
    del d
    n = 4096
    for r0 in (0, (1 << 18) - 100, L - n):
        inp = wl.host_indexer(w, 0, key_r0=r0, key_nr=n)
        vw = np.clip(vis.astype(np.int64) - r0, 0, n).astype(np.int32)
        _, ref64 = oracle.idx_score(inp["q8"], inp["q_scale"], inp["w"], inp["k8"],
                                    inp["k_scale"], vw, want64=True)
        rel = check_scores(scores[:, :, r0:r0 + n].cpu().numpy(), ref64, "window %d" % r0)
        _say("  window [%d, %d) max rel err %.3g" % (r0, r0 + n, rel))


def _finite_e4m3(rs, shape):
    """uniform over the 254 finite E4M3 codes (0x7F and 0xFF are NaN)"""
    c = rs.integers(0, 254, size=shape)
    return np.where(c < 0x7F, c, c + 1).astype(np.uint8)


@pytest.mark.parametrize("T", [1, 4, 6, 16, 21])
def test_idx_score_random_e4m3_bytes(T):
    """Codes drawn from every finite E4M3 byte (subnormals, both zeros, the
    largest magnitudes), positive scales spread over 2^-12 .. 2^12 and head
    weights in [0, 1) with exact zeros, plus edge rows: keys of all +0, all
    -0, only subnormals, all +-448; a query head of only subnormals and one
    of -0. Both kernels (T < 16 streams the keys, T >= 16 the tiled MFMA
    kernel) against the oracle. Head weights over 24 octaves let one head's
    dot product decide a score, and where it cancels the matrix cores'
    accumulation shows: the scores are held to 1e-3 of the terms' magnitude
    there (measured: within 1e-4 of it)."""
    B, L = 2, 3000 + 33
    _say("case: idx_score random E4M3 bytes T=%d" % T)
    rs = np.random.default_rng(500 + T)
    q8 = _finite_e4m3(rs, (B, T, 32, 128))
    k8 = _finite_e4m3(rs, (B, L, 128))
    sub = np.concatenate([np.arange(1, 8), np.arange(0x81, 0x88)]).astype(np.uint8)
    k8[0, 0] = 0x00
    k8[0, 1] = 0x80
    k8[0, 2] = rs.choice(sub, 128)
    k8[1, 5] = rs.choice(np.array([0x7E, 0xFE], np.uint8), 128)
    k8[1, L - 1] = rs.choice(sub, 128)
    q8[0, 0, 3] = rs.choice(sub, 128)
    q8[1, T - 1, 7] = 0x80
    q_scale = np.exp2(rs.uniform(-12, 12, size=(B, T, 32))).astype(np.float32)
    k_scale = np.exp2(rs.uniform(-12, 12, size=(B, L))).astype(np.float32)
    wt = rs.random((B, T, 32)).astype(np.float32)
    wt[wt < 0.1] = 0.0
    vis = rs.integers(L - 200, L + 1, size=(B, T)).astype(np.int32)
    _, ref64 = oracle.idx_score(q8, q_scale, wt, k8, k_scale, vis, want64=True)
    scores = torch.empty((B, T, L), dtype=torch.float32, device=DEV)
    lcs.idx_score(to_dev(q8), to_dev(q_scale), to_dev(wt), to_dev(k8), to_dev(k_scale),
                  to_dev(vis), scores)
    # magnitudes of the terms, decoded by torch's E4M3 cast (the head dot products
    # cancel here, and the matrix cores accumulate with less than fp32 precision)
    dec = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    terms = np.einsum("btj,btji,bsi->bts", wt.astype(np.float64) * q_scale, np.abs(dec[q8]),
                      np.abs(dec[k8])) * k_scale[:, None, :]
    got = scores.cpu().numpy()
    rel = check_scores(got, ref64, terms=terms)
    fin = np.isfinite(ref64)
    diff = np.abs(np.where(fin, got, 0) - np.where(fin, ref64, 0))
    over = float((diff / np.maximum(terms, 1e-300))[fin].max())
    _say("  max rel err %.3g; largest error over the terms' magnitude %.3g" % (rel, over))


@pytest.mark.parametrize("T", [1, 5, 16])
def test_idx_score_strided_cache(T):
    """Keys as a view k8[:, :L] of a cache of more positions per sequence (the
    batch stride passed through the C ABI is the cache's, not L); the rows past
    L hold other values and must not be read into the scores."""
    B, L, Lmax = 3, 5000, 7000
    _say("case: idx_score strided cache T=%d" % T)
    w = wl.Workload("idx-strided", seed=90 + T, B=B, T=T, L=Lmax, n_layers=1, plant_permyriad=100)
    inp = wl.host_indexer(w, 0)
    rs = np.random.default_rng(T)
    vis = rs.integers(L - 500, L + 1, size=(B, T)).astype(np.int32)
    _, ref64 = oracle.idx_score(inp["q8"], inp["q_scale"], inp["w"], inp["k8"][:, :L],
                                inp["k_scale"][:, :L], vis, want64=True)
    k8 = to_dev(inp["k8"])
    ks = to_dev(inp["k_scale"])
    scores = torch.empty((B, T, L), dtype=torch.float32, device=DEV)
    lcs.idx_score(to_dev(inp["q8"]), to_dev(inp["q_scale"]), to_dev(inp["w"]), k8[:, :L],
                  ks[:, :L], to_dev(vis), scores)
    rel = check_scores(scores.cpu().numpy(), ref64)
    _say("  max rel err %.3g" % rel)


def test_idx_score_prefill_full_size_sampled():
    """The chunked-prefill shape (4096 causal queries at the end of a 131072
    position cache), in the launch configuration the benchmark uses; rows
    sampled across the chunks and query ranges checked against the oracle."""
    w = wl.WORKLOADS["prefill"]
    _say("case: idx_score prefill full size %s" % w.name)
    B, T, L = w.B, w.T, w.L
    d = wl.dev_indexer(w, 0, DEV)
    vis = w.vis_len()
    scores = torch.empty((B, T, L), dtype=torch.float32, device=DEV)
    lcs.idx_score(d["q8"], d["q_scale"], d["w"], d["k8"], d["k_scale"], to_dev(vis), scores)
    torch.cuda.synchronize()
    del d
    inp = wl.host_indexer(w, 0)
    for t in (0, 7, 8, 1023, 2050, 4095):
        _, ref64 = oracle.idx_score(inp["q8"][:, t:t + 1], inp["q_scale"][:, t:t + 1],
                                    inp["w"][:, t:t + 1], inp["k8"], inp["k_scale"],
                                    vis[:, t:t + 1], want64=True)
        rel = check_scores(scores[:, t:t + 1].cpu().numpy(), ref64, "row t=%d" % t)
        _say("  t=%d max rel err %.3g" % (t, rel))


# ------------------------------------------------------------------ top-k
def _topk_case(name, B, T, L, k, seed):
    rs = np.random.default_rng(seed)
    vis = np.full((B, T), L, np.int32)
    if name == "normal":
        s = rs.standard_normal((B, T, L)).astype(np.float32)
    elif name == "ties":
        s = (rs.integers(0, 300, size=(B, T, L)) * 0.5).astype(np.float32)
    elif name == "equal":
        s = np.full((B, T, L), 3.0, np.float32)
    elif name == "ragged":
        s = rs.standard_normal((B, T, L)).astype(np.float32) * 100
        vis = rs.integers(0, L + 1, size=(B, T)).astype(np.int32)
        vis.flat[0] = 0
        vis.flat[-1] = min(L, k - 1) if L >= 1 else 0
        if vis.size > 2:
            vis.flat[1] = min(L, k)
            vis.flat[2] = min(L, k + 1)
    elif name == "signed-zero":
        s = rs.choice(np.array([-0.0, 0.0, 1.0, -1.0], np.float32), size=(B, T, L))
    elif name == "planted":
        s = np.abs(rs.standard_normal((B, T, L))).astype(np.float32) * 70
        s[..., rs.choice(L, 1311, replace=False)] += 200
    else:
        raise ValueError(name)
    return s, vis


TOPK_CASES = [
    ("normal", 1, 4, 8192, 2048), ("ragged", 2, 3, 8192 + 37, 2048), ("ties", 1, 2, 20000, 2048),
    ("equal", 1, 1, 10000, 2048), ("normal", 3, 1, 5000, 64), ("signed-zero", 1, 2, 9000, 1000),
    ("normal", 1, 2, 131072, 2048), ("planted", 2, 1, 131072, 2048), ("normal", 1, 300, 4001, 2048),
    ("ragged", 1, 5, 3001, 2048), ("normal", 1, 1, 1 << 20, 2048), ("ties", 1, 1, 1 << 20, 2048),
    ("normal", 2, 2, 1, 1), ("normal", 1, 1, 2048, 2048),
    # more entries around the threshold than the final kernel holds in
    # registers (16384): its passes over the lists in global memory
    ("equal", 1, 2, 40000, 2048),
    # >= 128 rows of <= 2^18 positions: the one-workgroup-per-row kernel
    ("normal", 1, 600, 4001, 2048), ("ragged", 1, 520, 20000, 2048),
    ("signed-zero", 2, 256, 3000, 1000), ("ties", 4, 128, 9000, 2048),
]


@pytest.mark.parametrize("case", TOPK_CASES, ids=lambda c: "%s-B%d-T%d-L%d-k%d" % c)
def test_topk_bit_exact_on_oracle_scores(case):
    name, B, T, L, k = case
    _say("case: topk %s B=%d T=%d L=%d k=%d" % case)
    s, vis = _topk_case(name, B, T, L, k, seed=B * 1000 + T * 10 + L % 97)
    ref = oracle.topk(s, vis, k)
    ds, dv = to_dev(s), to_dev(vis)
    idx = torch.full((B, T, k), -7, dtype=torch.int32, device=DEV)
    ws = _zeros(lcs.topk_workspace_bytes(B, T, L, k))
    lcs.topk_select(ds, dv, k, idx, ws)
    got = idx.cpu().numpy()
    bad = np.argwhere(np.any(got != ref, axis=-1))
    assert bad.size == 0, "rows differ: %s" % bad[:5].tolist()
    # the call restores the workspace's counters and histograms, so a second call on the
    # same workspace reproduces the result
    idx2 = torch.full((B, T, k), -9, dtype=torch.int32, device=DEV)
    lcs.topk_select(ds, dv, k, idx2, ws)
    assert torch.equal(idx, idx2)


@pytest.mark.parametrize("name", ["equal", "ties7"])
def test_topk_row_kernel_spills(name):
    """512 identical rows of 2^18 positions (the row kernel's largest L): with
    all-equal or 7-valued scores a wave's list gets up to 32768 entries, 2048
    in LDS and the rest in the workspace. Every row must give the oracle's
    selection of that row."""
    _say("case: topk row kernel spill %s" % name)
    B, T, L, k = 1, 512, 1 << 18, 2048
    rs = np.random.default_rng(7)
    if name == "equal":
        row = np.full(L, -1.5, np.float32)
    else:
        row = rs.choice(np.array([-3.0, -1.0, 0.0, 0.5, 2.0, 4.0, 9.0], np.float32), size=L)
    ref = oracle.topk(row[None, None, :], np.array([[L]], np.int32), k)[0, 0]
    ds = torch.from_numpy(row).to(DEV).view(1, 1, L).expand(B, T, L).contiguous()
    dv = torch.full((B, T), L, dtype=torch.int32, device=DEV)
    idx = torch.full((B, T, k), -7, dtype=torch.int32, device=DEV)
    ws = _zeros(lcs.topk_workspace_bytes(B, T, L, k))
    lcs.topk_select(ds, dv, k, idx, ws)
    got = idx.cpu().numpy()[0]
    bad = np.argwhere(np.any(got != ref[None, :], axis=-1))
    assert bad.size == 0, "rows differ: %s" % bad[:5].tolist()


def test_topk_row_kernel_sample_miss():
    """The row kernel estimates its threshold bucket from each wave's first
    1024 positions (wave w covers [w seg, (w+1) seg), seg = ceil(L / 8)). Here
    those windows hold 600 scores of 9, more than the sample rank it takes, so
    the estimate lands on the bucket of 9, while the true threshold lies among
    2000 tied scores of 8 placed outside the windows: the second compaction
    pass must run and keep the 1448 lowest-positioned 8s. 512 identical rows,
    against the oracle."""
    _say("case: topk row kernel sample miss")
    B, T, L, k = 1, 512, 100000, 2048
    rs = np.random.default_rng(11)
    row = rs.random(L).astype(np.float32)  # [0, 1): below both planted values
    seg = -(-L // 8)
    windows = np.concatenate([np.arange(w * seg, w * seg + 1024) for w in range(8)])
    outside = np.setdiff1d(np.arange(L), windows)
    row[rs.choice(windows, 600, replace=False)] = 9.0
    row[rs.choice(outside, 2000, replace=False)] = 8.0
    ref = oracle.topk(row[None, None, :], np.array([[L]], np.int32), k)[0, 0]
    assert (row[ref] == 9.0).sum() == 600 and (row[ref] == 8.0).sum() == k - 600
    ds = torch.from_numpy(row).to(DEV).view(1, 1, L).expand(B, T, L).contiguous()
    dv = torch.full((B, T), L, dtype=torch.int32, device=DEV)
    idx = torch.full((B, T, k), -7, dtype=torch.int32, device=DEV)
    ws = _zeros(lcs.topk_workspace_bytes(B, T, L, k))
    lcs.topk_select(ds, dv, k, idx, ws)
    got = idx.cpu().numpy()[0]
    bad = np.argwhere(np.any(got != ref[None, :], axis=-1))
    assert bad.size == 0, "rows differ: %s" % bad[:5].tolist()


def test_topk_workspace_reused_across_shapes():
    _say("case: topk workspace reuse")
    shapes = [(1, 1, 1 << 20, 2048), (4, 8, 30000, 2048), (1, 3, 7000, 512)]
    ws = _zeros(max(lcs.topk_workspace_bytes(*sh) for sh in shapes))
    for rep in range(2):
        for (B, T, L, k) in shapes:
            s, vis = _topk_case("ragged" if rep else "normal", B, T, L, k, seed=L + rep)
            idx = torch.empty((B, T, k), dtype=torch.int32, device=DEV)
            lcs.topk_select(to_dev(s), to_dev(vis), k, idx, ws)
            assert np.array_equal(idx.cpu().numpy(), oracle.topk(s, vis, k))


# ------------------------------------------------------------------ attention
def _attn_inputs(B, T, L, k, fp8, seed, pad=0, peak=False):
    rs = np.random.default_rng(seed)
    w = wl.Workload("attn-parity", seed=seed, B=B, T=T, L=L, n_layers=1, kv_fp8=fp8)
    q = wl.host_attn_q(w, 0)
    kv, sc = wl.host_kv(w, 0)
    idx = np.full((B, T, k), -1, np.int32)
    for b in range(B):
        for t in range(T):
            m = min(k - pad, L)
            idx[b, t, :m] = np.sort(rs.choice(L, m, replace=False))
    if peak:
        # every head's query points at the first selected row with logit 20, so the
        # output is close to that row: unit-scale outputs, where 2e-2 is tight
        for b in range(B):
            for t in range(T):
                s = idx[b, t, 0]
                if fp8:
                    r = np.array([oracle.e4m3(c) for c in kv[b, s]]) * float(sc[b, s])
                else:
                    r = bf16_to_f64(kv[b, s])
                qv = (r * (20.0 * 24.0 / np.dot(r, r))).astype(np.float32)
                q[b, t, :] = torch.from_numpy(qv).to(torch.bfloat16).view(torch.int16).numpy().view(
                    np.uint16)
    return q, kv, sc, idx


ATTN_CASES = [
    (1, 4, 8192, 2048, False, 0, False), (2, 3, 5000, 2048, True, 100, False),
    (40, 1, 3000, 2048, False, 0, False), (1, 1, 500, 100, False, 0, False),
    (300, 1, 4096, 2048, False, 7, False), (2, 1, 3000, 2048, False, 0, True), (2, 2, 3000, 1024, True, 0, True),
    (8, 1, 6000, 2048, True, 0, False), (1, 2, 200, 2048, True, 2048 - 200, False),
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=lambda c: "B%d-T%d-L%d-k%d-fp8%d-pad%d-peak%d" % c)
def test_sparse_mla_matches_oracle(case):
    B, T, L, k, fp8, pad, peak = case
    _say("case: sparse_mla B=%d T=%d L=%d k=%d fp8=%d pad=%d peak=%d" % case)
    q, kv, sc, idx = _attn_inputs(B, T, L, k, fp8, seed=B * 7 + T + L % 13, pad=pad, peak=peak)
    ref_out, ref_lse, ref64 = oracle.sparse_mla(q, kv, sc, idx, 1 / 24, want64=True)
    out = torch.empty((B, T, 64, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, T, 64), dtype=torch.float32, device=DEV)
    ws = _zeros(lcs.attn_workspace_bytes(B, T, k))
    lcs.sparse_mla_attn(to_dev(q), to_dev(kv), None if sc is None else to_dev(sc), to_dev(idx),
                        1 / 24, out, lse, ws)
    mx, ratio, lerr = check_attention(out, ref64, lse, ref_lse.astype(np.float64))
    _say("  max-abs %.3g (%.3g of rms), lse err %.3g" % (mx, ratio, lerr))


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_sparse_mla_strided_cache(fp8):
    """Latent rows (and FP8 row scales) as a view kv[:, :L] of a cache of more
    positions per sequence; selections reach the last row below L."""
    B, T, L, Lmax, k = 4, 1, 3000, 4100, 2048
    _say("case: sparse_mla strided cache fp8=%d" % fp8)
    w = wl.Workload("attn-strided", seed=95 + fp8, B=B, T=T, L=Lmax, n_layers=1, kv_fp8=fp8)
    q = wl.host_attn_q(w, 0)
    kv, sc = wl.host_kv(w, 0)
    rs = np.random.default_rng(3)
    idx = np.full((B, T, k), -1, np.int32)
    for b in range(B):
        sel = np.sort(np.concatenate([rs.choice(L - 1, k - 1 - b, replace=False), [L - 1]]))
        idx[b, 0, :len(sel)] = sel
    _, ref_lse, ref64 = oracle.sparse_mla(q, kv[:, :L], None if sc is None else sc[:, :L], idx,
                                          w.sm_scale, want64=True)
    kv_d = to_dev(kv)
    sc_d = None if sc is None else to_dev(sc)
    out = torch.empty((B, T, 64, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, T, 64), dtype=torch.float32, device=DEV)
    ws = _zeros(lcs.attn_workspace_bytes(B, T, k))
    lcs.sparse_mla_attn(to_dev(q), kv_d[:, :L], None if sc_d is None else sc_d[:, :L], to_dev(idx),
                        w.sm_scale, out, lse, ws)
    mx, ratio, lerr = check_attention(out, ref64, lse, ref_lse.astype(np.float64))
    _say("  max-abs %.3g (%.3g of rms), lse err %.3g" % (mx, ratio, lerr))


def test_sparse_mla_empty_selection():
    _say("case: sparse_mla all -1")
    q, kv, sc, idx = _attn_inputs(2, 1, 100, 64, False, seed=5)
    idx[:] = -1
    idx[1, 0, 10] = 7
    _, ref_lse, ref64 = oracle.sparse_mla(q, kv, sc, idx, 1 / 24, want64=True)
    out = torch.empty((2, 1, 64, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((2, 1, 64), dtype=torch.float32, device=DEV)
    ws = _zeros(lcs.attn_workspace_bytes(2, 1, 64))
    lcs.sparse_mla_attn(to_dev(q), to_dev(kv), None, to_dev(idx), 1 / 24, out, lse, ws)
    check_attention(out, ref64, lse, ref_lse.astype(np.float64))
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_sparse_mla_padding_rows(fp8):
    """Padding entries (-1) stand for no row: the kernels gather the
    sequence's own position 0 for them (paged: through its first table entry)
    and weight it zero, so a non-finite row 0 of an unmapped pool block does
    not matter. A query with no selected row outputs exact zeros and lse = -inf
    even where its sequence's position 0 is not finite. With and without
    splits (3 and 300 queries); paged equal to contiguous bit for bit."""
    from tests.test_gpu_paged import _pool
    for B, T in ((3, 1), (100, 3)):
        _say("case: sparse_mla padding rows, fp8=%d B=%d T=%d" % (fp8, B, T))
        L, k = 3000, 256
        q, kv, sc, idx = _attn_inputs(B, T, L, k, fp8, seed=17 + B, pad=40)
        idx[idx == 0] = -1  # row 0 is never selected (padding may sit in any slot)
        idx[0] = -1  # sequence 0: no selected row at all
        assert not (idx == 0).any() and (idx[1:] < 0).any()
        _, ref_lse, ref64 = oracle.sparse_mla(q, kv, sc, idx, 1 / 24, want64=True)
        bad_kv = kv.copy()
        bad_sc = None if sc is None else sc.copy()
        # non-finite position 0 in the sequence with no selection
        if fp8:
            bad_kv[0, 0] = 0x7F  # E4M3 NaN
            bad_sc[0, 0] = np.inf
        else:
            bad_kv[0, 0] = 0x7FC0  # bf16 NaN
        kv_d, idx_d, q_d = to_dev(bad_kv), to_dev(idx), to_dev(q)
        sc_d = None if sc is None else to_dev(bad_sc)
        ws = _zeros(lcs.attn_workspace_bytes(B, T, k))
        out = torch.empty((B, T, 64, 512), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((B, T, 64), dtype=torch.float32, device=DEV)
        lcs.sparse_mla_attn(q_d, kv_d, sc_d, idx_d, 1 / 24, out, lse, ws)
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all()
        assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
        check_attention(out, ref64, lse, ref_lse.astype(np.float64))
        # paged, with pool row 0 in a block no position maps to (the table uses
        # blocks 1..), NaN there too
        rs = np.random.default_rng(5 + B)
        nb_seq = (L + 63) // 64
        nb = B * nb_seq + 3
        table = np.zeros((B, nb_seq + 1), np.int32)
        table[:, :nb_seq] = 1 + rs.permutation(nb - 1)[:B * nb_seq].reshape(B, nb_seq)
        pos = np.arange(L)
        rows = torch.from_numpy(table[:, pos // 64].astype(np.int64) * 64 + pos % 64).to(DEV)
        pg = lcs.Paged(to_dev(table), 64, nb)
        kvp = _pool(kv_d, rows, nb, 64)
        scp = None if sc is None else _pool(sc_d, rows, nb, 64)
        flat = kvp.view((nb * 64,) + tuple(kvp.shape[2:]))
        if fp8:
            flat[0] = 0x7F
            scp.view(-1)[0] = float("inf")
        else:
            flat.view(torch.int16)[0] = 0x7FC0
        out_p = torch.empty_like(out)
        lse_p = torch.empty_like(lse)
        lcs.sparse_mla_attn_paged(q_d, kvp, scp, pg, idx_d, L, 1 / 24, out_p, lse_p, ws)
        torch.cuda.synchronize()
        assert torch.isfinite(out_p.float()).all()
        assert torch.equal(out_p.view(torch.int16), out.view(torch.int16))
        assert torch.equal(lse_p.view(torch.int32), lse.view(torch.int32))


@pytest.mark.parametrize("fp8", [True, False], ids=["fp8", "bf16"])
def test_sparse_mla_rows_past_32bit_offsets(fp8):
    """A sequence whose KV rows reach past 2^32 bytes (4.3 GB of KV for one
    sequence): the launcher then takes the 64-bit-addressed split-dims kernel.
    Positions spread over the whole range, the last eight rows included; the
    oracle runs on the gathered rows only (host-generated at those positions)."""
    row_bytes = 576 if fp8 else 1152
    L = (1 << 32) // row_bytes + 4096
    B, T, k = 1, 2, 2048
    _say("case: sparse_mla rows past 2^32 bytes, fp8=%d L=%d" % (fp8, L))
    w = wl.Workload("attn-long-rows", seed=11, B=B, T=T, L=L, n_layers=1, kv_fp8=fp8)
    kv, sc = wl.dev_kv(w, 0, DEV)
    q = wl.host_attn_q(w, 0)
    rs = np.random.default_rng(7)
    idx = np.empty((B, T, k), np.int32)
    for t in range(T):
        pos = np.unique(rs.integers(0, L - 8, size=3 * k))[: k - 8]
        pos = np.concatenate([pos, np.arange(L - 8, L)])
        assert len(pos) == k and pos[-1] * row_bytes >= (1 << 32)
        idx[0, t] = np.sort(rs.permutation(pos))
    out = torch.empty((B, T, 64, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, T, 64), dtype=torch.float32, device=DEV)
    ws = _zeros(lcs.attn_workspace_bytes(B, T, k))
    lcs.sparse_mla_attn(to_dev(q), kv, sc, to_dev(idx), 1 / 24, out, lse, ws)
    torch.cuda.synchronize()
    del kv, sc
    torch.cuda.empty_cache()
    for t in range(T):
        kv_s, sc_s = wl.host_kv_rows(w, 0, 0, idx[0, t])
        idx_s = np.arange(k, dtype=np.int32).reshape(1, 1, k)
        _, ref_lse, ref64 = oracle.sparse_mla(q[:, t:t + 1], kv_s, sc_s, idx_s, 1 / 24, want64=True)
        mx, ratio, lerr = check_attention(out[:, t:t + 1], ref64, lse[:, t:t + 1],
                                          ref_lse.astype(np.float64))
        _say("  t=%d max-abs %.3g, lse err %.3g" % (t, mx, lerr))


# ------------------------------------------------------------------ composite
def _dev_layers(layers):
    out = []
    for ly in layers:
        d = {}
        for f, a in ly.items():
            d[f] = None if a is None else to_dev(a)
        out.append(d)
    return out


def _run_composite(w, layers_h, sched, mtp_steps=0, mask=None):
    B, T, L, k = w.B, w.T, w.L, w.k
    vis = w.vis_len()
    layers_d = _dev_layers(layers_h)
    for ly in layers_d:
        ly["out"] = torch.empty((B, T, 64, 512), dtype=torch.bfloat16, device=DEV)
        ly["lse"] = torch.empty((B, T, 64), dtype=torch.float32, device=DEV)
    n_full = lcs.count_full_layers(sched, len(layers_h), mask, mtp_steps)
    idx_out = torch.empty((n_full, B, T, k), dtype=torch.int32, device=DEV)
    scores = torch.empty((B, T, L), dtype=torch.float32, device=DEV)
    ws = _zeros(lcs.indexshare_workspace_bytes(B, T, L, k))
    lcs.indexshare_forward(layers_d, sched, to_dev(vis), k, w.sm_scale, scores, idx_out, ws,
                           kv_dtype=lcs.KV_FP8_E4M3 if w.kv_fp8 else lcs.KV_BF16,
                           mtp_steps=mtp_steps, full_mask=mask)
    torch.cuda.synchronize()
    return layers_d, idx_out


def _host_layers(w, n, full_layers):
    layers = []
    for l in range(n):
        li = w.indexer_layer(l)
        ly = {}
        if l in full_layers:
            ly.update(wl.host_indexer(w, li))
        ly["q"] = wl.host_attn_q(w, l)
        kv, sc = wl.host_kv(w, li)
        ly["kv"] = kv
        if sc is not None:
            ly["kv_scale"] = sc
        layers.append(ly)
    return layers


def _compare_composite(w, layers_h, layers_d, idx_out, sched, mtp_steps=0, mask=None):
    vis = w.vis_len()
    outs, lses, ref_idx = oracle.indexshare(layers_h, sched, vis, w.k, w.sm_scale, kv_fp8=w.kv_fp8,
                                            mtp_steps=mtp_steps, mask=mask)
    got_idx = idx_out.cpu().numpy()
    full = w.full_layers() if mask is None else [l for l in range(len(layers_h)) if mask[l]]
    for f, l in enumerate(full):
        ly = layers_h[l]
        _, s64 = oracle.idx_score(ly["q8"], ly["q_scale"], ly["w"], ly["k8"], ly["k_scale"], vis,
                                  want64=True)
        ov, gap = check_selection(got_idx[f], ref_idx[f], s64)
        _say("  full layer %d: overlap %.5f worst gap %.3g" % (l, ov, gap))
    # every layer's attention against the oracle over the selection the GPU made
    # (the selection itself is checked above; attention is checked whatever it is)
    for l, ly in enumerate(layers_d):
        f = 0 if mtp_steps else sum(1 for x in full if x <= l) - 1
        src = layers_h[0 if mtp_steps else l]
        _, ref_lse, ref64 = oracle.sparse_mla(layers_h[l]["q"], src["kv"], src.get("kv_scale"),
                                              got_idx[f], w.sm_scale, want64=True)
        mx, _, lerr = check_attention(ly["out"], ref64, ly["lse"], ref_lse.astype(np.float64))
        _say("  layer %d attention max-abs %.3g, lse err %.3g" % (l, mx, lerr))


def test_indexshare_tiny_group_end_to_end():
    w = wl.WORKLOADS["tiny"]
    _say("case: composite %s" % w.name)
    layers_h = _host_layers(w, w.n_layers, w.full_layers())
    layers_d, idx_out = _run_composite(w, layers_h, wl.SCHED_GROUP4)
    _compare_composite(w, layers_h, layers_d, idx_out, wl.SCHED_GROUP4)


def test_indexshare_glm52_schedule_small():
    w = wl.Workload("glm52-small", seed=21, B=2, T=1, L=6000, n_layers=10, sched=wl.SCHED_GLM52,
                    kv_fp8=True)
    _say("case: composite %s" % w.name)
    layers_h = _host_layers(w, w.n_layers, w.full_layers())
    layers_d, idx_out = _run_composite(w, layers_h, lcs.SCHED_GLM52)
    assert idx_out.shape[0] == 4  # layers 0, 1, 2, 6
    _compare_composite(w, layers_h, layers_d, idx_out, lcs.SCHED_GLM52)
    # a shared layer's output equals a direct call with its full layer's selection
    for l, f in ((3, 2), (5, 2), (9, 3)):
        out = torch.empty_like(layers_d[l]["out"])
        ws = _zeros(lcs.attn_workspace_bytes(w.B, w.T, w.k))
        lcs.sparse_mla_attn(layers_d[l]["q"], layers_d[l]["kv"], layers_d[l]["kv_scale"],
                            idx_out[f], w.sm_scale, out, None, ws)
        assert torch.equal(out, layers_d[l]["out"])


FUSED_CASES = [
    # several chunks per row, GLM52 schedule (full layers 0, 1, 2, 6)
    ("chunks", 4, 20000, 2048, 7, wl.SCHED_GLM52,
     ([[20000], [13337], [1500], [0]], [[0], [19999], [2048], [20000]])),
    # one chunk per row (L <= 2048) with rows longer than k
    ("one-chunk", 3, 2000, 1000, 2, wl.SCHED_GROUP4,
     ([[2000], [1001], [999]], [[1000], [0], [2000]])),
    # >= 128 rows of <= 2^18 positions: the one-workgroup-per-row top-k, so
    # the composite keeps the indexer and the selection separate
    ("row-kernel", 520, 3000, 2048, 2, wl.SCHED_GROUP4,
     ([[3000]] * 519 + [[100]], [[2049]] * 520)),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: c[0])
def test_composite_fused_histogram_matches_separate_calls(case):
    """With one query per sequence the composite call builds the selection's
    first histogram inside the indexer launch (when the selection takes the
    chunked launches), and each selection leaves it zero for the next full
    layer (one clear per call). Every full layer's selection must equal
    separate idx_score + topk_select calls (each checked against the oracle
    elsewhere) bit for bit, for rows whose visible length is L, ragged, at
    most k (every position kept) and 0, over two calls that share one
    workspace filled with non-zero bytes."""
    name, B, L, k, n, sched, vis_sets = case
    w = wl.Workload("fused-" + name, seed=25, B=B, T=1, L=L, n_layers=n, sched=sched,
                    kv_fp8=True, k=k)
    _say("case: composite fused histogram %s B=%d L=%d k=%d" % (name, B, L, k))
    full = w.full_layers()
    T = 1
    layers = []
    for l in range(n):
        d = wl.dev_indexer(w, l, DEV) if l in full else {}
        d["q"] = wl.dev_attn_q(w, l, DEV)
        d["kv"], d["kv_scale"] = wl.dev_kv(w, l, DEV)
        d["out"] = torch.empty((B, T, 64, 512), dtype=torch.bfloat16, device=DEV)
        d["lse"] = torch.empty((B, T, 64), dtype=torch.float32, device=DEV)
        layers.append(d)
    idx_out = torch.empty((len(full), B, T, k), dtype=torch.int32, device=DEV)
    scores = torch.empty((B, T, L), dtype=torch.float32, device=DEV)
    ws = torch.full((lcs.indexshare_workspace_bytes(B, T, L, k),), 0x5A, dtype=torch.uint8,
                    device=DEV)  # not zero: the call clears what it needs
    tk_ws = _zeros(lcs.topk_workspace_bytes(B, T, L, k))
    ref = torch.empty((B, T, k), dtype=torch.int32, device=DEV)
    for vis in vis_sets:
        vis_d = to_dev(np.array(vis, np.int32))
        lcs.indexshare_forward(layers, sched, vis_d, k, w.sm_scale, scores, idx_out, ws,
                               kv_dtype=lcs.KV_FP8_E4M3)
        torch.cuda.synchronize()
        got = idx_out.cpu().numpy()
        for f, l in enumerate(full):
            ly = layers[l]
            lcs.idx_score(ly["q8"], ly["q_scale"], ly["w"], ly["k8"], ly["k_scale"], vis_d, scores)
            lcs.topk_select(scores, vis_d, k, ref, tk_ws)
            torch.cuda.synchronize()
            want = ref.cpu().numpy()
            bad = np.argwhere(got[f] != want)
            _say("  full layer %d: %d mismatches" % (l, len(bad)))
            assert bad.size == 0, (l, bad[:5])
    del layers, scores, ws
    torch.cuda.empty_cache()


def test_composite_decode128k_full_size_sampled():
    """The 128K decode group at full size (B=32, T=1, L=131072, layer 0 full,
    layers 1-3 reuse its selection, bf16 KV) through lcs_indexshare_forward in
    the benchmark's launch configuration (one query per sequence, so the
    indexer also builds the top-k histogram). Sampled sequences against the
    oracle: the selection under the gap rule, and every layer's output and
    lse over the selection the GPU made."""
    w = wl.WORKLOADS["decode128k"]
    _say("case: composite full size %s" % w.name)
    B, T, L, k = w.B, w.T, w.L, w.k
    full = w.full_layers()
    assert full == [0]
    layers = []
    for l in range(w.n_layers):
        d = wl.dev_indexer(w, l, DEV) if l in full else {}
        d["q"] = wl.dev_attn_q(w, l, DEV)
        kv, sc = wl.dev_kv(w, l, DEV)
        d["kv"] = kv
        if sc is not None:
            d["kv_scale"] = sc
        d["out"] = torch.empty((B, T, 64, 512), dtype=torch.bfloat16, device=DEV)
        d["lse"] = torch.empty((B, T, 64), dtype=torch.float32, device=DEV)
        layers.append(d)
    vis = w.vis_len()
    idx_out = torch.empty((len(full), B, T, k), dtype=torch.int32, device=DEV)
    scores = torch.empty((B, T, L), dtype=torch.float32, device=DEV)
    ws = _zeros(lcs.indexshare_workspace_bytes(B, T, L, k))
    lcs.indexshare_forward(layers, lcs.SCHED_GROUP4, to_dev(vis), k, w.sm_scale, scores, idx_out,
                           ws, kv_dtype=lcs.KV_BF16)
    torch.cuda.synchronize()
    got = idx_out.cpu().numpy()
    for b in (0, 19, 31):
        inp = wl.host_indexer(w, 0, b0=b, nb=1)
        s32, s64 = oracle.idx_score(inp["q8"], inp["q_scale"], inp["w"], inp["k8"],
                                    inp["k_scale"], vis[b:b + 1], want64=True)
        ref_idx = oracle.topk(s32, vis[b:b + 1], k)
        ov, gap = check_selection(got[0, b:b + 1], ref_idx, s64)
        _say("  b=%d selection overlap %.5f worst gap %.3g" % (b, ov, gap))
        sel = got[0, b, 0]
        idx_s = np.arange(k, dtype=np.int32).reshape(1, 1, k)
        for l in range(w.n_layers):
            q_h = wl.host_attn_q(w, l, b0=b, nb=1)
            kv_s, sc_s = wl.host_kv_rows(w, l, b, sel)
            _, ref_lse, ref64 = oracle.sparse_mla(q_h, kv_s, sc_s, idx_s, w.sm_scale, want64=True)
            mx, _, lerr = check_attention(layers[l]["out"][b:b + 1], ref64,
                                          layers[l]["lse"][b:b + 1], ref_lse.astype(np.float64))
            _say("  b=%d layer %d max-abs %.3g, lse err %.3g" % (b, l, mx, lerr))
    del layers, scores, ws
    torch.cuda.empty_cache()


def test_composite_decode1m_full_size_sampled():
    """The 1M decode schedule at full size (B=2, T=1, L=2^20, 78 layers, 21
    full under the GLM-5.2 schedule, E4M3 KV) through lcs_indexshare_forward
    as the benchmark launches it. Sequence 1 against the oracle: the
    selections of full layers 0 and 74 (the first and the last: the fused
    histogram restarted from zero 20 times in between) under the gap rule,
    and the outputs of layers 0, 1, 74 and 77 over the GPU's selections."""
    w = wl.WORKLOADS["decode1m"]
    _say("case: composite full size %s" % w.name)
    B, T, L, k = w.B, w.T, w.L, w.k
    full = w.full_layers()
    assert len(full) == 21 and full[-1] == 74
    layers = []
    for l in range(w.n_layers):
        d = wl.dev_indexer(w, l, DEV) if l in full else {}
        d["q"] = wl.dev_attn_q(w, l, DEV)
        kv, sc = wl.dev_kv(w, l, DEV)
        d["kv"], d["kv_scale"] = kv, sc
        d["out"] = torch.empty((B, T, 64, 512), dtype=torch.bfloat16, device=DEV)
        d["lse"] = torch.empty((B, T, 64), dtype=torch.float32, device=DEV)
        layers.append(d)
    vis = w.vis_len()
    idx_out = torch.empty((len(full), B, T, k), dtype=torch.int32, device=DEV)
    scores = torch.empty((B, T, L), dtype=torch.float32, device=DEV)
    ws = _zeros(lcs.indexshare_workspace_bytes(B, T, L, k))
    lcs.indexshare_forward(layers, lcs.SCHED_GLM52, to_dev(vis), k, w.sm_scale, scores, idx_out,
                           ws, kv_dtype=lcs.KV_FP8_E4M3)
    torch.cuda.synchronize()
    got = idx_out.cpu().numpy()
    b = 1
    for f in (0, 20):
        l = full[f]
        inp = wl.host_indexer(w, l, b0=b, nb=1)
        s32, s64 = oracle.idx_score(inp["q8"], inp["q_scale"], inp["w"], inp["k8"],
                                    inp["k_scale"], vis[b:b + 1], want64=True)
        ref_idx = oracle.topk(s32, vis[b:b + 1], k)
        ov, gap = check_selection(got[f, b:b + 1], ref_idx, s64)
        _say("  layer %d selection overlap %.5f worst gap %.3g" % (l, ov, gap))
    idx_s = np.arange(k, dtype=np.int32).reshape(1, 1, k)
    for l in (0, 1, 74, 77):
        f = sum(1 for x in full if x <= l) - 1
        sel = got[f, b, 0]
        q_h = wl.host_attn_q(w, l, b0=b, nb=1)
        kv_s, sc_s = wl.host_kv_rows(w, l, b, sel)
        _, ref_lse, ref64 = oracle.sparse_mla(q_h, kv_s, sc_s, idx_s, w.sm_scale, want64=True)
        mx, _, lerr = check_attention(layers[l]["out"][b:b + 1], ref64,
                                      layers[l]["lse"][b:b + 1], ref_lse.astype(np.float64))
        _say("  layer %d max-abs %.3g, lse err %.3g" % (l, mx, lerr))
    del layers, scores, ws
    torch.cuda.empty_cache()


def test_composite_prefill_and_mtp_full_size_sampled():
    """The chunked prefill (B=1, T=4096 causal queries, L=131072, 4 layers,
    bf16 KV; the top-k takes the one-workgroup-per-row kernel) and the MTP
    draft round (B=8, L=2^20, 7 steps on step 0's selection and KV, E4M3) at
    full size through lcs_indexshare_forward as the benchmark launches them;
    sampled queries against the oracle as in the decode tests."""
    for name, sched, mtp, samples, att_layers in (
            ("prefill", lcs.SCHED_GROUP4, 0, ((0, 0), (0, 1500), (0, 4095)), (0, 3)),
            ("mtp1m", 0, 7, ((3, 0),), (0, 6))):
        w = wl.WORKLOADS[name]
        _say("case: composite full size %s" % w.name)
        B, T, L, k = w.B, w.T, w.L, w.k
        n = w.n_layers
        layers = []
        for l in range(n):
            li = w.indexer_layer(l)
            d = wl.dev_indexer(w, l, DEV) if l in w.full_layers() else {}
            d["q"] = wl.dev_attn_q(w, l, DEV)
            if li == l:
                kv, sc = wl.dev_kv(w, l, DEV)
                d["kv"] = kv
                if sc is not None:
                    d["kv_scale"] = sc
            d["out"] = torch.empty((B, T, 64, 512), dtype=torch.bfloat16, device=DEV)
            d["lse"] = torch.empty((B, T, 64), dtype=torch.float32, device=DEV)
            layers.append(d)
        vis = w.vis_len()
        n_full = lcs.count_full_layers(sched, n, None, mtp)
        idx_out = torch.empty((n_full, B, T, k), dtype=torch.int32, device=DEV)
        scores = torch.empty((B, T, L), dtype=torch.float32, device=DEV)
        ws = _zeros(lcs.indexshare_workspace_bytes(B, T, L, k))
        lcs.indexshare_forward(layers, sched, to_dev(vis), k, w.sm_scale, scores, idx_out, ws,
                               kv_dtype=lcs.KV_FP8_E4M3 if w.kv_fp8 else lcs.KV_BF16,
                               mtp_steps=mtp)
        torch.cuda.synchronize()
        got = idx_out.cpu().numpy()
        idx_s = np.arange(k, dtype=np.int32).reshape(1, 1, k)
        for b, t in samples:
            inp = wl.host_indexer(w, 0, b0=b, nb=1)
            q_sl = (slice(None), slice(t, t + 1))
            s32, s64 = oracle.idx_score(inp["q8"][q_sl], inp["q_scale"][q_sl], inp["w"][q_sl],
                                        inp["k8"], inp["k_scale"], vis[b:b + 1, t:t + 1],
                                        want64=True)
            ref_idx = oracle.topk(s32, vis[b:b + 1, t:t + 1], k)
            ov, gap = check_selection(got[0, b:b + 1, t:t + 1], ref_idx, s64)
            _say("  b=%d t=%d selection overlap %.5f worst gap %.3g" % (b, t, ov, gap))
            sel = got[0, b, t]
            kv_s, sc_s = wl.host_kv_rows(w, 0, b, sel[sel >= 0])
            idx_v = np.full((1, 1, k), -1, np.int32)
            idx_v[0, 0, :int((sel >= 0).sum())] = np.arange(int((sel >= 0).sum()), dtype=np.int32)
            for l in att_layers:
                if not mtp:
                    kv_s, sc_s = wl.host_kv_rows(w, l, b, sel[sel >= 0])
                q_h = wl.host_attn_q(w, l, b0=b, nb=1)[:, t:t + 1]
                _, ref_lse, ref64 = oracle.sparse_mla(q_h, kv_s, sc_s, idx_v, w.sm_scale,
                                                      want64=True)
                mx, _, lerr = check_attention(layers[l]["out"][b:b + 1, t:t + 1], ref64,
                                              layers[l]["lse"][b:b + 1, t:t + 1],
                                              ref_lse.astype(np.float64))
                _say("  b=%d t=%d layer %d max-abs %.3g, lse err %.3g" % (b, t, l, mx, lerr))
        del layers, scores, ws, idx_out
        torch.cuda.empty_cache()


def test_mtp_draft_reuse_small():
    w = wl.Workload("mtp-small", seed=22, B=3, T=1, L=7000, n_layers=7, kv_fp8=True, mtp_steps=7)
    _say("case: composite %s" % w.name)
    layers_h = _host_layers(w, 7, [0])
    layers_d, idx_out = _run_composite(w, layers_h, 0, mtp_steps=7)
    assert idx_out.shape[0] == 1
    _compare_composite(w, layers_h, layers_d, idx_out, 0, mtp_steps=7)
    # same q at every step -> bit-identical outputs (same selection, same KV)
    for ly in layers_d:
        ly["q"] = layers_d[0]["q"]
    layers_d2, _ = _run_composite(w, [dict(layers_h[0], q=layers_h[0]["q"])] +
                                  [dict(ly, q=layers_h[0]["q"]) for ly in layers_h[1:]], 0,
                                  mtp_steps=7)
    for ly in layers_d2[1:]:
        assert torch.equal(ly["out"], layers_d2[0]["out"])


def test_verify_multi_token_small():
    """MTP verify / multi-token decode: 1 + 5 draft tokens per sequence in one
    pass, causal among themselves, through the whole group."""
    w = wl.Workload("verify-small", seed=24, B=3, T=6, L=7000, n_layers=4, prefix=7000 - 6,
                    plant_permyriad=100)
    _say("case: composite %s" % w.name)
    layers_h = _host_layers(w, 4, [0])
    layers_d, idx_out = _run_composite(w, layers_h, lcs.SCHED_GROUP4)
    _compare_composite(w, layers_h, layers_d, idx_out, lcs.SCHED_GROUP4)


def test_prefill_causal_small():
    w = wl.Workload("prefill-small", seed=23, B=1, T=40, L=9000, n_layers=4, prefix=9000 - 40)
    _say("case: composite %s" % w.name)
    layers_h = _host_layers(w, 4, [0])
    layers_d, idx_out = _run_composite(w, layers_h, wl.SCHED_GROUP4)
    _compare_composite(w, layers_h, layers_d, idx_out, wl.SCHED_GROUP4)


def test_composite_verify128k_full_size_sampled():
    """The multi-token verify at full size (B=32, T=1+5 causal queries per
    sequence at the end of a 131072-position cache, one 4-layer group, bf16
    KV) through lcs_indexshare_forward as the benchmark launches it: the six
    queries share one pass over the keys, 16 key tiles per wave. Sampled
    queries against the oracle: their scores (the call leaves the full
    layer's scores in its scratch), selections under the gap rule, and the
    outputs of layers 0 and 3 over the GPU's selection."""
    w = wl.WORKLOADS["verify128k"]
    _say("case: composite full size %s" % w.name)
    B, T, L, k = w.B, w.T, w.L, w.k
    layers = []
    for l in range(w.n_layers):
        d = wl.dev_indexer(w, l, DEV) if l in w.full_layers() else {}
        d["q"] = wl.dev_attn_q(w, l, DEV)
        d["kv"], _ = wl.dev_kv(w, l, DEV)
        d["out"] = torch.empty((B, T, 64, 512), dtype=torch.bfloat16, device=DEV)
        d["lse"] = torch.empty((B, T, 64), dtype=torch.float32, device=DEV)
        layers.append(d)
    vis = w.vis_len()
    idx_out = torch.empty((1, B, T, k), dtype=torch.int32, device=DEV)
    scores = torch.empty((B, T, L), dtype=torch.float32, device=DEV)
    ws = _zeros(lcs.indexshare_workspace_bytes(B, T, L, k))
    lcs.indexshare_forward(layers, lcs.SCHED_GROUP4, to_dev(vis), k, w.sm_scale, scores, idx_out,
                           ws, kv_dtype=lcs.KV_BF16)
    torch.cuda.synchronize()
    got = idx_out.cpu().numpy()
    idx_s = np.arange(k, dtype=np.int32).reshape(1, 1, k)
    for b, t in ((0, 0), (13, 3), (31, 5)):
        inp = wl.host_indexer(w, 0, b0=b, nb=1)
        q_sl = (slice(None), slice(t, t + 1))
        s32, s64 = oracle.idx_score(inp["q8"][q_sl], inp["q_scale"][q_sl], inp["w"][q_sl],
                                    inp["k8"], inp["k_scale"], vis[b:b + 1, t:t + 1], want64=True)
        rel = check_scores(scores[b:b + 1, t:t + 1].cpu().numpy(), s64, "b=%d t=%d" % (b, t))
        ref_idx = oracle.topk(s32, vis[b:b + 1, t:t + 1], k)
        ov, gap = check_selection(got[0, b:b + 1, t:t + 1], ref_idx, s64)
        _say("  b=%d t=%d scores max rel %.3g, selection overlap %.5f worst gap %.3g"
             % (b, t, rel, ov, gap))
        sel = got[0, b, t]
        for l in (0, 3):
            q_h = wl.host_attn_q(w, l, b0=b, nb=1)[:, t:t + 1]
            kv_s, sc_s = wl.host_kv_rows(w, l, b, sel)
            _, ref_lse, ref64 = oracle.sparse_mla(q_h, kv_s, sc_s, idx_s, w.sm_scale, want64=True)
            mx, _, lerr = check_attention(layers[l]["out"][b:b + 1, t:t + 1], ref64,
                                          layers[l]["lse"][b:b + 1, t:t + 1],
                                          ref_lse.astype(np.float64))
            _say("  b=%d t=%d layer %d max-abs %.3g, lse err %.3g" % (b, t, l, mx, lerr))
    del layers, scores, ws
    torch.cuda.empty_cache()
