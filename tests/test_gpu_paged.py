"""GPU parity of the paged-KV calls (through the C ABI): the same logical
caches laid out in pools of blocks, in a random block order with garbage in
every pool row no position maps to, must give the oracle's results on the
logical caches (scores, selections, attention outputs, under the usual
tolerances) and the contiguous calls' results bit for bit, and the paged
cache append must write what the oracle's append writes into the logical
cache."""
import sys

import numpy as np
import pytest
import torch

import long_context_sparse_12_amd as lcs
import oracle
from synth import workloads as wl
from tests.parity import DEV, check_attention, check_scores, check_selection, to_dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _zeros(nbytes):
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=DEV)


def _layout(B, L, bs, seed, spare=3):
    """block table [B][max_blocks] (one unused entry per sequence) over a pool of
    B * ceil(L / bs) + spare blocks in random order; the pool row of every
    (b, p) as a device tensor [B][L]"""
    rs = np.random.default_rng(seed)
    nb_seq = (L + bs - 1) // bs
    n_blocks = B * nb_seq + spare
    perm = rs.permutation(n_blocks)[:B * nb_seq].reshape(B, nb_seq)
    table = np.zeros((B, nb_seq + 1), np.int32)
    table[:, :nb_seq] = perm
    p = np.arange(L)
    rows = table[:, p // bs].astype(np.int64) * bs + p % bs
    return lcs.Paged(to_dev(table), bs, n_blocks), torch.from_numpy(rows).to(DEV), n_blocks


def _pool(cache, rows, n_blocks, bs):
    """pool [n_blocks][bs][...] holding cache [B][L][...] at `rows`, random
    bytes everywhere else"""
    tail = tuple(cache.shape[2:])
    nbytes = n_blocks * bs * int(np.prod(tail, dtype=np.int64)) * cache.element_size()
    g = torch.Generator(device=DEV).manual_seed(n_blocks)
    raw = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=DEV, generator=g)
    pool = raw.view(cache.dtype).view((n_blocks * bs,) + tail)
    if cache.dtype == torch.float32:  # garbage scales: finite
        pool.copy_(torch.rand_like(pool) * 3 + 0.5)
    pool[rows.reshape(-1)] = cache.reshape((-1,) + tail)
    return pool.view((n_blocks, bs) + tail)


IDX_CASES = [  # (B, T, L, bs)
    (2, 1, 8229, 64), (3, 3, 5000, 128), (1, 4, 20000, 1024), (2, 37, 3000, 64), (1, 16, 2500, 256),
]


@pytest.mark.parametrize("case", IDX_CASES, ids=lambda c: "B%d-T%d-L%d-bs%d" % c)
def test_idx_score_paged_equals_contiguous(case):
    B, T, L, bs = case
    _say("case: idx_score paged B=%d T=%d L=%d bs=%d" % case)
    w = wl.Workload("paged-idx", seed=70 + T, B=B, T=T, L=L, n_layers=1, plant_permyriad=100,
                    prefix=(L - T) if T > 1 else -1)
    d = wl.dev_indexer(w, 0, DEV)
    vis = torch.from_numpy(w.vis_len()).to(DEV)
    ref = torch.empty((B, T, L), dtype=torch.float32, device=DEV)
    lcs.idx_score(d["q8"], d["q_scale"], d["w"], d["k8"], d["k_scale"], vis, ref)
    pg, rows, nb = _layout(B, L, bs, seed=L + bs)
    k8p = _pool(d["k8"], rows, nb, bs)
    ksp = _pool(d["k_scale"], rows, nb, bs)
    got = torch.full((B, T, L), 7.0, dtype=torch.float32, device=DEV)
    lcs.idx_score_paged(d["q8"], d["q_scale"], d["w"], k8p, ksp, pg, vis, L, got)
    torch.cuda.synchronize()
    inp = wl.host_indexer(w, 0)
    _, ref64 = oracle.idx_score(inp["q8"], inp["q_scale"], inp["w"], inp["k8"], inp["k_scale"],
                                w.vis_len(), want64=True)
    rel = check_scores(got.cpu().numpy(), ref64)
    _say("  against the oracle: max rel err %.3g" % rel)
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))


ATTN_CASES = [  # (B, T, L, k, fp8, bs, pad)
    (2, 1, 5000, 2048, False, 64, 0), (2, 1, 5000, 2048, True, 128, 100), (40, 1, 3000, 2048, True, 64, 0),
    (1, 3, 9000, 100, False, 512, 7), (8, 1, 6000, 2048, False, 64, 0), (3, 2, 4100, 1024, True, 1024, 0),
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=lambda c: "B%d-T%d-L%d-k%d-fp8%d-bs%d-pad%d" % c)
def test_sparse_mla_paged_equals_contiguous(case):
    B, T, L, k, fp8, bs, pad = case
    _say("case: sparse_mla paged B=%d T=%d L=%d k=%d fp8=%d bs=%d pad=%d" % case)
    rs = np.random.default_rng(B * 11 + L)
    w = wl.Workload("paged-attn", seed=80 + B, B=B, T=T, L=L, n_layers=1, kv_fp8=fp8)
    q = wl.dev_attn_q(w, 0, DEV)
    kv, sc = wl.dev_kv(w, 0, DEV)
    idx = np.full((B, T, k), -1, np.int32)
    for b in range(B):
        for t in range(T):
            m = min(k - pad, L)
            idx[b, t, :m] = np.sort(rs.choice(L, m, replace=False))
    idx_d = to_dev(idx)
    ws = _zeros(lcs.attn_workspace_bytes(B, T, k))
    out_r = torch.empty((B, T, 64, 512), dtype=torch.bfloat16, device=DEV)
    lse_r = torch.empty((B, T, 64), dtype=torch.float32, device=DEV)
    lcs.sparse_mla_attn(q, kv, sc, idx_d, w.sm_scale, out_r, lse_r, ws)
    pg, rows, nb = _layout(B, L, bs, seed=L + bs + 1)
    kvp = _pool(kv, rows, nb, bs)
    scp = None if sc is None else _pool(sc, rows, nb, bs)
    out = torch.empty_like(out_r)
    lse = torch.empty_like(lse_r)
    lcs.sparse_mla_attn_paged(q, kvp, scp, pg, idx_d, L, w.sm_scale, out, lse, ws)
    torch.cuda.synchronize()
    kv_h, sc_h = wl.host_kv(w, 0)
    _, ref_lse, ref64 = oracle.sparse_mla(wl.host_attn_q(w, 0), kv_h, sc_h, idx, w.sm_scale,
                                          want64=True)
    mx, _, lerr = check_attention(out, ref64, lse, ref_lse.astype(np.float64))
    _say("  against the oracle: max-abs %.3g, lse err %.3g" % (mx, lerr))
    assert torch.equal(out.view(torch.int16), out_r.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse_r.view(torch.int32))


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_cache_append_paged_matches_oracle(fp8):
    """the logical caches read back through the table equal the oracle's
    append on the logical caches before; pool rows no position maps to keep
    their bytes"""
    _say("case: cache_append paged fp8=%d" % fp8)
    B, T, L, bs = 3, 5, 300, 64
    rs = np.random.default_rng(91 + fp8)
    pg, rows, nb = _layout(B, L, bs, seed=93)
    # distinct positions per sequence in [-4, L + 4): row 0 and row L - 1 are
    # written, some tokens are skipped
    pos = np.stack([rs.permutation(L + 8)[:T] - 4 for _ in range(B)]).astype(np.int32)
    pos[0] = np.concatenate([[0], 1 + rs.permutation(L + 3)[:T - 1]])
    pos[1] = np.concatenate([[L - 1], rs.permutation(L - 1)[:T - 1]])
    k_new = torch.randn((B, T, 128), device=DEV).to(torch.bfloat16)
    kv_new = torch.randn((B, T, 576), device=DEV).to(torch.bfloat16)
    g = torch.Generator(device=DEV).manual_seed(5)
    k8p = torch.randint(0, 256, (nb, bs, 128), dtype=torch.uint8, device=DEV, generator=g)
    ksp = torch.rand((nb, bs), device=DEV, generator=g)
    if fp8:
        kvp = torch.randint(0, 256, (nb, bs, 576), dtype=torch.uint8, device=DEV, generator=g)
        kvsp = torch.rand((nb, bs), device=DEV, generator=g)
    else:
        kvp = torch.randint(-30000, 30000, (nb, bs, 576), dtype=torch.int16, device=DEV,
                            generator=g).view(torch.bfloat16)
        kvsp = None
    flat = rows.reshape(-1)

    def logical(pool):
        return pool.reshape((nb * bs,) + tuple(pool.shape[2:]))[flat].reshape(
            (B, L) + tuple(pool.shape[2:])).cpu().numpy()
    before = [logical(k8p), logical(ksp),
              logical(kvp) if fp8 else logical(kvp.view(torch.int16)).view(np.uint16),
              logical(kvsp) if fp8 else None]
    pools_before = [x.clone() for x in (k8p, ksp, kvp) + ((kvsp,) if fp8 else ())]
    ref = oracle.cache_append(k_new.view(torch.int16).cpu().numpy().view(np.uint16),
                              kv_new.view(torch.int16).cpu().numpy().view(np.uint16), pos,
                              before[0], before[1], before[2], before[3])
    lcs.cache_append_paged(to_dev(pos), L, pg, k_new=k_new, k8_pool=k8p, k_scale_pool=ksp,
                           kv_new=kv_new, kv_pool=kvp, kv_scale_pool=kvsp)
    torch.cuda.synchronize()
    after = [logical(k8p), logical(ksp),
             logical(kvp) if fp8 else logical(kvp.view(torch.int16)).view(np.uint16),
             logical(kvsp) if fp8 else None]
    for name, a, r in zip(("k8", "k_scale", "kv", "kv_scale"), after, ref):
        if r is not None:
            assert np.array_equal(a.view(np.uint8), r.view(np.uint8)), name
    # rows outside the logical caches: untouched
    mapped = torch.zeros(nb * bs, dtype=torch.bool, device=DEV)
    mapped[flat] = True
    for p_now, p_old in zip((k8p, ksp, kvp) + ((kvsp,) if fp8 else ()), pools_before):
        a = p_now.reshape((nb * bs, -1))[~mapped]
        b = p_old.reshape((nb * bs, -1))[~mapped]
        assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                           b.view(torch.uint8) if b.dtype != torch.uint8 else b)


def test_paged_path_decode128k_shape():
    """one full layer of the 128K decode group (B=32, L=131072, bf16 KV) with
    64-row blocks: indexer, selection and attention over paged caches give the
    contiguous results bit for bit (the latent pool is 4.8 GB, past 32-bit
    offsets)"""
    _say("case: paged path B=32 L=131072 bs=64")
    w = wl.WORKLOADS["decode128k"]
    B, T, L, k, bs = w.B, w.T, w.L, w.k, 64
    d = wl.dev_indexer(w, 0, DEV)
    q = wl.dev_attn_q(w, 0, DEV)
    kv, _ = wl.dev_kv(w, 0, DEV)
    vis = torch.from_numpy(w.vis_len()).to(DEV)
    ws_t = _zeros(lcs.topk_workspace_bytes(B, T, L, k))
    ws_a = _zeros(lcs.attn_workspace_bytes(B, T, k))
    sc_r = torch.empty((B, T, L), dtype=torch.float32, device=DEV)
    lcs.idx_score(d["q8"], d["q_scale"], d["w"], d["k8"], d["k_scale"], vis, sc_r)
    idx_r = torch.empty((B, T, k), dtype=torch.int32, device=DEV)
    lcs.topk_select(sc_r, vis, k, idx_r, ws_t)
    out_r = torch.empty((B, T, 64, 512), dtype=torch.bfloat16, device=DEV)
    lcs.sparse_mla_attn(q, kv, None, idx_r, w.sm_scale, out_r, None, ws_a)
    pg, rows, nb = _layout(B, L, bs, seed=123)
    k8p = _pool(d["k8"], rows, nb, bs)
    ksp = _pool(d["k_scale"], rows, nb, bs)
    del d["k8"], d["k_scale"]
    kvp = _pool(kv, rows, nb, bs)
    del kv
    sc = torch.empty_like(sc_r)
    lcs.idx_score_paged(d["q8"], d["q_scale"], d["w"], k8p, ksp, pg, vis, L, sc)
    idx = torch.empty_like(idx_r)
    lcs.topk_select(sc, vis, k, idx, ws_t)
    out = torch.empty_like(out_r)
    lse = torch.empty((B, T, 64), dtype=torch.float32, device=DEV)
    lcs.sparse_mla_attn_paged(q, kvp, None, pg, idx, L, w.sm_scale, out, lse, ws_a)
    torch.cuda.synchronize()
    # sampled sequences against the oracle on the logical caches
    got_idx = idx.cpu().numpy()
    vis_h = w.vis_len()
    idx_s = np.arange(k, dtype=np.int32).reshape(1, 1, k)
    for b in (2, 29):
        inp = wl.host_indexer(w, 0, b0=b, nb=1)
        s32, s64 = oracle.idx_score(inp["q8"], inp["q_scale"], inp["w"], inp["k8"],
                                    inp["k_scale"], vis_h[b:b + 1], want64=True)
        rel = check_scores(sc[b:b + 1].cpu().numpy(), s64, "b=%d" % b)
        ov, gap = check_selection(got_idx[b:b + 1], oracle.topk(s32, vis_h[b:b + 1], k), s64)
        sel = got_idx[b, 0]
        kv_s, _ = wl.host_kv_rows(w, 0, b, sel)
        _, ref_lse, ref64 = oracle.sparse_mla(wl.host_attn_q(w, 0, b0=b, nb=1), kv_s, None, idx_s,
                                              w.sm_scale, want64=True)
        mx, _, lerr = check_attention(out[b:b + 1], ref64, lse[b:b + 1], ref_lse.astype(np.float64))
        _say("  b=%d against the oracle: scores %.3g, overlap %.5f (gap %.3g), max-abs %.3g"
             % (b, rel, ov, gap, mx))
    assert torch.equal(sc.view(torch.int32), sc_r.view(torch.int32))
    assert torch.equal(idx, idx_r)
    assert torch.equal(out.view(torch.int16), out_r.view(torch.int16))
