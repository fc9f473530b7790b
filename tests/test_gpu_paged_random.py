"""Seeded random shapes of the paged-KV calls against the oracle on the
logical caches and against the contiguous calls bit for bit: pools of 64- to
1024-row blocks in random order with random bytes in unmapped rows, batch,
queries per sequence (key-streaming and tiled indexer), cache length, k,
ragged visible lengths (0, k - 1, k, k + 1, L and random) and both latent-row
types. Per case: the paged indexer's scores (oracle tolerance, and equal to
the contiguous call's), the selection over them (equal to the oracle's top-k
of those scores), and the paged attention over that selection (oracle
tolerance, and equal to the contiguous call's)."""
import sys

import numpy as np
import pytest
import torch

import long_context_sparse_12_amd as lcs
import oracle
from synth import workloads as wl
from tests.parity import DEV, check_attention, check_scores, to_dev
from tests.test_gpu_paged import _layout, _pool

pytestmark = pytest.mark.gpu

N_CASES = 16


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _zeros(nbytes):
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=DEV)


def _case(i):
    rs = np.random.default_rng(7700 + i)
    B = int(rs.choice([1, 2, 3, 4]))
    T = int(rs.choice([1, 1, 2, 3, 5, 6, 16, 23]))
    bs = int(rs.choice([64, 128, 256, 512, 1024]))
    k = int(rs.choice([1, 7, 100, 1000, 2048]))
    L = int(rs.integers(1, max(2, 60_000 // (B * T)) + 1))
    if B * T * min(k, L) > 20_000:
        k = max(1, 20_000 // (B * T))
    edges = [0, L, min(L, k), min(L, k + 1), max(0, min(L, k - 1))]
    vis = rs.integers(0, L + 1, size=B * T)
    for j in range(min(len(edges), B * T)):
        vis[j] = edges[j]
    rs.shuffle(vis)
    return B, T, L, k, bs, bool(rs.integers(0, 2)), vis.reshape(B, T).astype(np.int32)


@pytest.mark.parametrize("i", range(N_CASES))
def test_paged_random_shape(i):
    B, T, L, k, bs, fp8, vis = _case(i)
    _say("case: paged random %d B=%d T=%d L=%d k=%d bs=%d fp8=%d" % (i, B, T, L, k, bs, fp8))
    w = wl.Workload("paged-random-%d" % i, seed=1300 + i, B=B, T=T, L=L, n_layers=1,
                    kv_fp8=fp8, plant_permyriad=100, k=k)
    d = wl.dev_indexer(w, 0, DEV)
    dvis = to_dev(vis)
    # indexer: paged against contiguous and the oracle
    ref = torch.empty((B, T, L), dtype=torch.float32, device=DEV)
    lcs.idx_score(d["q8"], d["q_scale"], d["w"], d["k8"], d["k_scale"], dvis, ref)
    pg, rows, nb = _layout(B, L, bs, seed=100 + i)
    k8p = _pool(d["k8"], rows, nb, bs)
    ksp = _pool(d["k_scale"], rows, nb, bs)
    got = torch.full((B, T, L), 7.0, dtype=torch.float32, device=DEV)
    lcs.idx_score_paged(d["q8"], d["q_scale"], d["w"], k8p, ksp, pg, dvis, L, got)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))
    inp = wl.host_indexer(w, 0)
    _, ref64 = oracle.idx_score(inp["q8"], inp["q_scale"], inp["w"], inp["k8"], inp["k_scale"],
                                vis, want64=True)
    rel = check_scores(got.cpu().numpy(), ref64)
    # selection over the paged scores: the oracle's top-k of the same scores
    idx = torch.full((B, T, k), -7, dtype=torch.int32, device=DEV)
    lcs.topk_select(got, dvis, k, idx, _zeros(lcs.topk_workspace_bytes(B, T, L, k)))
    got_idx = idx.cpu().numpy()
    assert np.array_equal(got_idx, oracle.topk(got.cpu().numpy(), vis, k))
    # attention over that selection: paged against contiguous and the oracle
    q = wl.dev_attn_q(w, 0, DEV)
    kv, sc = wl.dev_kv(w, 0, DEV)
    ws = _zeros(lcs.attn_workspace_bytes(B, T, k))
    out_r = torch.empty((B, T, 64, 512), dtype=torch.bfloat16, device=DEV)
    lse_r = torch.empty((B, T, 64), dtype=torch.float32, device=DEV)
    lcs.sparse_mla_attn(q, kv, sc, idx, w.sm_scale, out_r, lse_r, ws)
    pg2, rows2, nb2 = _layout(B, L, bs, seed=200 + i)
    kvp = _pool(kv, rows2, nb2, bs)
    scp = None if sc is None else _pool(sc, rows2, nb2, bs)
    out = torch.empty_like(out_r)
    lse = torch.empty_like(lse_r)
    lcs.sparse_mla_attn_paged(q, kvp, scp, pg2, idx, L, w.sm_scale, out, lse, ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_r.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse_r.view(torch.int32))
    kv_h, sc_h = wl.host_kv(w, 0)
    _, ref_lse, out64 = oracle.sparse_mla(wl.host_attn_q(w, 0), kv_h, sc_h, got_idx, w.sm_scale,
                                          want64=True)
    mx, _, lerr = check_attention(out, out64, lse, ref_lse.astype(np.float64))
    _say("  scores rel err %.3g; attention max-abs %.3g, lse err %.3g" % (rel, mx, lerr))
