"""HIP graph capture of the hot path. The allocation-free attention call and
whole composite steps (lcs_indexshare_forward: indexer, top-k and every
layer's attention) are captured once into a graph (torch.cuda.CUDAGraph; the
binding passes the capturing stream) and replayed three times. Between the
replays the outputs are overwritten by eager fills and the device is
synchronised; every replay must reproduce the eager call's outputs bit for
bit. The path launches kernels only (no memset, copy or allocation nodes), and
each replay clears the top-k histograms with its own clear kernel."""
import sys

import numpy as np
import pytest
import torch

import long_context_sparse_12_amd as lcs
from synth import workloads as wl
from tests.parity import DEV, to_dev

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _replay_and_check(g, pairs):
    """pairs: (graph output, eager output); the graph output is overwritten
    before every replay"""
    for rep in range(REPLAYS):
        for got, _ in pairs:
            if got.dtype.is_floating_point:
                got.fill_(7.0)
            else:
                got.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (got, ref) in enumerate(pairs):
            assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8)), \
                "replay %d: output %d differs from the eager call" % (rep, i)


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_graph_replay_noalloc_attention(fp8):
    B, T, L, k = 8, 2, 6000, 1024
    _say("case: graph replay of sparse_mla_attn_noalloc B=%d T=%d L=%d k=%d fp8=%d" %
         (B, T, L, k, fp8))
    w = wl.Workload("graph-attn", seed=41, B=B, T=T, L=L, n_layers=1, kv_fp8=fp8)
    q = wl.dev_attn_q(w, 0, DEV)
    kv, sc = wl.dev_kv(w, 0, DEV)
    rs = np.random.default_rng(5)
    idx_h = np.full((B, T, k), -1, np.int32)
    for b in range(B):
        for t in range(T):
            m = k - (13 if b == 1 else 0)  # one query with padding
            idx_h[b, t, :m] = np.sort(rs.choice(L, m, replace=False))
    idx = to_dev(idx_h)
    out_e = torch.empty((B, T, 64, 512), dtype=torch.bfloat16, device=DEV)
    lse_e = torch.empty((B, T, 64), dtype=torch.float32, device=DEV)
    # eager first: it also looks up the scratch's device address
    lcs.sparse_mla_attn_noalloc(q, kv, sc, idx, w.sm_scale, out_e, lse_e)
    torch.cuda.synchronize()
    out_g = torch.empty_like(out_e)
    lse_g = torch.empty_like(lse_e)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lcs.sparse_mla_attn_noalloc(q, kv, sc, idx, w.sm_scale, out_g, lse_g)
    _replay_and_check(g, [(out_g, out_e), (lse_g, lse_e)])


def _layers(w):
    full = w.full_layers()
    layers = []
    for l in range(w.n_layers):
        d = wl.dev_indexer(w, l, DEV) if l in full else {}
        d["q"] = wl.dev_attn_q(w, l, DEV)
        kv, sc = wl.dev_kv(w, l, DEV)
        d["kv"] = kv
        d["kv_scale"] = sc
        layers.append(d)
    return layers


def _outputs(w, n_full):
    B, T, L, k = w.B, w.T, w.L, w.k
    outs = [(torch.empty((B, T, 64, 512), dtype=torch.bfloat16, device=DEV),
             torch.empty((B, T, 64), dtype=torch.float32, device=DEV)) for _ in range(w.n_layers)]
    idx_out = torch.empty((n_full, B, T, k), dtype=torch.int32, device=DEV)
    scores = torch.empty((B, T, L), dtype=torch.float32, device=DEV)
    return outs, idx_out, scores


def _forward(w, layers, outs, idx_out, scores, vis, ws):
    for d, (o, s) in zip(layers, outs):
        d["out"] = o
        d["lse"] = s
    lcs.indexshare_forward(layers, w.sched, vis, w.k, w.sm_scale, scores, idx_out, ws,
                           kv_dtype=lcs.KV_FP8_E4M3 if w.kv_fp8 else lcs.KV_BF16)


CASES = [  # name, B, T, L, layers, schedule, fp8, prefix (causal chunk, or -1)
    ("group4-bf16", 4, 1, 30000, 4, wl.SCHED_GROUP4, False, -1),  # fused histogram, chunked top-k
    ("glm52-fp8", 2, 1, 50000, 8, wl.SCHED_GLM52, True, -1),      # 4 full layers of 8
    ("verify-bf16", 3, 6, 20000, 4, wl.SCHED_GROUP4, False, 20000 - 6),  # causal 6-query indexer
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_graph_replay_composite(case):
    name, B, T, L, n_layers, sched, fp8, prefix = case
    _say("case: graph replay of indexshare_forward %s B=%d T=%d L=%d layers=%d" %
         (name, B, T, L, n_layers))
    w = wl.Workload("graph-" + name, seed=47, B=B, T=T, L=L, n_layers=n_layers, sched=sched,
                    kv_fp8=fp8, plant_permyriad=100, prefix=prefix)
    layers = _layers(w)
    n_full = lcs.count_full_layers(sched, n_layers)
    assert n_full == len(w.full_layers())
    vis = to_dev(w.vis_len())
    ws = torch.empty(max(lcs.indexshare_workspace_bytes(B, T, L, w.k), 256), dtype=torch.uint8,
                     device=DEV)
    ws.fill_(0xA5)  # the call must not depend on the workspace's contents
    outs_e, idx_e, scores_e = _outputs(w, n_full)
    _forward(w, layers, outs_e, idx_e, scores_e, vis, ws)
    torch.cuda.synchronize()
    outs_g, idx_g, scores_g = _outputs(w, n_full)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _forward(w, layers, outs_g, idx_g, scores_g, vis, ws)
    pairs = [(idx_g, idx_e), (scores_g, scores_e)]
    for (og, sg), (oe, se) in zip(outs_g, outs_e):
        pairs += [(og, oe), (sg, se)]
    _replay_and_check(g, pairs)
