"""Seeded random shapes of the whole path through the composite call
(lcs_indexshare_forward) against the oracle: batch, queries per sequence
(one pass of the key-streaming indexer, two passes, and the tiled prefill
indexer), cache length, k, ragged visible lengths (0, k - 1, k, k + 1, L and
random), bf16 or E4M3 latent rows and the three fixed schedules. For every
full layer the selection must equal the oracle's top-k of the GPU's own scores
exactly, and agree with the oracle's top-k of its own scores up to near-ties;
every layer's attention is checked against the oracle over the GPU's
selection. Sizes keep the fp64 oracle within a few seconds per case."""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import long_context_sparse_12_amd as lcs
import oracle
from synth import workloads as wl
from tests.parity import DEV, check_attention, check_selection, to_dev

pytestmark = pytest.mark.gpu

N_CASES = 24


@dataclasses.dataclass(frozen=True)
class _Ragged(wl.Workload):
    vis: tuple = ()

    def vis_len(self):
        return np.array(self.vis, np.int32).reshape(self.B, self.T)


def _case(i):
    rs = np.random.default_rng(9000 + i)
    B = int(rs.choice([1, 2, 3, 5]))
    T = int(rs.choice([1, 1, 2, 3, 6, 7, 16, 19]))
    k = int(rs.choice([1, 5, 64, 100, 1000, 2048]))
    sched = int(rs.choice([wl.SCHED_GROUP4, wl.SCHED_GLM52, wl.SCHED_ALL_FULL]))
    n_layers = {wl.SCHED_GROUP4: int(rs.integers(1, 6)), wl.SCHED_GLM52: int(rs.integers(3, 8)),
                wl.SCHED_ALL_FULL: int(rs.integers(1, 4))}[sched]
    # indexer work B*T*L <= 120K scores; attention work B*T*layers*min(k, L) <= 40K rows
    L = int(rs.integers(1, max(2, 120_000 // (B * T)) + 1))
    while B * T * n_layers * min(k, L) > 40_000 and n_layers > 1:
        n_layers -= 1
    if B * T * min(k, L) > 40_000:
        k = max(1, 40_000 // (B * T))
    edges = [0, L, min(L, k), min(L, k + 1), max(0, min(L, k - 1))]
    vis = rs.integers(0, L + 1, size=B * T)
    for j in range(min(len(edges), B * T)):
        vis[j] = edges[j]
    rs.shuffle(vis)
    w = _Ragged("random-%d" % i, seed=700 + i, B=B, T=T, L=L, n_layers=n_layers, sched=sched,
                kv_fp8=bool(rs.integers(0, 2)), plant_permyriad=int(rs.choice([0, 100])), k=k,
                vis=tuple(int(v) for v in vis))
    return w


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("i", range(N_CASES))
def test_composite_random_shape(i):
    w = _case(i)
    B, T, L, k = w.B, w.T, w.L, w.k
    full = w.full_layers()
    _say("case: random composite %d B=%d T=%d L=%d k=%d layers=%d sched=%d fp8=%d" %
         (i, B, T, L, k, w.n_layers, w.sched, w.kv_fp8))
    vis = w.vis_len()
    layers_h = []
    for l in range(w.n_layers):
        ly = {}
        if l in full:
            ly.update(wl.host_indexer(w, l))
        ly["q"] = wl.host_attn_q(w, l)
        kv, sc = wl.host_kv(w, l)
        ly["kv"] = kv
        if sc is not None:
            ly["kv_scale"] = sc
        layers_h.append(ly)
    layers_d = []
    for ly in layers_h:
        d = {key: to_dev(v) for key, v in ly.items()}
        d.setdefault("kv_scale", None)
        d["out"] = torch.empty((B, T, 64, 512), dtype=torch.bfloat16, device=DEV)
        d["lse"] = torch.empty((B, T, 64), dtype=torch.float32, device=DEV)
        layers_d.append(d)
    n_full = lcs.count_full_layers(w.sched, w.n_layers)
    assert n_full == len(full)
    idx_out = torch.full((n_full, B, T, k), -7, dtype=torch.int32, device=DEV)
    scores = torch.empty((B, T, L), dtype=torch.float32, device=DEV)
    ws = torch.zeros(max(lcs.indexshare_workspace_bytes(B, T, L, k), 256), dtype=torch.uint8,
                     device=DEV)
    dvis = to_dev(vis)
    lcs.indexshare_forward(layers_d, w.sched, dvis, k, w.sm_scale, scores, idx_out, ws,
                           kv_dtype=lcs.KV_FP8_E4M3 if w.kv_fp8 else lcs.KV_BF16)
    torch.cuda.synchronize()
    got_idx = idx_out.cpu().numpy()
    for f, l in enumerate(full):
        ly, d = layers_h[l], layers_d[l]
        # the GPU's own scores of this layer (the same kernels as in the composite)
        gs = torch.empty((B, T, L), dtype=torch.float32, device=DEV)
        lcs.idx_score(d["q8"], d["q_scale"], d["w"], d["k8"], d["k_scale"], dvis, gs)
        exact = oracle.topk(gs.cpu().numpy(), vis, k)
        assert np.array_equal(got_idx[f], exact), "layer %d: selection differs from the " \
            "oracle's top-k of the GPU scores" % l
        _, s64 = oracle.idx_score(ly["q8"], ly["q_scale"], ly["w"], ly["k8"], ly["k_scale"], vis,
                                  want64=True)
        ref = oracle.topk(s64, vis, k)
        ov, gap = check_selection(got_idx[f], ref, s64)
        _say("  full layer %d: exact on GPU scores; overlap with the oracle's %.5f (gap %.3g)" %
             (l, ov, gap))
    for l, d in enumerate(layers_d):
        f = sum(1 for x in full if x <= l) - 1
        _, ref_lse, ref64 = oracle.sparse_mla(layers_h[l]["q"], layers_h[l]["kv"],
                                              layers_h[l].get("kv_scale"), got_idx[f],
                                              w.sm_scale, want64=True)
        mx, _, lerr = check_attention(d["out"], ref64, d["lse"], ref_lse.astype(np.float64))
        _say("  layer %d attention max-abs %.3g, lse err %.3g" % (l, mx, lerr))
