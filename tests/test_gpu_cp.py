"""GPU parity of the context-parallel halves (through the C ABI): candidates,
merge and localisation bit for bit against the oracle; the LSE combine against
the oracle's double-precision combine; and the whole split path -- the cache
cut into shards, each shard scoring, selecting and attending over its own
rows -- against the unsplit run on the same inputs: selections bit for bit,
outputs within the attention tolerance."""
import sys

import numpy as np
import pytest
import torch

import long_context_sparse_12_amd as lcs
import oracle
from synth import workloads as wl
from tests.parity import DEV, bf16_to_f64, check_attention, to_dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _zeros(nbytes):
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=DEV)


def _cands(rs, G, Q, k_in, ties, empty_frac):
    """candidates of G shards for Q queries: distinct positions per query,
    scores from 5 values (ties, with both zeros) or N(0,1); some empty slots"""
    n = G * k_in
    pos = np.stack([rs.permutation(3 * n)[:n] for _ in range(Q)]).astype(np.int32)
    if ties:
        sc = rs.choice(np.array([-1.5, -0.0, 0.0, 0.25, 2.0], np.float32), size=(Q, n))
    else:
        sc = rs.standard_normal((Q, n)).astype(np.float32)
    empty = rs.random((Q, n)) < empty_frac
    pos[empty] = -1
    sc[empty] = -np.inf
    # [Q][G][k_in] -> [G][Q][k_in]
    return (np.ascontiguousarray(sc.reshape(Q, G, k_in).transpose(1, 0, 2)),
            np.ascontiguousarray(pos.reshape(Q, G, k_in).transpose(1, 0, 2)))


MERGE_CASES = [  # (G, Q, k_in, k, ties, empty_frac)
    (8, 3, 2048, 2048, True, 0.0), (8, 2, 2048, 2048, False, 0.3), (16, 2, 2048, 2048, False, 0.0),
    (3, 5, 100, 64, True, 0.5), (1, 4, 2048, 2048, False, 0.2), (5, 3, 700, 2048, True, 0.9),
    (2, 3, 40, 7, True, 0.0),
]


@pytest.mark.parametrize("case", MERGE_CASES, ids=lambda c: "G%d-Q%d-kin%d-k%d-ties%d-empty%.1f" % c)
def test_topk_merge_bit_exact(case):
    G, Q, k_in, k, ties, empty = case
    _say("case: topk_merge G=%d Q=%d k_in=%d k=%d ties=%d empty=%.1f" % case)
    rs = np.random.default_rng(G * 100 + Q + k_in)
    cs, ci = _cands(rs, G, Q, k_in, ties, empty)
    ci[:, -1] = -1  # one query with no candidate at all
    cs[:, -1] = -np.inf
    ref = oracle.topk_merge(cs, ci, k)
    idx = torch.full((Q, 1, k), 12345, dtype=torch.int32, device=DEV)
    lcs.topk_merge(to_dev(cs).view(G, Q, 1, k_in), to_dev(ci).view(G, Q, 1, k_in), k, idx)
    got = idx.cpu().numpy()[:, 0]
    bad = np.argwhere(got != ref)
    assert bad.size == 0, (bad[:5], got[tuple(bad[0])], ref[tuple(bad[0])])


def test_candidates_and_localize_bit_exact():
    _say("case: topk_candidates / idx_localize")
    rs = np.random.default_rng(77)
    B, T, L, k = 3, 2, 900, 256
    scores = rs.standard_normal((B, T, L)).astype(np.float32)
    idx = np.stack([np.sort(rs.choice(L, k, replace=False)) for _ in range(B * T)]).reshape(
        B, T, k).astype(np.int32)
    idx[0, 1, 200:] = -1
    idx[2, 0, :] = -1
    ref_s, ref_i = oracle.topk_candidates(scores, idx, 5000)
    cs = torch.empty((B, T, k), dtype=torch.float32, device=DEV)
    ci = torch.empty((B, T, k), dtype=torch.int32, device=DEV)
    lcs.topk_candidates(to_dev(scores), to_dev(idx), 5000, cs, ci)
    assert np.array_equal(cs.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))
    assert np.array_equal(ci.cpu().numpy(), ref_i)
    # localize: ascending lists and a shuffled one (list order is kept)
    idx[1, 1] = rs.permutation(idx[1, 1])
    for lo, hi in [(0, 300), (300, 301), (450, 900), (0, 900), (901, 2000), (0, 0)]:
        ref = oracle.idx_localize(idx, lo, hi)
        loc = torch.full((B, T, k), 777, dtype=torch.int32, device=DEV)
        lcs.idx_localize(to_dev(idx), lo, hi, loc)
        assert np.array_equal(loc.cpu().numpy(), ref), (lo, hi)


@pytest.mark.parametrize("G", [1, 5, 8, 12])
def test_lse_combine_matches_oracle(G):
    """G <= 8: one split group per workgroup; G = 12: four groups merged in LDS"""
    _say("case: lse_combine G=%d" % G)
    rs = np.random.default_rng(500 + G)
    Q = 5
    po = torch.from_numpy(rs.standard_normal((G, Q, 1, 64, 512)).astype(np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    pl = (rs.standard_normal((G, Q, 1, 64)) * 6).astype(np.float32)
    pl[0, 1] = -np.inf  # one shard without rows for query 1
    pl[:, 2, 0, :7] = -np.inf  # no shard has rows for some heads of query 2
    if G > 1:
        pl[1, 3] += 90.0  # one shard dominates query 3
    ref_o, ref_l, ref64 = oracle.lse_combine(po, pl, want64=True)
    out = torch.empty((Q, 1, 64, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((Q, 1, 64), dtype=torch.float32, device=DEV)
    lcs.lse_combine(to_dev(po), to_dev(pl), out, lse)
    g = bf16_to_f64(out)
    # half a bf16 step of the result, plus fp32 arithmetic on the weights
    big = np.abs(bf16_to_f64(po)).max(axis=0)
    assert np.all(np.abs(g - ref64) <= 2.0 ** -8 * np.abs(ref64) + 1e-5 * big + 1e-30)
    gl = lse.cpu().numpy().astype(np.float64)
    rl = ref_l.astype(np.float64)
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl))
    fin = np.isfinite(rl)
    assert np.all(np.abs(gl[fin] - rl[fin]) <= 1e-5 * np.abs(rl[fin]) + 1e-5)
    assert torch.all(out[2, 0, :7] == 0)


def _split_path(w, G, check_oracle):
    """one full layer of workload w, unsplit and cut into G shards; returns
    (idx_unsplit, idx_merged, out_unsplit, lse_unsplit, out_split, lse_split)"""
    B, T, L, k, sm = w.B, w.T, w.L, w.k, w.sm_scale
    ind = wl.dev_indexer(w, 0, DEV)
    q = wl.dev_attn_q(w, 0, DEV)
    kv, sc = wl.dev_kv(w, 0, DEV)
    vis = torch.from_numpy(w.vis_len()).to(DEV)
    ws_t = _zeros(lcs.topk_workspace_bytes(B, T, L, k))
    ws_a = _zeros(lcs.attn_workspace_bytes(B, T, k))
    scores = torch.empty((B, T, L), dtype=torch.float32, device=DEV)
    lcs.idx_score(ind["q8"], ind["q_scale"], ind["w"], ind["k8"], ind["k_scale"], vis, scores)
    idx_u = torch.empty((B, T, k), dtype=torch.int32, device=DEV)
    lcs.topk_select(scores, vis, k, idx_u, ws_t)
    out_u = torch.empty((B, T, 64, 512), dtype=torch.bfloat16, device=DEV)
    lse_u = torch.empty((B, T, 64), dtype=torch.float32, device=DEV)
    lcs.sparse_mla_attn(q, kv, sc, idx_u, sm, out_u, lse_u, ws_a)
    if check_oracle:
        # the merge below must equal the definition applied to these scores
        ref = oracle.topk(scores.cpu().numpy(), w.vis_len(), k)
        assert np.array_equal(idx_u.cpu().numpy(), ref)
    del scores

    Ls = (L + G - 1) // G
    bounds = [(g * Ls, min(L, (g + 1) * Ls)) for g in range(G)]
    cand_s = torch.empty((G, B, T, k), dtype=torch.float32, device=DEV)
    cand_i = torch.empty((G, B, T, k), dtype=torch.int32, device=DEV)
    shard = []
    for g, (lo, hi) in enumerate(bounds):
        # each shard holds its own rows (its own allocations: clone, since a
        # slice of a single sequence would be a view at an unaligned offset)
        # and sees the visible part of its range
        k8 = ind["k8"][:, lo:hi].clone()
        ks = ind["k_scale"][:, lo:hi].clone()
        vis_g = (vis - lo).clamp(0, hi - lo).to(torch.int32).contiguous()
        s_g = torch.empty((B, T, hi - lo), dtype=torch.float32, device=DEV)
        lcs.idx_score(ind["q8"], ind["q_scale"], ind["w"], k8, ks, vis_g, s_g)
        i_g = torch.empty((B, T, k), dtype=torch.int32, device=DEV)
        lcs.topk_select(s_g, vis_g, k, i_g, ws_t)
        lcs.topk_candidates(s_g, i_g, lo, cand_s[g], cand_i[g])
        del k8, ks, s_g
        shard.append((kv[:, lo:hi].clone(), None if sc is None else sc[:, lo:hi].clone()))
    idx_m = torch.empty((B, T, k), dtype=torch.int32, device=DEV)
    lcs.topk_merge(cand_s, cand_i, k, idx_m)
    part_o = torch.empty((G, B, T, 64, 512), dtype=torch.bfloat16, device=DEV)
    part_l = torch.empty((G, B, T, 64), dtype=torch.float32, device=DEV)
    for g, (lo, hi) in enumerate(bounds):
        local = torch.empty_like(idx_m)
        lcs.idx_localize(idx_m, lo, hi, local)
        kv_g, sc_g = shard[g]
        lcs.sparse_mla_attn(q, kv_g, sc_g, local, sm, part_o[g], part_l[g], ws_a)
    out_s = torch.empty_like(out_u)
    lse_s = torch.empty_like(lse_u)
    lcs.lse_combine(part_o, part_l, out_s, lse_s)
    torch.cuda.synchronize()
    return idx_u, idx_m, out_u, lse_u, out_s, lse_s, q, kv, sc


SPLIT_CASES = [  # (B, T, L, fp8, causal, G)
    (2, 1, 20037, False, False, 8), (2, 3, 16411, True, True, 3), (3, 1, 6000, True, False, 5),
    (1, 2, 2500, False, True, 8),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "B%d-T%d-L%d-fp8%d-causal%d-G%d" % c)
def test_split_path_equals_unsplit(case):
    B, T, L, fp8, causal, G = case
    _say("case: split path B=%d T=%d L=%d fp8=%d causal=%d G=%d" % case)
    w = wl.Workload("cp-parity", seed=60 + L % 97, B=B, T=T, L=L, n_layers=1, kv_fp8=fp8,
                    plant_permyriad=100, prefix=(L - T) if causal else -1)
    idx_u, idx_m, out_u, lse_u, out_s, lse_s, q, kv, sc = _split_path(w, G, check_oracle=True)
    assert torch.equal(idx_m, idx_u)
    check_attention(out_s, bf16_to_f64(out_u), lse_s, lse_u.cpu().numpy().astype(np.float64))
    # and against the oracle's attention over the merged selection
    _, ref_l, ref64 = oracle.sparse_mla(q.view(torch.int16).cpu().numpy().view(np.uint16),
                                        kv.cpu().numpy() if fp8 else
                                        kv.view(torch.int16).cpu().numpy().view(np.uint16),
                                        None if sc is None else sc.cpu().numpy(),
                                        idx_m.cpu().numpy(), w.sm_scale, want64=True)
    mx, ratio, lerr = check_attention(out_s, ref64, lse_s, ref_l.astype(np.float64))
    _say("  vs oracle: max-abs %.3g (%.3g of rms), lse err %.3g" % (mx, ratio, lerr))


def test_split_path_1m_fp8_eight_shards():
    """the 1M-token FP8 decode layer (B=2, L=2^20) cut into 8 shards of 131072
    rows, one GPU's share each under 8-way context parallelism"""
    _say("case: split path B=2 L=2^20 fp8 G=8")
    w = wl.WORKLOADS["decode1m"]
    idx_u, idx_m, out_u, lse_u, out_s, lse_s, *_ = _split_path(w, 8, check_oracle=False)
    assert torch.equal(idx_m, idx_u)
    mx, ratio, lerr = check_attention(out_s, bf16_to_f64(out_u), lse_s,
                                      lse_u.cpu().numpy().astype(np.float64))
    _say("  vs unsplit: max-abs %.3g (%.3g of rms), lse err %.3g" % (mx, ratio, lerr))
