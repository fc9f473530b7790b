"""The allocation-free attention call (lcs_sparse_mla_attn_noalloc, split
partials in the library's static scratch) against lcs_sparse_mla_attn with a
caller workspace, through the C ABI: two calls in a row on one GPU, the second
smaller (the scratch keeps the first call's partials, which must not leak into
the second), each bit for bit equal to the workspace call and within the
attention tolerance of the oracle on sampled queries."""
import sys

import numpy as np
import pytest
import torch

import long_context_sparse_12_amd as lcs
import oracle
from synth import workloads as wl
from tests.parity import DEV, check_attention, to_dev

pytestmark = pytest.mark.gpu

CASES = [  # (B, T, L, k, fp8): 32 queries x 8 splits, then 3 queries x 16 splits
    (32, 1, 8192, 2048, False),
    (3, 1, 3000, 1500, True),
]


def test_noalloc_matches_workspace_call():
    for B, T, L, k, fp8 in CASES:
        print("case: sparse_mla_attn_noalloc B=%d T=%d L=%d k=%d fp8=%d" % (B, T, L, k, fp8),
              flush=True)
        sys.stdout.flush()
        assert 0 < lcs.attn_workspace_bytes(B, T, k) <= 20 << 20  # the scratch is used
        w = wl.Workload("noalloc", seed=31 + B, B=B, T=T, L=L, n_layers=1, kv_fp8=fp8)
        q_h = wl.host_attn_q(w, 0)
        kv_h, sc_h = wl.host_kv(w, 0)
        rs = np.random.default_rng(B)
        idx_h = np.full((B, T, k), -1, np.int32)
        for b in range(B):
            for t in range(T):
                m = k - (7 if b == 0 else 0)  # one query with padding
                idx_h[b, t, :m] = np.sort(rs.choice(L, m, replace=False))
        q, kv, idx = to_dev(q_h), to_dev(kv_h), to_dev(idx_h)
        sc = None if sc_h is None else to_dev(sc_h)
        ws = torch.zeros(lcs.attn_workspace_bytes(B, T, k), dtype=torch.uint8, device=DEV)
        out_r = torch.empty((B, T, 64, 512), dtype=torch.bfloat16, device=DEV)
        lse_r = torch.empty((B, T, 64), dtype=torch.float32, device=DEV)
        lcs.sparse_mla_attn(q, kv, sc, idx, w.sm_scale, out_r, lse_r, ws)
        out = torch.full_like(out_r, 3.0)
        lse = torch.full_like(lse_r, 3.0)
        lcs.sparse_mla_attn_noalloc(q, kv, sc, idx, w.sm_scale, out, lse)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), out_r.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), lse_r.view(torch.int32))
        for b in (0, B - 1):
            _, ref_lse, ref64 = oracle.sparse_mla(q_h[b:b + 1], kv_h[b:b + 1],
                                                  None if sc_h is None else sc_h[b:b + 1],
                                                  idx_h[b:b + 1], w.sm_scale, want64=True)
            mx, _, lerr = check_attention(out[b:b + 1], ref64, lse[b:b + 1],
                                          ref_lse.astype(np.float64))
            print("  b=%d against the oracle: max-abs %.3g, lse err %.3g" % (b, mx, lerr),
                  flush=True)
