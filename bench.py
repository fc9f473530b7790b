#!/usr/bin/env python3
"""Decode throughput of the DSA + IndexShare attention path on one MI355X.

A step is one pass of the whole path (indexer -> top-k -> sparse MLA on every
layer, the top-k reused by the shared layers) over one batch of seeded
synthetic inputs already resident in HBM. The default workload is the 128K
decode group: B = 32 sequences, L = 131072 cached positions, one 4-layer
IndexShare group (layer 0 full, layers 1-3 reuse its top-2048), bf16 latent
KV, FP8 indexer keys with 1 % planted +3 sigma keys.

Printed: one JSON line with the step throughput, the dominant kernel's
roofline (HIP events on the launch stream), the IndexShare on/off speed-up
and the CPU oracle timed on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("decode tokens/s/GPU at L=128K & 1M (indexer+top-k+sparse attn); % HBM roofline")
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
FP8_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 MFMA, published
IDX_BYTES_PER_KEY = 132  # 128 E4M3 codes + fp32 scale
IDX_PREFILL_MIN_T = 16  # T at which idx_score switches to the dense FP8-MFMA kernel
IDX_BYTES_PER_QUERY = 32 * 128 + 32 * 4 + 32 * 4  # q8, q_scale, w
ATT_BYTES_PER_QUERY_IO = 64 * 576 * 2 + 64 * 512 * 2 + 64 * 4  # q, out, lse
ROTATIONS = 3  # query sets cycled between steps so no step reuses another's gathers

# HBM traffic of the indexer launch from rocprofv3 --pmc (FETCH_SIZE, WRITE_SIZE),
# scaled by the copy-kernel calibration; valid only for the kernel source it was
# taken on (sha256 of csrc/idx_score.hip, first 16 hex digits).
TRAFFIC = {
    "decode-B32-L131072-group4": {"sha": "6bfa7e3d3b42758a", "bytes": 572135072},
    "decode-B2-L1048576-78layers-fp8kv": {"sha": "6bfa7e3d3b42758a", "bytes": 285334803},
}


def _sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode128k",
                    choices=["tiny", "decode128k", "prefill", "decode1m", "mtp1m", "verify128k"])
    ap.add_argument("--cpu-rows", type=int, default=None, help="sequences in the oracle sample")
    ap.add_argument("--cpu-layers", type=int, default=None, help="layers in the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-off", action="store_true", help="skip the IndexShare-off run")
    ap.add_argument("--only-composite", action="store_true",
                    help="time the composite steps only (for profiling runs)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="also run a plain device copy of this many MiB (3 times), the "
                         "reference kernel for scaling HBM byte counters")
    return ap.parse_args()


class Setup:
    """Device tensors of one workload: per layer the indexer inputs (full
    layers, or every layer for the IndexShare-off run), attention queries and
    latent KV; ROTATIONS query sets per layer."""

    def __init__(self, w, want_off):
        import torch

        from synth import workloads as wl
        self.w = w
        dev = "cuda:0"
        self.dev = dev
        n = w.n_layers
        full = set(w.full_layers())
        need_idx = set(range(n)) if want_off else full
        self.vis = torch.from_numpy(w.vis_len()).to(dev)
        # keys and KV: one copy per (indexer) layer
        self.keys, self.kv = {}, {}
        for l in range(n):
            li = w.indexer_layer(l)
            if l in need_idx and li not in self.keys:
                d = wl.dev_indexer(w, li, dev, keys=True)
                self.keys[li] = (d["k8"], d["k_scale"])
            if li not in self.kv:
                self.kv[li] = wl.dev_kv(w, li, dev)
        # rotated query sets: set r of layer l uses generator layer id l + 1000 r
        self.q = []
        for r in range(ROTATIONS):
            per = []
            for l in range(n):
                d = {}
                if l in need_idx:
                    qi = wl.dev_indexer(w, l + 1000 * r, dev, keys=False)
                    d.update(qi)
                d["q"] = wl.dev_attn_q(w, l + 1000 * r, dev)
                per.append(d)
            self.q.append(per)
        B, T, L, k = w.B, w.T, w.L, w.k
        self.scores = torch.empty((B, T, L), dtype=torch.float32, device=dev)
        n_full_max = n if want_off else len(full)
        self.idx_out = torch.empty((n_full_max, B, T, k), dtype=torch.int32, device=dev)
        self.out = [torch.empty((B, T, 64, 512), dtype=torch.bfloat16, device=dev) for _ in range(n)]
        self.lse = [torch.empty((B, T, 64), dtype=torch.float32, device=dev) for _ in range(n)]
        import long_context_sparse_12_amd as lcs
        self.ws = torch.zeros(lcs.indexshare_workspace_bytes(B, T, L, k), dtype=torch.uint8,
                              device=dev)
        self.ws_topk = torch.zeros(lcs.topk_workspace_bytes(B, T, L, k), dtype=torch.uint8,
                                   device=dev)
        self.ws_attn = torch.zeros(max(lcs.attn_workspace_bytes(B, T, k), 256), dtype=torch.uint8,
                                   device=dev)
        torch.cuda.synchronize()

    def layers(self, r, off):
        w = self.w
        out = []
        for l in range(w.n_layers):
            li = w.indexer_layer(l)
            d = dict(self.q[r][l])
            if (off or l in w.full_layers()) and li in self.keys:
                d["k8"], d["k_scale"] = self.keys[li]
            d["kv"], d["kv_scale"] = self.kv[li]
            d["out"], d["lse"] = self.out[l], self.lse[l]
            out.append(d)
        return out


def run_composite(s, lcs, steps, off):
    w = s.w
    sched = lcs.SCHED_ALL_FULL if off else (lcs.SCHED_GLM52 if w.sched == 1 else lcs.SCHED_GROUP4)
    mtp = 0 if off else w.mtp_steps
    lays = [s.layers(r, off) for r in range(ROTATIONS)]
    kvd = lcs.KV_FP8_E4M3 if w.kv_fp8 else lcs.KV_BF16
    for i in range(steps):
        lcs.indexshare_forward(lays[i % ROTATIONS], sched, s.vis, w.k, w.sm_scale, s.scores,
                               s.idx_out, s.ws, kv_dtype=kvd, mtp_steps=mtp)


def timed(fn, steps, warmup):
    import torch
    fn(warmup)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    fn(steps)
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def kernel_breakdown(s, lcs, steps):
    """The same step issued as the individual C-ABI calls, with HIP events
    recorded on the launch stream around each call; returns mean microseconds
    per launch of each kind."""
    import torch
    w = s.w
    lays = [s.layers(r, False) for r in range(ROTATIONS)]
    full = set(w.full_layers())
    ev = []
    for i in range(steps):
        ly = lays[i % ROTATIONS]
        cur = None
        for l in range(w.n_layers):
            d = ly[l]
            if (w.mtp_steps == 0 and l in full) or (w.mtp_steps and l == 0):
                e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
                e[0].record()
                lcs.idx_score(d["q8"], d["q_scale"], d["w"], d["k8"], d["k_scale"], s.vis, s.scores)
                e[1].record()
                cur = s.idx_out[0]
                lcs.topk_select(s.scores, s.vis, w.k, cur, s.ws_topk)
                e[2].record()
                ev.append(("idx_score", e[0], e[1]))
                ev.append(("topk_select", e[1], e[2]))
            kvl = ly[0] if w.mtp_steps else d
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record()
            lcs.sparse_mla_attn(d["q"], kvl["kv"], kvl["kv_scale"], cur, w.sm_scale, d["out"],
                                d["lse"], s.ws_attn)
            e[1].record()
            ev.append(("sparse_mla_attn", e[0], e[1]))
    torch.cuda.synchronize()
    acc = {}
    for name, a, b in ev:
        acc.setdefault(name, []).append(a.elapsed_time(b) * 1000.0)
    return {k: sum(v) / len(v) for k, v in acc.items()}, {k: len(v) for k, v in acc.items()}


def time_cache_append(w, lcs, steps):
    """One cache append of a layer that keeps both caches: the B*T new tokens'
    indexer keys (quantised) and latent rows (copied, or quantised for an FP8
    cache) written at each sequence's next positions. Dedicated caches of
    max(T, 4096) rows per sequence take the writes, so the step's inputs stay
    as generated; the writes are the same scattered rows as in a full cache.
    Returns (mean microseconds per launch, algorithmic bytes per launch)."""
    import torch
    dev = "cuda:0"
    B, T = w.B, w.T
    Lc = max(T, 4096)
    g = torch.Generator(device=dev).manual_seed(7)
    k_new = torch.randn((B, T, 128), generator=g, device=dev).to(torch.bfloat16)
    kv_new = torch.randn((B, T, 576), generator=g, device=dev).to(torch.bfloat16)
    pos = (torch.arange(T, dtype=torch.int32, device=dev) + (Lc - T)).repeat(B, 1).contiguous()
    k8 = torch.zeros((B, Lc, 128), dtype=torch.uint8, device=dev)
    ks = torch.zeros((B, Lc), dtype=torch.float32, device=dev)
    if w.kv_fp8:
        kv = torch.zeros((B, Lc, 576), dtype=torch.uint8, device=dev)
        kvs = torch.zeros((B, Lc), dtype=torch.float32, device=dev)
    else:
        kv = torch.zeros((B, Lc, 576), dtype=torch.bfloat16, device=dev)
        kvs = None

    def run(n):
        for _ in range(n):
            lcs.cache_append(pos, k_new=k_new, k8=k8, k_scale=ks, kv_new=kv_new, kv=kv,
                             kv_scale=kvs)
    # A launch this small takes less GPU time than one call through Python
    # takes on the host, so the launches are captured once into a HIP graph
    # (the kernel records no memset) and the graph is replayed: the time is
    # then the GPU's own, as in a decode loop that replays its step.
    us = _graph_us(run, steps)
    tok = B * T
    nbytes = tok * (4 + 128 * 2 + 128 + 4 + 576 * 2 + (576 + 4 if w.kv_fp8 else 576 * 2))
    return us, nbytes


def _graph_us(run, n):
    """mean microseconds per launch of n launches captured into one HIP graph
    and replayed (launches too short for Python to keep the GPU busy)"""
    import torch
    run(3)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=cap):
        run(n)
    torch.cuda.current_stream().wait_stream(cap)
    return timed(lambda m: [graph.replay() for _ in range(m)], 5, 2) * 1000.0 / n


def time_context_parallel(w, lcs, G=8, n=50):
    """The single-device halves of G-way context parallelism for one full layer
    of the workload's queries: one shard's candidate gather, the merge of G x k
    candidates, one shard's localisation and the LSE combine of G shard
    outputs. Inputs are random tensors of the real shapes (scores N(0,1),
    distinct positions), resident in HBM. Returns {kernel: (us, bytes)}."""
    import torch
    dev = "cuda:0"
    Q, k = w.B * w.T, w.k
    Ls = w.L // G
    g = torch.Generator(device=dev).manual_seed(11)
    scores = torch.randn((Q, 1, Ls), generator=g, device=dev)
    idx = torch.stack([torch.sort(torch.randperm(Ls, generator=g, device=dev)[:k])[0]
                       for _ in range(Q)]).to(torch.int32).view(Q, 1, k)
    cs = torch.empty((G, Q, 1, k), dtype=torch.float32, device=dev)
    ci = torch.empty((G, Q, 1, k), dtype=torch.int32, device=dev)
    for sh in range(G):
        lcs.topk_candidates(scores, idx, sh * Ls, cs[sh], ci[sh])
    merged = torch.empty((Q, 1, k), dtype=torch.int32, device=dev)
    local = torch.empty_like(merged)
    po = torch.randn((G, Q, 1, 64, 512), generator=g, device=dev).to(torch.bfloat16)
    pl = torch.randn((G, Q, 1, 64), generator=g, device=dev)
    out = torch.empty((Q, 1, 64, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((Q, 1, 64), dtype=torch.float32, device=dev)
    res = {}
    res["topk_candidates"] = (_graph_us(lambda m: [lcs.topk_candidates(
        scores, idx, Ls, cs[1], ci[1]) for _ in range(m)], n), Q * k * (4 + 4 + 4 + 4))
    res["topk_merge"] = (_graph_us(lambda m: [lcs.topk_merge(cs, ci, k, merged)
                                              for _ in range(m)], n), Q * (G * k * 8 + k * 4))
    res["idx_localize"] = (_graph_us(lambda m: [lcs.idx_localize(merged, Ls, 2 * Ls, local)
                                                for _ in range(m)], n), Q * k * 8)
    res["lse_combine"] = (_graph_us(lambda m: [lcs.lse_combine(po, pl, out, lse)
                                               for _ in range(m)], n),
                          Q * ((G + 1) * (64 * 512 * 2 + 64 * 4)))
    return res


def copy_peak_gbs(mb=1024, n=10):
    """Measured device-to-device copy bandwidth, bytes read + written per second
    (a torch copy of `mb` MiB, n times between HIP events after two warm-up
    copies): the practical HBM ceiling the kernels are also compared with."""
    import torch
    src = torch.ones(mb << 20, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / n
    del src, dst
    torch.cuda.empty_cache()
    return 2.0 * (mb << 20) / sec / 1e9


def time_paged(s, lcs, bs=64, n=20):
    """One full layer of the workload with its keys and latent rows laid out in
    pools of bs-row blocks, the blocks in a random order, against the same
    layer contiguous: mean microseconds per launch of the indexer and of the
    attention (HIP events on the launch stream around n launches each)."""
    import numpy as np
    import torch
    w = s.w
    dev = "cuda:0"
    B, T, L, k = w.B, w.T, w.L, w.k
    nb_seq = (L + bs - 1) // bs
    n_blocks = B * nb_seq
    rs = np.random.default_rng(17)
    table = rs.permutation(n_blocks).reshape(B, nb_seq).astype(np.int32)
    pos = np.arange(L)
    rows = torch.from_numpy((table[:, pos // bs].astype(np.int64) * bs + pos % bs).reshape(-1)).to(dev)
    paged = lcs.Paged(torch.from_numpy(table).to(dev), bs, n_blocks)

    def pool(x):
        p = torch.empty((n_blocks * bs,) + tuple(x.shape[2:]), dtype=x.dtype, device=dev)
        p[rows] = x.reshape((-1,) + tuple(x.shape[2:]))
        return p
    d = s.layers(0, False)[0]
    k8p, ksp = pool(d["k8"]), pool(d["k_scale"])
    kvp = pool(d["kv"])
    kvsp = pool(d["kv_scale"]) if d["kv_scale"] is not None else None
    idx = torch.empty((B, T, k), dtype=torch.int32, device=dev)
    lcs.idx_score(d["q8"], d["q_scale"], d["w"], d["k8"], d["k_scale"], s.vis, s.scores)
    lcs.topk_select(s.scores, s.vis, k, idx, s.ws_topk)
    out = torch.empty((B, T, 64, 512), dtype=torch.bfloat16, device=dev)
    calls = {
        "idx_score": lambda: lcs.idx_score(d["q8"], d["q_scale"], d["w"], d["k8"], d["k_scale"],
                                           s.vis, s.scores),
        "idx_score_paged": lambda: lcs.idx_score_paged(d["q8"], d["q_scale"], d["w"], k8p, ksp,
                                                       paged, s.vis, L, s.scores),
        "sparse_mla_attn": lambda: lcs.sparse_mla_attn(d["q"], d["kv"], d["kv_scale"], idx,
                                                       w.sm_scale, out, None, s.ws_attn),
        "sparse_mla_attn_paged": lambda: lcs.sparse_mla_attn_paged(
            d["q"], kvp, kvsp, paged, idx, L, w.sm_scale, out, None, s.ws_attn),
    }
    res = {}
    for name, fn in calls.items():
        res[name] = round(timed(lambda m: [fn() for _ in range(m)], n, 3) * 1000.0, 2)
    del k8p, ksp, kvp, kvsp
    return res


def step_bytes(w, off):
    """algorithmic HBM bytes of one step (keys+scales+queries, gathered rows and
    attention I/O); intermediates (scores, selections) are not counted"""
    n_full = w.n_layers if off else len(w.full_layers())
    q = w.B * w.T
    row = 580 if w.kv_fp8 else 1152
    idx = n_full * (w.B * w.L * IDX_BYTES_PER_KEY + q * IDX_BYTES_PER_QUERY)
    att = w.n_layers * q * (w.k * row + ATT_BYTES_PER_QUERY_IO)
    return idx + att


def cpu_baseline(w, rows, max_layers):
    """The oracle (single-threaded C, double precision) on a bounded sample of
    the same workload: `rows` sequences (one query each), the first
    `max_layers` layers of the pass (indexer over the full cache + top-k on
    full layers, sparse MLA on every layer). The time of a whole pass is the
    mean indexer+top-k time x full layers + mean attention time x layers.
    Input generation is not timed."""
    import numpy as np

    import oracle
    from synth import workloads as wl
    rs = np.random.default_rng(0)
    picks = sorted(rs.choice(w.B, size=min(rows, w.B), replace=False).tolist())
    full = w.full_layers()
    n_lay = min(max_layers, w.n_layers)
    t_idx, t_att = [], []
    for b in picks:
        t = 0  # one query row of the sequence
        vis = w.vis_len()[b:b + 1, t:t + 1]
        cur = None
        for l in range(n_lay):
            li = w.indexer_layer(l)
            if l in full:
                inp = wl.host_indexer(w, li, b0=b, nb=1)
                t0 = time.perf_counter()
                sc = oracle.idx_score(inp["q8"][:, t:t + 1], inp["q_scale"][:, t:t + 1],
                                      inp["w"][:, t:t + 1], inp["k8"], inp["k_scale"], vis)
                cur = oracle.topk(sc, vis, w.k)
                t_idx.append(time.perf_counter() - t0)
            q = wl.host_attn_q(w, l, b0=b, nb=1)[:, t:t + 1]
            sel = cur[0, 0]
            valid = sel[sel >= 0]
            kv, ksc = wl.host_kv_rows(w, li, b, valid)
            idx = np.full((1, 1, w.k), -1, np.int32)
            idx[0, 0, :len(valid)] = np.arange(len(valid), dtype=np.int32)
            t0 = time.perf_counter()
            oracle.sparse_mla(q, kv, ksc, idx, w.sm_scale, L=len(valid))
            t_att.append(time.perf_counter() - t0)
    per_pass = (sum(t_idx) / len(t_idx)) * len(full) + (sum(t_att) / len(t_att)) * w.n_layers
    measured = sum(t_idx) + sum(t_att)
    sample = "%d of %d sequences x 1 query, layers 0-%d of %d (%.1f s measured)" % (
        len(picks), w.B, n_lay - 1, w.n_layers, measured)
    if n_lay < w.n_layers:
        sample += "; whole pass extrapolated from the per-layer means"
    return per_pass, sample


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU; multi-GPU runs are not part of it "
              "(got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    import long_context_sparse_12_amd as lcs
    from synth import workloads as wl

    w = wl.WORKLOADS[args.workload]
    if args.copy_calibration_mb:
        n = args.copy_calibration_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    has_off = (w.n_layers > 1) and not args.no_off
    t_setup = time.time()
    s = Setup(w, want_off=has_off)
    print("setup %s: %.1f s" % (w.name, time.time() - t_setup), file=sys.stderr, flush=True)

    ms = timed(lambda n: run_composite(s, lcs, n, False), args.steps, args.warmup)
    tokens = w.B * w.T * (w.mtp_steps if w.mtp_steps else 1)
    value = tokens / (ms / 1000.0)
    print("timed %d steps: %.3f ms/step" % (args.steps, ms), file=sys.stderr, flush=True)
    sb = step_bytes(w, False)
    res = {
        "metric": METRIC, "value": round(value, 1),
        "unit": ("draft tokens/s" if w.mtp_steps else
                 "prefill tokens/s" if w.T >= IDX_PREFILL_MIN_T else
                 "verified tokens/s" if w.prefix >= 0 else "tokens/s"),
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8+bf16 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "L": w.L, "layers": w.n_layers,
                   "topk": w.k, "kv": "fp8-e4m3" if w.kv_fp8 else "bf16",
                   "schedule": "mtp-reuse" if w.mtp_steps else
                   ("glm52" if w.sched == 1 else "group4")},
        "step_hbm": {"algorithmic_bytes": sb, "achieved_GBs": round(sb / (ms / 1e3) / 1e9, 1),
                     "frac": round(sb / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)},
    }
    if not args.only_composite:
        ker, counts = kernel_breakdown(s, lcs, max(args.steps // 2, 3))
        idx_us = ker["idx_score"]
        sha = _sha(os.path.join(ROOT, "long_context_sparse_12_amd", "csrc", "idx_score.hip"))
        tr = TRAFFIC.get(w.name)
        traffic = tr["bytes"] if tr and tr["sha"] == sha else None
        if w.T >= IDX_PREFILL_MIN_T:
            # dense FP8 contraction: 32 heads x 128 dims = 4096 MACs = 8192 FLOP per
            # visible (t, s) pair
            flops = 8192.0 * float(w.vis_len().astype("int64").sum())
            achieved = flops / (idx_us * 1e-6) / 1e12
            res["roofline"] = {"kernel": "idx_score (prefill indexer)", "bound": "mfma",
                               "achieved": round(achieved, 1), "peak": FP8_PEAK_TFLOPS,
                               "unit": "TFLOP/s", "frac": round(achieved / FP8_PEAK_TFLOPS, 4),
                               "traffic": traffic, "flop_per_launch": flops,
                               "avg_launch_us": round(idx_us, 2)}
        else:
            launch_bytes = w.B * w.L * IDX_BYTES_PER_KEY + w.B * w.T * IDX_BYTES_PER_QUERY
            achieved = launch_bytes / (idx_us * 1e-6) / 1e9
            cp = copy_peak_gbs()
            res["roofline"] = {"kernel": "idx_score (decode indexer)", "bound": "hbm",
                               "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                               "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                               "traffic": traffic, "bytes_per_launch": launch_bytes,
                               "avg_launch_us": round(idx_us, 2),
                               "copy_peak_measured": round(cp, 1),
                               "frac_of_copy_peak": round(achieved / cp, 4)}
        res["kernels_us"] = {k: round(v, 2) for k, v in ker.items()}
        res["launches_per_step"] = {k: v // max(args.steps // 2, 3) for k, v in counts.items()}
        ap_us, ap_bytes = time_cache_append(w, lcs, 50)
        res["cache_append"] = {"tokens": w.B * w.T, "us_per_launch": round(ap_us, 2),
                               "bytes_per_launch": ap_bytes,
                               "achieved_GBs": round(ap_bytes / (ap_us * 1e-6) / 1e9, 1),
                               "note": "keys + latent rows of one layer; not part of the step"}
        if not w.mtp_steps:
            res["paged"] = {"block_size": 64, "note": "one full layer, blocks in random order; "
                            "not part of the step", "us_per_launch": time_paged(s, lcs)}
        if w.T < IDX_PREFILL_MIN_T:
            cp = time_context_parallel(w, lcs)
            res["context_parallel"] = {
                "shards": 8, "note": "single-device halves of 8-way context parallelism for one "
                "full layer; not part of the step",
                "us_per_launch": {kk: round(v[0], 2) for kk, v in cp.items()},
                "bytes_per_launch": {kk: v[1] for kk, v in cp.items()}}
    if has_off:
        ms_off = timed(lambda n: run_composite(s, lcs, n, True), args.steps, args.warmup)
        res["indexshare"] = {"on_ms": round(ms, 4), "off_ms": round(ms_off, 4),
                             "speedup": round(ms_off / ms, 3),
                             "off_value": round(tokens / (ms_off / 1e3), 1)}
    del s
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        big = w.L > 200000
        rows = args.cpu_rows or (1 if big else 8)
        lay = args.cpu_layers or (2 if big else w.n_layers)
        per_pass, sample = cpu_baseline(w, rows, lay)
        per_tok = tokens / (w.B * w.T)  # tokens of one query row per pass (MTP: draft steps)
        res["cpu_baseline"] = {"value": round(per_tok / per_pass, 4), "unit": res["unit"],
                               "cores": 1, "kind": "oracle", "sample": sample}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
