#!/usr/bin/env python3
"""Decode throughput of the DSA + IndexShare attention path on one MI355X.

A step is one pass of the whole path (indexer -> top-k -> sparse MLA on every
layer, the top-k reused by the shared layers) over one batch of seeded
synthetic inputs already resident in HBM. The headline workload is the 128K
decode group: B = 32 sequences, L = 131072 cached positions, one 4-layer
IndexShare group (layer 0 full, layers 1-3 reuse its top-2048), bf16 latent
KV, FP8 indexer keys with 1 % planted +3 sigma keys. The same line carries a
record for each other workload of the metric: the 78-layer schedule at 1M
(B = 2, FP8 KV), the MTP draft round at 1M (B = 8, 7 steps) and the chunked
prefill (T = 4096 at L = 131072).

Timing: every step is bracketed alone by HIP events on the launch stream,
and a 1 GiB device read between steps (outside the events) evicts the 256 MB
memory-side cache, so no step is served from another's reads. (A read, not a
write: a write would leave the cache full of dirty lines, and the next step
would pay for writing them back.)

Printed: one JSON line with the step throughput, the dominant kernel's
roofline (the indexer, from back-to-back launches between HIP events), the
whole step's share of the HBM roofline, the IndexShare on/off speed-up and the
CPU oracle timed on a bounded sample of the same workload (one pinned core,
and one pinned process per host core).
"""
import argparse
import hashlib
import json
import os
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("decode tokens/s/GPU at L=128K & 1M (indexer+top-k+sparse attn); % HBM roofline")
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
FP8_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 MFMA, published
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
IDX_BYTES_PER_KEY = 132  # 128 E4M3 codes + fp32 scale
IDX_PREFILL_MIN_T = 16  # T at which idx_score switches to the dense FP8-MFMA kernel
IDX_BYTES_PER_QUERY = 32 * 128 + 32 * 4 + 32 * 4  # q8, q_scale, w
ATT_BYTES_PER_QUERY_IO = 64 * 576 * 2 + 64 * 512 * 2 + 64 * 4  # q, out, lse
ROTATIONS = 3  # query sets cycled between steps
EVICT_BYTES = 1 << 30  # read between timed steps: 4x the memory-side cache
CPU_WORKERS_MAX = 16  # oracle processes of the all-cores leg (the host's share per GPU)

# HBM traffic of the indexer launch from rocprofv3 --pmc (FETCH_SIZE, WRITE_SIZE),
# scaled by the copy-kernel calibration; valid only for the kernel source it was
# taken on (sha256 of csrc/idx_score.hip, first 16 hex digits).
TRAFFIC = {
    "decode-B32-L131072-group4": {"sha": "c879e1043bd19435", "bytes": 572730834},
    "decode-B2-L1048576-78layers-fp8kv": {"sha": "c879e1043bd19435", "bytes": 285335671},
    "mtp-B8-L1048576-7steps-fp8kv": {"sha": "c879e1043bd19435", "bytes": 1142176075},
}

WORKLOAD_KEYS = ["tiny", "decode128k", "prefill", "decode1m", "mtp1m", "verify128k"]


def _sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode128k", choices=WORKLOAD_KEYS)
    ap.add_argument("--also", default="decode1m,mtp1m,prefill",
                    help="comma-separated workloads reported as records beside the headline "
                         "('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-off", action="store_true", help="skip the IndexShare-off runs")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the cache-append, paged and context-parallel timings")
    ap.add_argument("--only-composite", action="store_true",
                    help="time the composite steps of the headline workload only (profiling)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="also run a plain device copy of this many MiB (3 times), the "
                         "reference kernel for scaling HBM byte counters")
    ap.add_argument("--cpu-worker", default=None, help=argparse.SUPPRESS)
    return ap.parse_args()


# ---------------------------------------------------------------- GPU side
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
                    d.update(wl.dev_indexer(w, l + 1000 * r, dev, keys=False))
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
        self.evict_buf = torch.ones(EVICT_BYTES // 4, dtype=torch.float32, device=dev)
        self.evict_sum = torch.empty((), dtype=torch.float32, device=dev)
        torch.sum(self.evict_buf, 0, out=self.evict_sum)
        torch.cuda.synchronize()

    def evict(self, i=0):
        """a 1 GiB device read: pushes every earlier read out of the memory-side
        cache and leaves it holding clean lines"""
        torch = sys.modules["torch"]
        torch.sum(self.evict_buf, 0, out=self.evict_sum)

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


def step_fn(s, lcs, off):
    """one composite call per step i (query set i mod ROTATIONS)"""
    w = s.w
    sched = lcs.SCHED_ALL_FULL if off else (lcs.SCHED_GLM52 if w.sched == 1 else lcs.SCHED_GROUP4)
    mtp = 0 if off else w.mtp_steps
    lays = [s.layers(r, off) for r in range(ROTATIONS)]
    kvd = lcs.KV_FP8_E4M3 if w.kv_fp8 else lcs.KV_BF16

    def run(i):
        lcs.indexshare_forward(lays[i % ROTATIONS], sched, s.vis, w.k, w.sm_scale, s.scores,
                               s.idx_out, s.ws, kv_dtype=kvd, mtp_steps=mtp)
    return run


def timed_steps(s, fn, steps, warmup):
    """warm-up steps, then `steps` steps each between its own pair of HIP events
    on the launch stream, with the cache-evicting read before each (outside the
    events); both ends synchronised. Returns the per-step milliseconds."""
    import torch
    for i in range(warmup):
        s.evict(i)
        fn(i)
    torch.cuda.synchronize()
    ev = []
    for i in range(steps):
        s.evict(i)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn(i)
        e1.record()
        ev.append((e0, e1))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def _summary(ms):
    return {"mean": round(statistics.fmean(ms), 4), "median": round(statistics.median(ms), 4),
            "min": round(min(ms), 4), "max": round(max(ms), 4)}


def launches_us(s, fn, n):
    """mean microseconds per launch of n back-to-back launches fn(0..n-1) between
    one pair of HIP events on the launch stream (after an evicting read)"""
    import torch
    fn(0)
    s.evict()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1000.0 / n


def kernel_times(s, lcs, n):
    """Mean microseconds per launch of each C-ABI call of the step, each kind
    issued back to back (n launches, query sets and key sets rotated) between
    one pair of HIP events."""
    w = s.w
    full = w.full_layers()
    lays = [s.layers(r, False) for r in range(ROTATIONS)]
    # key sets to rotate over: every layer that has keys resident
    key_layers = sorted(s.keys)
    res = {}

    def idx_call(i):
        d = lays[i % ROTATIONS][full[0]]
        k8, ks = s.keys[key_layers[i % len(key_layers)]]
        lcs.idx_score(d["q8"], d["q_scale"], d["w"], k8, ks, s.vis, s.scores)
    res["idx_score"] = launches_us(s, idx_call, n)
    cur = s.idx_out[0]
    lcs.topk_select(s.scores, s.vis, w.k, cur, s.ws_topk)
    res["topk_select"] = launches_us(
        s, lambda i: lcs.topk_select(s.scores, s.vis, w.k, cur, s.ws_topk), n)

    def att_call(i):
        ly = lays[i % ROTATIONS]
        l = i % w.n_layers
        kvl = ly[0] if w.mtp_steps else ly[l]
        lcs.sparse_mla_attn(ly[l]["q"], kvl["kv"], kvl["kv_scale"], cur, w.sm_scale,
                            ly[l]["out"], ly[l]["lse"], s.ws_attn)
    res["sparse_mla_attn"] = launches_us(s, att_call, max(n, 2 * w.n_layers))
    return res


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
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 5 * 1000.0 / n


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
    cs1, ci1 = torch.empty_like(cs[1]), torch.empty_like(ci[1])
    res = {}
    res["topk_candidates"] = (_graph_us(lambda m: [lcs.topk_candidates(
        scores, idx, Ls, cs1, ci1) for _ in range(m)], n), Q * k * (4 + 4 + 4 + 4))
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
    attention (n back-to-back launches between HIP events)."""
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
        "idx_score": lambda i: lcs.idx_score(d["q8"], d["q_scale"], d["w"], d["k8"], d["k_scale"],
                                             s.vis, s.scores),
        "idx_score_paged": lambda i: lcs.idx_score_paged(d["q8"], d["q_scale"], d["w"], k8p, ksp,
                                                         paged, s.vis, L, s.scores),
        "sparse_mla_attn": lambda i: lcs.sparse_mla_attn(d["q"], d["kv"], d["kv_scale"], idx,
                                                         w.sm_scale, out, None, s.ws_attn),
        "sparse_mla_attn_paged": lambda i: lcs.sparse_mla_attn_paged(
            d["q"], kvp, kvsp, paged, idx, L, w.sm_scale, out, None, s.ws_attn),
    }
    res = {name: round(launches_us(s, fn, n), 2) for name, fn in calls.items()}
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


def _roof(amount, us, peak, unit, what):
    achieved = amount / (us * 1e-6) / (1e9 if unit == "GB/s" else 1e12)
    key = "bytes_per_launch" if unit == "GB/s" else "flop_per_launch"
    return {"bound": "hbm" if unit == "GB/s" else "mfma", "achieved": round(achieved, 1),
            "peak": peak, "unit": unit, "frac": round(achieved / peak, 4), key: amount,
            "avg_launch_us": round(us, 2), "counts": what}


def kernel_rooflines(w, ker):
    """The selection and the attention calls against their own bounds, from the
    mean launch times in kernels_us (back-to-back launches between HIP events).
    The selection reads every visible score once and writes k indices per
    query; the attention (with its split combine, which the call launches)
    reads the selected rows, its queries and selections and writes out and lse
    (HBM), or, at many queries per sequence, performs 64 heads x (576 + 512)
    MACs per selected row (bf16 MFMA)."""
    q = w.B * w.T
    vis = w.vis_len().astype("int64")
    scores = int(vis.sum()) * 4 + q * w.k * 4
    res = {"topk_select": _roof(scores, ker["topk_select"], HBM_PEAK_GBS, "GB/s",
                                "visible scores read once + indices written")}
    rows = int(vis.clip(max=w.k).sum())
    if w.T >= IDX_PREFILL_MIN_T:
        flops = 2.0 * rows * 64 * (576 + 512)
        res["sparse_mla_attn"] = _roof(flops, ker["sparse_mla_attn"], BF16_PEAK_TFLOPS, "TFLOP/s",
                                       "QK (576 dims) and PV (512 dims) per head and row")
    else:
        row = 580 if w.kv_fp8 else 1152
        nbytes = rows * (row + 4) + q * ATT_BYTES_PER_QUERY_IO
        res["sparse_mla_attn"] = _roof(nbytes, ker["sparse_mla_attn"], HBM_PEAK_GBS, "GB/s",
                                       "selected rows + indices, q, out, lse")
    return res


def _unit(w):
    return ("draft tokens/s" if w.mtp_steps else
            "prefill tokens/s" if w.T >= IDX_PREFILL_MIN_T else
            "verified tokens/s" if w.prefix >= 0 else "tokens/s")


def _tokens(w):
    return w.B * w.T * (w.mtp_steps if w.mtp_steps else 1)


def measure(w, args, lcs, headline):
    """all GPU figures of one workload as a dict (the headline's carry extras)"""
    import torch
    has_off = (w.n_layers > 1) and not args.no_off
    t_setup = time.time()
    s = Setup(w, want_off=has_off)
    print("setup %s: %.1f s" % (w.name, time.time() - t_setup), file=sys.stderr, flush=True)
    ms = timed_steps(s, step_fn(s, lcs, False), args.steps, args.warmup)
    mean = statistics.fmean(ms)
    tokens = _tokens(w)
    sb = step_bytes(w, False)
    print("%s: %d steps, %.4f ms/step (median %.4f)" % (w.name, args.steps, mean,
                                                          statistics.median(ms)),
          file=sys.stderr, flush=True)
    rec = {
        "value": round(tokens / (mean / 1000.0), 1), "unit": _unit(w),
        "ms_per_step": round(mean, 4), "step_ms": _summary(ms),
        "config": {"workload": w.name, "B": w.B, "T": w.T, "L": w.L, "layers": w.n_layers,
                   "topk": w.k, "kv": "fp8-e4m3" if w.kv_fp8 else "bf16",
                   "schedule": "mtp-reuse" if w.mtp_steps else
                   ("glm52" if w.sched == 1 else "group4")},
        "step_hbm": {"algorithmic_bytes": sb,
                     "achieved_GBs": round(sb / (mean / 1e3) / 1e9, 1),
                     "frac": round(sb / (mean / 1e3) / 1e9 / HBM_PEAK_GBS, 4)},
    }
    if not args.only_composite:
        n = max(args.steps, 10)
        ker = kernel_times(s, lcs, n)
        idx_us = ker["idx_score"]
        sha = _sha(os.path.join(ROOT, "long_context_sparse_12_amd", "csrc", "idx_score.hip"))
        tr = TRAFFIC.get(w.name)
        traffic = tr["bytes"] if tr and tr["sha"] == sha else None
        if w.T >= IDX_PREFILL_MIN_T:
            # dense FP8 contraction: 32 heads x 128 dims = 4096 MACs = 8192 FLOP per
            # visible (t, s) pair
            flops = 8192.0 * float(w.vis_len().astype("int64").sum())
            achieved = flops / (idx_us * 1e-6) / 1e12
            rec["roofline"] = {"kernel": "idx_score (prefill indexer)", "bound": "mfma",
                               "achieved": round(achieved, 1), "peak": FP8_PEAK_TFLOPS,
                               "unit": "TFLOP/s", "frac": round(achieved / FP8_PEAK_TFLOPS, 4),
                               "traffic": traffic, "flop_per_launch": flops,
                               "avg_launch_us": round(idx_us, 2)}
        else:
            launch_bytes = w.B * w.L * IDX_BYTES_PER_KEY + w.B * w.T * IDX_BYTES_PER_QUERY
            achieved = launch_bytes / (idx_us * 1e-6) / 1e9
            rec["roofline"] = {"kernel": "idx_score (decode indexer)", "bound": "hbm",
                               "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                               "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                               "traffic": traffic, "bytes_per_launch": launch_bytes,
                               "avg_launch_us": round(idx_us, 2)}
            if headline:
                cp = copy_peak_gbs()
                rec["roofline"]["copy_peak_measured"] = round(cp, 1)
                rec["roofline"]["frac_of_copy_peak"] = round(achieved / cp, 4)
        rec["kernels_us"] = {k: round(v, 2) for k, v in ker.items()}
        rec["kernel_rooflines"] = kernel_rooflines(w, ker)
        if headline and not args.no_extras:
            ap_us, ap_bytes = time_cache_append(w, lcs, 50)
            rec["cache_append"] = {"tokens": w.B * w.T, "us_per_launch": round(ap_us, 2),
                                   "bytes_per_launch": ap_bytes,
                                   "achieved_GBs": round(ap_bytes / (ap_us * 1e-6) / 1e9, 1),
                                   "note": "keys + latent rows of one layer; not part of the step"}
            if not w.mtp_steps:
                rec["paged"] = {"block_size": 64, "note": "one full layer, blocks in random "
                                "order; not part of the step", "us_per_launch": time_paged(s, lcs)}
            if w.T < IDX_PREFILL_MIN_T:
                cp = time_context_parallel(w, lcs)
                rec["context_parallel"] = {
                    "shards": 8, "note": "single-device halves of 8-way context parallelism "
                    "for one full layer; not part of the step",
                    "us_per_launch": {kk: round(v[0], 2) for kk, v in cp.items()},
                    "bytes_per_launch": {kk: v[1] for kk, v in cp.items()}}
    if has_off:
        ms_off = timed_steps(s, step_fn(s, lcs, True), max(args.steps // 2, 3),
                             max(args.warmup // 2, 1))
        off = statistics.fmean(ms_off)
        rec["indexshare"] = {"on_ms": round(mean, 4), "off_ms": round(off, 4),
                             "speedup": round(off / mean, 3),
                             "off_value": round(tokens / (off / 1e3), 1),
                             "off_step_hbm_frac": round(step_bytes(w, True) / (off / 1e3) / 1e9
                                                        / HBM_PEAK_GBS, 4)}
    del s
    torch.cuda.empty_cache()
    return rec


# ---------------------------------------------------------------- CPU oracle
def cpu_worker(spec):
    """Runs in a fresh interpreter that never touches the GPU: the oracle on the
    given (sequence, query) rows of a workload, each through the given layers
    (indexer + top-k over the whole cache on full layers, sparse MLA on every
    layer). Pins itself to one core when asked. Prints the timings as JSON."""
    import numpy as np

    import oracle
    from synth import workloads as wl
    if spec.get("core") is not None:
        os.sched_setaffinity(0, {spec["core"]})
    w = wl.WORKLOADS[spec["workload"]]
    full = w.full_layers()
    t_idx, t_att = [], []
    for b, t, layers in spec["items"]:
        vis = w.vis_len()[b:b + 1, t:t + 1]
        cur = None
        for l in layers:
            li = w.indexer_layer(l)
            if l in full or cur is None:
                inp = wl.host_indexer(w, li, b0=b, nb=1)  # generation is not timed
                t0 = time.perf_counter()
                sc = oracle.idx_score(inp["q8"][:, t:t + 1], inp["q_scale"][:, t:t + 1],
                                      inp["w"][:, t:t + 1], inp["k8"], inp["k_scale"], vis)
                cur = oracle.topk(sc, vis, w.k)
                t_idx.append(time.perf_counter() - t0)
                del inp, sc
            q = wl.host_attn_q(w, l, b0=b, nb=1)[:, t:t + 1]
            sel = cur[0, 0]
            valid = sel[sel >= 0]
            kv, ksc = wl.host_kv_rows(w, li, b, valid)
            idx = np.full((1, 1, w.k), -1, np.int32)
            idx[0, 0, :len(valid)] = np.arange(len(valid), dtype=np.int32)
            t0 = time.perf_counter()
            oracle.sparse_mla(q, kv, ksc, idx, w.sm_scale, L=len(valid))
            t_att.append(time.perf_counter() - t0)
    print(json.dumps({"t_idx": t_idx, "t_att": t_att}), flush=True)


def _spawn_workers(specs):
    env = dict(os.environ)
    for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        env[v] = "1"
    procs = [subprocess.Popen([sys.executable, os.path.abspath(__file__), "--cpu-worker",
                               json.dumps(sp)], stdout=subprocess.PIPE, env=env, text=True)
             for sp in specs]
    t0 = time.perf_counter()
    outs = []
    for p in procs:
        o, _ = p.communicate(timeout=600)
        if p.returncode != 0:
            raise RuntimeError("oracle worker failed (%d)" % p.returncode)
        outs.append(json.loads(o.strip().splitlines()[-1]))
    return outs, time.perf_counter() - t0


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, key):
    """The oracle (plain single-threaded C, double precision) on a bounded
    sample of the workload, timed on this host's cores in the same run: one
    process pinned to one core, then one pinned process per core (at most
    CPU_WORKERS_MAX) on disjoint rows and layers, all at once. The time of a
    whole pass of one query row is the mean indexer+top-k time x full layers +
    the mean attention time x layers; the throughput is rows per second of
    such passes (summed over the concurrent processes), in the workload's
    tokens."""
    cores = sorted(os.sched_getaffinity(0))
    n_workers = min(CPU_WORKERS_MAX, len(cores))
    full = w.full_layers()
    n_full = len(full)
    n_att = w.n_layers
    per_row_tokens = w.mtp_steps if w.mtp_steps else 1
    big = w.L > 200000

    def layers_for(i):
        # one full layer and the layer after it (or the draft steps), rotated per process
        if w.mtp_steps:
            return list(range(w.n_layers))
        if big:
            f = full[i % n_full]
            return [f, f + 1] if f + 1 < w.n_layers else [f]
        return list(range(w.n_layers))

    def rows_for(i):
        b = i % w.B
        t = (i * 977) % w.T
        return b, t

    def rate(out):
        ti = sum(out["t_idx"]) / len(out["t_idx"])
        ta = sum(out["t_att"]) / len(out["t_att"])
        per_pass = ti * n_full + ta * n_att
        return per_row_tokens / per_pass, sum(out["t_idx"]) + sum(out["t_att"])

    n_single = 1 if (big or w.T >= IDX_PREFILL_MIN_T) else 3
    single = [{"workload": key, "core": cores[0],
               "items": [list(rows_for(7 * i)) + [layers_for(i)] for i in range(n_single)]}]
    (o1,), _ = _spawn_workers(single)
    v1, cpu1 = rate(o1)
    specs = [{"workload": key, "core": cores[i],
              "items": [list(rows_for(i)) + [layers_for(i)]]} for i in range(n_workers)]
    outs, wall = _spawn_workers(specs)
    vn = sum(rate(o)[0] for o in outs)
    cpun = sum(rate(o)[1] for o in outs)
    lay = ("layers %s" % layers_for(0)) if big else "every layer"
    return {"value": round(vn, 4), "unit": _unit(w), "cores": n_workers, "kind": "oracle",
            "sample": "%d processes pinned one per core, one query row each (%s), all at once; "
                      "%.1f s of CPU work timed, %.1f s wall; a whole pass estimated from the "
                      "per-layer means" % (n_workers, lay, cpun, wall),
            "single_core": {"value": round(v1, 4), "cores": 1, "pinned_core": cores[0],
                            "sample": "%d query row(s), %.1f s of CPU work timed" % (n_single, cpu1)},
            "nproc": len(cores), "cpu_model": _cpu_model()}


# ---------------------------------------------------------------- main
def main():
    args = parse()
    if args.cpu_worker is not None:
        cpu_worker(json.loads(args.cpu_worker))
        return
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU; multi-GPU runs are not part of it "
              "(got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    import long_context_sparse_12_amd as lcs
    from synth import workloads as wl

    if args.copy_calibration_mb:
        n = args.copy_calibration_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    w = wl.WORKLOADS[args.workload]
    head = measure(w, args, lcs, headline=True)
    res = {"metric": METRIC, "value": head.pop("value"), "unit": head.pop("unit"), "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": head.pop("ms_per_step"),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "fp8+bf16 (fp32 accumulate)", "data": "synthetic",
           "config": head.pop("config")}
    res.update(head)
    extra = [k for k in args.also.split(",") if k and k != args.workload] \
        if not args.only_composite else []
    if extra:
        res["workloads"] = {}
        for key in extra:
            rec = measure(wl.WORKLOADS[key], args, lcs, headline=False)
            res["workloads"][key] = rec
    if not args.no_cpu_baseline and not args.only_composite:
        res["cpu_baseline"] = cpu_baseline(w, args.workload)
        for key in extra:
            res["workloads"][key]["cpu_baseline"] = cpu_baseline(wl.WORKLOADS[key], key)
            print("cpu baseline %s done" % key, file=sys.stderr, flush=True)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
