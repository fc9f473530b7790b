"""TEST INFRASTRUCTURE ONLY: ctypes front end of liboracle.so, the plain C
double-precision oracle (oracle.c). Only the tests, the smoke check and the
benchmark's CPU-baseline leg import this; the product path never does.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_lib = ctypes.CDLL(os.path.join(HERE, "liboracle.so"))
_p, _i32 = ctypes.c_void_p, ctypes.c_int32

_lib.oracle_e4m3.argtypes = [ctypes.c_uint8]
_lib.oracle_e4m3.restype = ctypes.c_double
_lib.oracle_bf16.argtypes = [ctypes.c_uint16]
_lib.oracle_bf16.restype = ctypes.c_double
_lib.oracle_round_bf16.argtypes = [ctypes.c_double]
_lib.oracle_round_bf16.restype = ctypes.c_uint16
_lib.oracle_idx_score.argtypes = [_p] * 6 + [_i32] * 3 + [_p, _p]
_lib.oracle_topk.argtypes = [_p, _p] + [_i32] * 4 + [_p]
_lib.oracle_sparse_mla.argtypes = [_p, _p, _i32, _p, _p] + [_i32] * 4 + [ctypes.c_double] + [_p] * 3
_lib.oracle_is_full_layer.argtypes = [_i32, _i32, _p]
for _f in ("oracle_idx_score", "oracle_topk", "oracle_sparse_mla", "oracle_is_full_layer",
           "oracle_indexshare"):
    getattr(_lib, _f).restype = ctypes.c_int

SCHED_GROUP4, SCHED_GLM52, SCHED_ALL_FULL, SCHED_MASK = 0, 1, 2, 3


class _Layer(ctypes.Structure):
    _fields_ = [(n, _p) for n in ("q8", "q_scale", "w", "k8", "k_scale", "q", "kv", "kv_scale",
                                  "out", "lse")]


_lib.oracle_indexshare.argtypes = [ctypes.POINTER(_Layer), _i32, _i32, _p, _i32, _i32, _p] + \
    [_i32] * 4 + [ctypes.c_double, _p]


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _check(rc, what):
    if rc != 0:
        raise ValueError("oracle %s rejected its input (code %d)" % (what, rc))


def e4m3(code):
    return _lib.oracle_e4m3(int(code))


def bf16(bits):
    return _lib.oracle_bf16(int(bits))


def round_bf16(x):
    return int(_lib.oracle_round_bf16(float(x)))


def idx_score(q8, q_scale, w, k8, k_scale, vis_len, want64=False):
    """q8[B,T,32,128] u8, q_scale/w[B,T,32] f32, k8[B,L,128] u8, k_scale[B,L] f32,
    vis_len[B,T] i32 -> scores[B,T,L] f32 (and the double values if want64)"""
    q8, k8 = _c(q8, np.uint8), _c(k8, np.uint8)
    q_scale, w, k_scale = _c(q_scale, np.float32), _c(w, np.float32), _c(k_scale, np.float32)
    vis_len = _c(vis_len, np.int32)
    B, T = q8.shape[0], q8.shape[1]
    L = k8.shape[1]
    assert q8.shape == (B, T, 32, 128) and k8.shape == (B, L, 128)
    assert q_scale.shape == (B, T, 32) and w.shape == (B, T, 32) and k_scale.shape == (B, L)
    assert vis_len.shape == (B, T)
    out = np.empty((B, T, L), np.float32)
    out64 = np.empty((B, T, L), np.float64) if want64 else None
    _check(_lib.oracle_idx_score(q8.ctypes.data, q_scale.ctypes.data, w.ctypes.data,
                                 k8.ctypes.data, k_scale.ctypes.data, vis_len.ctypes.data, B, T,
                                 L, out.ctypes.data, out64.ctypes.data if want64 else None),
           "idx_score")
    return (out, out64) if want64 else out


def topk(scores, vis_len, k):
    scores = _c(scores, np.float32)
    vis_len = _c(vis_len, np.int32)
    B, T, L = scores.shape
    idx = np.empty((B, T, k), np.int32)
    _check(_lib.oracle_topk(scores.ctypes.data, vis_len.ctypes.data, B, T, L, k, idx.ctypes.data),
           "topk")
    return idx


def sparse_mla(q, kv, kv_scale, idx, sm_scale, L=None, want64=False):
    """q[B,T,64,576] bf16 bits (u16), kv[B,L,576] bf16 bits (u16) or E4M3 codes (u8) with
    kv_scale[B,L], idx[B,T,k] -> (out bf16 bits [B,T,64,512], lse f32 [B,T,64][, out64])"""
    q = _c(q, np.uint16)
    fp8 = kv.dtype == np.uint8
    kv = _c(kv, np.uint8 if fp8 else np.uint16)
    idx = _c(idx, np.int32)
    B, T = q.shape[0], q.shape[1]
    L = kv.shape[1] if L is None else L
    k = idx.shape[-1]
    ks = _c(kv_scale, np.float32) if fp8 else None
    out = np.empty((B, T, 64, 512), np.uint16)
    lse = np.empty((B, T, 64), np.float32)
    out64 = np.empty((B, T, 64, 512), np.float64) if want64 else None
    _check(_lib.oracle_sparse_mla(q.ctypes.data, kv.ctypes.data, 1 if fp8 else 0,
                                  ks.ctypes.data if fp8 else None, idx.ctypes.data, B, T, L, k,
                                  float(sm_scale), out.ctypes.data, lse.ctypes.data,
                                  out64.ctypes.data if want64 else None), "sparse_mla")
    return (out, lse, out64) if want64 else (out, lse)


def is_full_layer(sched, l, mask=None):
    buf = None if mask is None else np.ascontiguousarray(mask, np.uint8)
    return bool(_lib.oracle_is_full_layer(sched, l, buf.ctypes.data if buf is not None else None))


def indexshare(layers, sched, vis_len, k, sm_scale, kv_fp8=False, mtp_steps=0, mask=None):
    """layers: list of dicts of numpy arrays (q8, q_scale, w, k8, k_scale on full layers;
    q, kv, kv_scale always). Returns (outs, lses, idx_out)."""
    n = len(layers)
    keep = []
    arr = (_Layer * n)()
    vis_len = _c(vis_len, np.int32)
    B, T = vis_len.shape
    L = None
    outs, lses = [], []
    for i, ly in enumerate(layers):
        conv = {}
        for f, dt in (("q8", np.uint8), ("q_scale", np.float32), ("w", np.float32),
                      ("k8", np.uint8), ("k_scale", np.float32), ("q", np.uint16),
                      ("kv", np.uint8 if kv_fp8 else np.uint16), ("kv_scale", np.float32)):
            if ly.get(f) is not None:
                conv[f] = _c(ly[f], dt)
                setattr(arr[i], f, conv[f].ctypes.data)
        if "kv" in conv:
            L = conv["kv"].shape[1]
        o = np.empty((B, T, 64, 512), np.uint16)
        s = np.empty((B, T, 64), np.float32)
        arr[i].out, arr[i].lse = o.ctypes.data, s.ctypes.data
        outs.append(o)
        lses.append(s)
        keep.append(conv)
    n_full = 1 if mtp_steps else sum(is_full_layer(sched, l, mask) for l in range(n))
    idx_out = np.empty((n_full, B, T, k), np.int32)
    mbuf = None if mask is None else np.ascontiguousarray(mask, np.uint8)
    _check(_lib.oracle_indexshare(arr, n, sched, mbuf.ctypes.data if mbuf is not None else None,
                                  mtp_steps, 1 if kv_fp8 else 0, vis_len.ctypes.data, B, T, L, k,
                                  float(sm_scale), idx_out.ctypes.data), "indexshare")
    return outs, lses, idx_out


_lib.oracle_encode_e4m3.argtypes = [ctypes.c_double]
_lib.oracle_encode_e4m3.restype = ctypes.c_uint8
_lib.oracle_quantize_e4m3.argtypes = [_p, ctypes.c_int64, _i32, _p, _p]
_lib.oracle_quantize_e4m3.restype = ctypes.c_int
_lib.oracle_cache_append.argtypes = [_p, _p, _i32, _p] + [_i32] * 3 + [_p] * 4
_lib.oracle_cache_append.restype = ctypes.c_int


def encode_e4m3(v):
    """finite value -> E4M3 code (saturating, nearest, ties to the even code)"""
    return int(_lib.oracle_encode_e4m3(float(v)))


def quantize_e4m3(x_bits):
    """x_bits [..., D] uint16 bf16 bits -> (codes uint8 [..., D], scales f32 [...])"""
    x = _c(x_bits, np.uint16)
    D = x.shape[-1]
    rows = x.size // D
    codes = np.empty(x.shape, np.uint8)
    scales = np.empty(x.shape[:-1], np.float32)
    _check(_lib.oracle_quantize_e4m3(x.ctypes.data, rows, D, codes.ctypes.data,
                                     scales.ctypes.data), "quantize_e4m3")
    return codes, scales


def cache_append(k_new, kv_new, pos, k8, k_scale, kv, kv_scale):
    """Writes the new tokens into copies of the caches and returns them.
    k_new [B][T][128] / kv_new [B][T][576] uint16 bf16 bits (either may be
    None), pos [B][T] int32; k8 [B][L][128] u8, k_scale [B][L] f32,
    kv [B][L][576] (uint16 bf16 bits, or uint8 codes with kv_scale [B][L]).
    Returns (k8, k_scale, kv, kv_scale) with None where not given."""
    pos = _c(pos, np.int32)
    B, T = pos.shape
    kn = _c(k_new, np.uint16) if k_new is not None else None
    vn = _c(kv_new, np.uint16) if kv_new is not None else None
    k8o = np.array(k8, np.uint8, copy=True) if k8 is not None else None
    kso = np.array(k_scale, np.float32, copy=True) if k_scale is not None else None
    fp8 = kv is not None and np.asarray(kv).dtype == np.uint8
    kvo = np.array(kv, np.uint8 if fp8 else np.uint16, copy=True) if kv is not None else None
    kvso = np.array(kv_scale, np.float32, copy=True) if kv_scale is not None else None
    L = (k8o if k8o is not None else kvo).shape[1]
    ptr = lambda a: a.ctypes.data if a is not None else None  # noqa: E731
    _check(_lib.oracle_cache_append(ptr(kn), ptr(vn), int(fp8), pos.ctypes.data, B, T, L,
                                    ptr(k8o), ptr(kso), ptr(kvo), ptr(kvso)), "cache_append")
    return k8o, kso, kvo, kvso


_lib.oracle_topk_candidates.argtypes = [_p, _p] + [_i32] * 4 + [_p, _p]
_lib.oracle_topk_merge.argtypes = [_p, _p] + [_i32] * 4 + [_p]
_lib.oracle_idx_localize.argtypes = [_p] + [_i32] * 4 + [_p]
_lib.oracle_lse_combine.argtypes = [_p, _p, _i32, _i32, _p, _p, _p]
for _f in ("oracle_topk_candidates", "oracle_topk_merge", "oracle_idx_localize",
           "oracle_lse_combine"):
    getattr(_lib, _f).restype = ctypes.c_int


def topk_candidates(scores, idx, pos_base):
    """scores [..., L] f32, idx [..., k] i32 -> (cand_score [..., k], cand_idx [..., k])"""
    s = _c(scores, np.float32)
    ix = _c(idx, np.int32)
    L, k = s.shape[-1], ix.shape[-1]
    Q = ix.size // k
    cs = np.empty(ix.shape, np.float32)
    ci = np.empty(ix.shape, np.int32)
    _check(_lib.oracle_topk_candidates(s.ctypes.data, ix.ctypes.data, Q, L, k, pos_base,
                                       cs.ctypes.data, ci.ctypes.data), "topk_candidates")
    return cs, ci


def topk_merge(cand_score, cand_idx, k):
    """cand_* [G, ..., k_in] -> idx [..., k]"""
    cs = _c(cand_score, np.float32)
    ci = _c(cand_idx, np.int32)
    G, k_in = ci.shape[0], ci.shape[-1]
    Q = ci.size // (G * k_in)
    out = np.empty(ci.shape[1:-1] + (k,), np.int32)
    _check(_lib.oracle_topk_merge(cs.ctypes.data, ci.ctypes.data, G, Q, k_in, k, out.ctypes.data),
           "topk_merge")
    return out


def idx_localize(idx, lo, hi):
    ix = _c(idx, np.int32)
    k = ix.shape[-1]
    out = np.empty_like(ix)
    _check(_lib.oracle_idx_localize(ix.ctypes.data, ix.size // k, k, lo, hi, out.ctypes.data),
           "idx_localize")
    return out


def lse_combine(part_out, part_lse, want64=False):
    """part_out [G, ..., 64, 512] uint16 bf16 bits, part_lse [G, ..., 64] f32 ->
    (out uint16 [..., 64, 512], lse f32 [..., 64][, out64])"""
    po = _c(part_out, np.uint16)
    pl = _c(part_lse, np.float32)
    G = po.shape[0]
    Q = po.size // (G * 64 * 512)
    out = np.empty(po.shape[1:], np.uint16)
    lse = np.empty(pl.shape[1:], np.float32)
    o64 = np.empty(po.shape[1:], np.float64) if want64 else None
    _check(_lib.oracle_lse_combine(po.ctypes.data, pl.ctypes.data, G, Q, out.ctypes.data,
                                   lse.ctypes.data, o64.ctypes.data if want64 else None),
           "lse_combine")
    return (out, lse, o64) if want64 else (out, lse)
