"""Python binding of liblcs.so, the gfx950 DSA + IndexShare attention path.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
declared in include/lcs.h. PyTorch supplies device memory and the current
stream. Importing fails loudly if the library has not been built; there is no
fallback implementation.
"""
import ctypes
import os

# torch first: its HIP runtime (soname libamdhip64.so.7) is then the one the
# process uses, and liblcs.so binds to it instead of loading a second runtime
import torch  # noqa: F401

__all__ = [
    "LcsError", "idx_score", "topk_workspace_bytes", "topk_select", "attn_workspace_bytes",
    "sparse_mla_attn", "count_full_layers", "indexshare_workspace_bytes", "indexshare_forward",
    "SCHED_GROUP4", "SCHED_GLM52", "SCHED_ALL_FULL", "SCHED_MASK", "KV_BF16", "KV_FP8_E4M3",
    "LIB_PATH", "quantize_e4m3", "cache_append", "topk_candidates", "topk_merge", "idx_localize",
    "lse_combine", "Paged", "idx_score_paged", "sparse_mla_attn_paged", "cache_append_paged",
    "sparse_mla_attn_noalloc",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblcs.so")
if not os.path.exists(LIB_PATH):
    raise ImportError("%s is missing: run __graft_entry__.build() first" % LIB_PATH)
_lib = ctypes.CDLL(LIB_PATH)

SCHED_GROUP4, SCHED_GLM52, SCHED_ALL_FULL, SCHED_MASK = 0, 1, 2, 3
KV_BF16, KV_FP8_E4M3 = 0, 1
IDX_HEADS, IDX_DIM, ATT_HEADS, KV_LATENT, KV_DIM = 32, 128, 64, 512, 576

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t
_f32 = ctypes.c_float


class _PagedC(ctypes.Structure):
    _fields_ = [("block_table", _p), ("max_blocks", _i32), ("block_size", _i32),
                ("n_blocks", _i32)]


class Paged:
    """A paged cache layout: block_table [B, max_blocks] int32 device tensor mapping each
    sequence's position blocks to pool blocks of block_size rows; n_blocks pool blocks."""

    def __init__(self, block_table, block_size, n_blocks):
        self.block_table = block_table
        self.block_size = int(block_size)
        self.n_blocks = int(n_blocks)

    def _c(self):
        return ctypes.byref(_PagedC(self.block_table.data_ptr(), self.block_table.shape[1],
                                    self.block_size, self.n_blocks))


class _Layer(ctypes.Structure):
    _fields_ = [(n, _p) for n in ("q8", "q_scale", "w", "k8", "k_scale", "q", "kv", "kv_scale",
                                  "out", "lse")]


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_i64 = ctypes.c_int64
_c_idx_score = _sig("lcs_idx_score", ctypes.c_int, [_p] * 5 + [_i64, _p] + [_i32] * 3 + [_p, _p])
_c_topk_ws = _sig("lcs_topk_workspace_bytes", _sz, [_i32] * 4)
_c_topk = _sig("lcs_topk_select", ctypes.c_int, [_p, _p] + [_i32] * 4 + [_p, _p, _sz, _p])
_c_attn_ws = _sig("lcs_attn_workspace_bytes", _sz, [_i32] * 3)
_c_attn = _sig("lcs_sparse_mla_attn", ctypes.c_int,
               [_p, _p, ctypes.c_int, _p, _i64, _p] + [_i32] * 4 + [_f32, _p, _p, _p, _sz, _p])
_c_attn_na = _sig("lcs_sparse_mla_attn_noalloc", ctypes.c_int,
                  [_p, _p, ctypes.c_int, _p, _i64, _p] + [_i32] * 4 + [_f32, _p, _p, _p])
_c_count = _sig("lcs_count_full_layers", _i32, [ctypes.c_int, _i32, _p, _i32])
_c_is_ws = _sig("lcs_indexshare_workspace_bytes", _sz, [_i32] * 4)
_c_is = _sig("lcs_indexshare_forward", ctypes.c_int,
             [ctypes.POINTER(_Layer), _i32, ctypes.c_int, _p, _i32, ctypes.c_int, _p]
             + [_i32] * 4 + [_f32, _p, _p, _p, _sz, _p])
_c_quant = _sig("lcs_quantize_e4m3", ctypes.c_int, [_p, ctypes.c_int64, _i32, _p, _p, _p])
_c_append = _sig("lcs_cache_append", ctypes.c_int,
                 [_p, _p, ctypes.c_int, _p] + [_i32] * 3 + [_p] * 5)
_c_cand = _sig("lcs_topk_candidates", ctypes.c_int, [_p, _p] + [_i32] * 5 + [_p, _p, _p])
_c_merge = _sig("lcs_topk_merge", ctypes.c_int, [_p, _p] + [_i32] * 5 + [_p, _p])
_c_local = _sig("lcs_idx_localize", ctypes.c_int, [_p] + [_i32] * 5 + [_p, _p])
_c_comb = _sig("lcs_lse_combine", ctypes.c_int, [_p, _p] + [_i32] * 3 + [_p, _p, _p])
_c_idx_paged = _sig("lcs_idx_score_paged", ctypes.c_int, [_p] * 6 + [_p] + [_i32] * 3 + [_p, _p])
_c_attn_paged = _sig("lcs_sparse_mla_attn_paged", ctypes.c_int,
                     [_p, _p, ctypes.c_int, _p, _p, _p] + [_i32] * 4 + [_f32, _p, _p, _p, _sz, _p])
_c_append_paged = _sig("lcs_cache_append_paged", ctypes.c_int,
                       [_p, _p, ctypes.c_int, _p] + [_i32] * 3 + [_p] * 6)
_c_status = _sig("lcs_status_string", ctypes.c_char_p, [ctypes.c_int])
_c_last = _sig("lcs_last_error", ctypes.c_char_p, [])


class LcsError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__("lcs status %d (%s): %s" % (status, _c_status(status).decode(), detail))


def _check(rc):
    if rc != 0:
        raise LcsError(rc, _c_last().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _batch_stride(cache, row_width, scale=None):
    """Rows from one sequence of a [B, L, row_width] cache view to the next (its rows
    themselves dense), checked against the view of its per-row scales [B, L]"""
    if cache.dim() != 3 or cache.shape[2] != row_width or cache.stride(2) != 1 or \
            (cache.shape[1] > 1 and cache.stride(1) != row_width) or cache.stride(0) % row_width:
        raise ValueError("cache must be a [B, L, %d] view with dense rows" % row_width)
    stride = cache.stride(0) // row_width
    if cache.shape[0] == 1:
        stride = cache.shape[1]
    if scale is not None and scale.shape[0] > 1 and \
            (scale.stride(1) != 1 or scale.stride(0) != stride):
        raise ValueError("scales must have the cache's batch stride (%d rows)" % stride)
    if scale is not None and scale.stride(-1) != 1:
        raise ValueError("scales must be dense along L")
    return stride


def _stream(stream):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


def idx_score(q8, q_scale, w, k8, k_scale, vis_len, scores, stream=None):
    """scores[B,T,L] (fp32) from q8[B,T,32,128], q_scale/w[B,T,32], k8[B,L,128],
    k_scale[B,L], vis_len[B,T] (int32). k8/k_scale may be views of a longer cache
    (k8[:, :L]): their batch stride is passed on."""
    B, T = q8.shape[0], q8.shape[1]
    L = k8.shape[1]
    _check(_c_idx_score(_ptr(q8), _ptr(q_scale), _ptr(w), _ptr(k8), _ptr(k_scale),
                        _batch_stride(k8, IDX_DIM, k_scale), _ptr(vis_len), B, T, L,
                        _ptr(scores), _stream(stream)))


def topk_workspace_bytes(B, T, L, k):
    return int(_c_topk_ws(B, T, L, k))


def topk_select(scores, vis_len, k, idx, workspace, stream=None):
    """idx[B,T,k] (int32) from scores[B,T,L]; workspace: uint8 device tensor of at least
    topk_workspace_bytes(B, T, L, k) bytes."""
    B, T, L = scores.shape
    _check(_c_topk(_ptr(scores), _ptr(vis_len), B, T, L, k, _ptr(idx), _ptr(workspace),
                   0 if workspace is None else workspace.numel() * workspace.element_size(),
                   _stream(stream)))


def attn_workspace_bytes(B, T, k):
    return int(_c_attn_ws(B, T, k))


def _kv_dtype(kv):
    import torch
    if kv.dtype in (torch.uint8, torch.float8_e4m3fn):
        return KV_FP8_E4M3
    return KV_BF16


def sparse_mla_attn(q, kv, kv_scale, idx, sm_scale, out, lse=None, workspace=None, stream=None):
    """out[B,T,64,512] (bf16) from q[B,T,64,576] (bf16), kv[B,L,576] (bf16, or uint8 E4M3
    codes with kv_scale[B,L]), idx[B,T,k]. kv/kv_scale may be views of a longer cache."""
    B, T = q.shape[0], q.shape[1]
    L = kv.shape[1]
    k = idx.shape[-1]
    _check(_c_attn(_ptr(q), _ptr(kv), _kv_dtype(kv), _ptr(kv_scale),
                   _batch_stride(kv, KV_DIM, kv_scale), _ptr(idx), B, T, L, k,
                   float(sm_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                   0 if workspace is None else workspace.numel() * workspace.element_size(),
                   _stream(stream)))


def sparse_mla_attn_noalloc(q, kv, kv_scale, idx, sm_scale, out, lse=None, stream=None):
    """sparse_mla_attn with its split partials in the library's static scratch (no
    workspace; calls on one GPU must not overlap in time)."""
    B, T = q.shape[0], q.shape[1]
    L = kv.shape[1]
    k = idx.shape[-1]
    _check(_c_attn_na(_ptr(q), _ptr(kv), _kv_dtype(kv), _ptr(kv_scale),
                      _batch_stride(kv, KV_DIM, kv_scale), _ptr(idx), B, T, L, k,
                      float(sm_scale), _ptr(out), _ptr(lse), _stream(stream)))


def count_full_layers(sched, n_layers, full_mask=None, mtp_steps=0):
    buf = None
    if full_mask is not None:
        buf = (ctypes.c_uint8 * n_layers)(*[1 if x else 0 for x in full_mask])
    n = _c_count(sched, n_layers, ctypes.cast(buf, _p) if buf is not None else None, mtp_steps)
    if n < 0:
        raise ValueError("invalid schedule arguments")
    return int(n)


def indexshare_workspace_bytes(B, T, L, k):
    return int(_c_is_ws(B, T, L, k))


def indexshare_forward(layers, sched, vis_len, k, sm_scale, scores_scratch, idx_out, workspace,
                       kv_dtype=KV_BF16, mtp_steps=0, full_mask=None, stream=None):
    """layers: list of dicts with keys q8, q_scale, w, k8, k_scale (full layers), q, kv,
    kv_scale, out, lse (tensors or None). Shapes as in the single calls."""
    n = len(layers)
    arr = (_Layer * n)()
    for i, ly in enumerate(layers):
        for f, _ in _Layer._fields_:
            setattr(arr[i], f, _ptr(ly.get(f)))
    B, T = vis_len.shape
    L = scores_scratch.shape[-1]
    buf = None
    if full_mask is not None:
        buf = (ctypes.c_uint8 * n)(*[1 if x else 0 for x in full_mask])
    _check(_c_is(arr, n, sched, ctypes.cast(buf, _p) if buf is not None else None, mtp_steps,
                 kv_dtype, _ptr(vis_len), B, T, L, k, float(sm_scale), _ptr(scores_scratch),
                 _ptr(idx_out), _ptr(workspace),
                 workspace.numel() * workspace.element_size() if workspace is not None else 0,
                 _stream(stream)))


def quantize_e4m3(x, codes, scales, stream=None):
    """codes[..., D] (uint8 E4M3) and scales[...] (fp32) from x[..., D] (bf16), D = 128 or
    576: one scale per row, scale = max|x| / 448."""
    D = x.shape[-1]
    _check(_c_quant(_ptr(x), x.numel() // D if D else 0, D, _ptr(codes), _ptr(scales),
                    _stream(stream)))


def cache_append(pos, k_new=None, k8=None, k_scale=None, kv_new=None, kv=None, kv_scale=None,
                 stream=None):
    """Writes token (b, t) of k_new[B,T,128] / kv_new[B,T,576] (bf16) into row pos[b,t]
    (int32) of k8[B,L,128] + k_scale[B,L] and of kv[B,L,576] (bf16, or uint8 E4M3 codes
    with kv_scale[B,L]); positions outside [0, L) are skipped."""
    B, T = pos.shape
    L = (k8 if k8 is not None else kv).shape[1]
    kd = _kv_dtype(kv) if kv is not None else KV_BF16
    _check(_c_append(_ptr(k_new), _ptr(kv_new), kd, _ptr(pos), B, T, L, _ptr(k8), _ptr(k_scale),
                     _ptr(kv), _ptr(kv_scale), _stream(stream)))


def topk_candidates(scores, idx, pos_base, cand_score, cand_idx, stream=None):
    """cand_score/cand_idx[B,T,k] = (scores[b,t,idx], idx + pos_base) of one shard's
    selection idx[B,T,k] over its scores[B,T,L]; (-inf, -1) for empty slots."""
    B, T, L = scores.shape
    k = idx.shape[-1]
    _check(_c_cand(_ptr(scores), _ptr(idx), B, T, L, k, int(pos_base), _ptr(cand_score),
                   _ptr(cand_idx), _stream(stream)))


def topk_merge(cand_score, cand_idx, k, idx, stream=None):
    """idx[B,T,k] from the candidates cand_*[G,B,T,k_in] of G shards."""
    G, B, T, k_in = cand_idx.shape
    _check(_c_merge(_ptr(cand_score), _ptr(cand_idx), G, B, T, k_in, k, _ptr(idx),
                    _stream(stream)))


def idx_localize(idx, lo, hi, local, stream=None):
    """local[B,T,k] = entries of idx[B,T,k] in [lo, hi), minus lo, then -1."""
    B, T, k = idx.shape
    _check(_c_local(_ptr(idx), B, T, k, int(lo), int(hi), _ptr(local), _stream(stream)))


def lse_combine(part_out, part_lse, out, lse=None, stream=None):
    """out[B,T,64,512] (and lse[B,T,64]) from G shard outputs part_out[G,B,T,64,512] (bf16)
    and part_lse[G,B,T,64] (fp32, natural log)."""
    G, B, T = part_out.shape[:3]
    _check(_c_comb(_ptr(part_out), _ptr(part_lse), G, B, T, _ptr(out), _ptr(lse),
                   _stream(stream)))


def idx_score_paged(q8, q_scale, w, k8_pool, k_scale_pool, paged, vis_len, L, scores,
                    stream=None):
    """lcs_idx_score over the key pools k8_pool [n_blocks, bs, 128] / k_scale_pool
    [n_blocks, bs] of a Paged layout; scores [B, T, L]."""
    B, T = q8.shape[0], q8.shape[1]
    _check(_c_idx_paged(_ptr(q8), _ptr(q_scale), _ptr(w), _ptr(k8_pool), _ptr(k_scale_pool),
                        paged._c(), _ptr(vis_len), B, T, L, _ptr(scores), _stream(stream)))


def sparse_mla_attn_paged(q, kv_pool, kv_scale_pool, paged, idx, L, sm_scale, out, lse=None,
                          workspace=None, stream=None):
    """lcs_sparse_mla_attn over the latent pool kv_pool [n_blocks, bs, 576] (bf16, or uint8
    E4M3 codes with kv_scale_pool [n_blocks, bs]) of a Paged layout."""
    B, T = q.shape[0], q.shape[1]
    k = idx.shape[-1]
    _check(_c_attn_paged(_ptr(q), _ptr(kv_pool), _kv_dtype(kv_pool), _ptr(kv_scale_pool),
                         paged._c(), _ptr(idx), B, T, L, k, float(sm_scale), _ptr(out), _ptr(lse),
                         _ptr(workspace),
                         0 if workspace is None else workspace.numel() * workspace.element_size(),
                         _stream(stream)))


def cache_append_paged(pos, L, paged, k_new=None, k8_pool=None, k_scale_pool=None, kv_new=None,
                       kv_pool=None, kv_scale_pool=None, stream=None):
    """lcs_cache_append into the pools of a Paged layout (positions outside [0, L) skipped)."""
    B, T = pos.shape
    kd = _kv_dtype(kv_pool) if kv_pool is not None else KV_BF16
    _check(_c_append_paged(_ptr(k_new), _ptr(kv_new), kd, _ptr(pos), B, T, L, paged._c(),
                           _ptr(k8_pool), _ptr(k_scale_pool), _ptr(kv_pool), _ptr(kv_scale_pool),
                           _stream(stream)))
