"""Helpers shared by the GPU parity tests, the smoke check and the benchmark's
sampled checks: host<->device transfer and the acceptance rules.

Acceptance rules (all stated as tolerances of the outputs):
  scores   |gpu - ref| <= 1e-3 * |ref| + 1e-6 * max_s |ref[row]| (the second
           term covers ReLU zeros); -inf exactly where the reference is -inf;
           on arbitrary E4M3 bytes also + 1e-3 of the terms' magnitude
  top-k    bit-identical when fed the reference scores
  end-to-end selections: per query, every position in the symmetric difference
           lies within 1e-3 (relative) of the reference threshold score tau
           (the reference's m-th largest score), and over all queries the
           overlap is >= 99.9 % of the selected positions
  attention max |gpu - ref| <= 2e-2 on the bf16 outputs (reported with the
           ratio to the output RMS), lse within 2e-3 absolute
"""
import numpy as np
import torch

DEV = "cuda:0"


def to_dev(a, dtype=None):
    """numpy -> device tensor. uint16 arrays are bf16 bit patterns."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    t = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return t if dtype is None else t.to(dtype)


def bf16_to_f64(x):
    """bf16 tensor (device or host) or uint16 numpy bits -> float64 numpy"""
    if isinstance(x, np.ndarray):
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double().numpy()
    return x.detach().to("cpu").double().numpy()


def check_scores(gpu, ref64, what="scores", terms=None):
    """terms (optional, same shape): the score formula over the magnitudes of its
    terms, k_scale * sum_j w_j q_scale_j sum_i |q_ji k_i|. When given, each score
    may also differ by 1e-3 of it: the FP8 matrix cores accumulate a dot product
    with less than fp32 precision (measured: within 1e-4 of the terms' magnitude),
    which only shows where a head's dot product cancels, as on arbitrary bytes."""
    gpu = np.asarray(gpu, np.float64)
    ninf = np.isneginf(ref64)
    assert np.array_equal(np.isneginf(gpu), ninf), what + ": -inf pattern differs"
    fin = ~ninf
    rowmax = np.where(fin, np.abs(ref64), 0).max(axis=-1, keepdims=True)
    err = np.abs(np.where(fin, gpu, 0) - np.where(fin, ref64, 0))
    bound = 1e-3 * np.abs(np.where(fin, ref64, 0)) + 1e-6 * rowmax
    if terms is not None:
        bound = bound + 1e-3 * np.where(fin, terms, 0)
    bad = err > bound
    assert not bad.any(), "%s: %d elements out of tolerance, worst rel %.3g" % (
        what, int(bad.sum()), float((err / np.maximum(np.abs(np.where(fin, ref64, 1)), 1e-30)).max()))
    rel = err[fin] / np.maximum(np.abs(ref64[fin]), 1e-30)
    return float(rel.max()) if rel.size else 0.0


def check_selection(gpu_idx, ref_idx, ref_scores64, rel_gap=1e-3, min_overlap=0.999):
    """gpu_idx/ref_idx [..., k] (ascending, -1 padded); ref_scores64 [..., L]"""
    gpu_idx = np.asarray(gpu_idx).reshape(-1, gpu_idx.shape[-1])
    ref_idx = np.asarray(ref_idx).reshape(-1, ref_idx.shape[-1])
    sc = np.asarray(ref_scores64).reshape(-1, ref_scores64.shape[-1])
    total = inter = 0
    worst_gap = 0.0
    for r in range(ref_idx.shape[0]):
        a = set(int(x) for x in gpu_idx[r] if x >= 0)
        b = set(int(x) for x in ref_idx[r] if x >= 0)
        assert len(a) == len(b), "row %d: %d vs %d selected" % (r, len(a), len(b))
        assert np.all(np.diff(gpu_idx[r][gpu_idx[r] >= 0]) > 0), "row %d not ascending" % r
        total += len(b)
        inter += len(a & b)
        if a != b:
            tau = min(sc[r, s] for s in b)
            for s in a ^ b:
                gap = abs(sc[r, s] - tau) / max(abs(tau), 1e-30)
                worst_gap = max(worst_gap, gap)
                assert gap <= rel_gap, "row %d pos %d: score gap %.3g to tau" % (r, s, gap)
    overlap = inter / max(total, 1)
    assert overlap >= min_overlap, "overlap %.5f" % overlap
    return overlap, worst_gap


def check_attention(gpu_out, ref_out64, gpu_lse=None, ref_lse=None, atol=2e-2):
    g = bf16_to_f64(gpu_out)
    err = np.abs(g - ref_out64)
    mx = float(err.max())
    rms = float(np.sqrt(np.mean(ref_out64 ** 2)))
    assert mx <= atol, "attention max-abs %.4g (rms of reference %.4g)" % (mx, rms)
    lse_err = 0.0
    if gpu_lse is not None:
        gl = gpu_lse.detach().cpu().numpy().astype(np.float64)
        fin = np.isfinite(ref_lse)
        assert np.array_equal(np.isneginf(gl), np.isneginf(ref_lse))
        lse_err = float(np.abs(gl[fin] - ref_lse[fin]).max()) if fin.any() else 0.0
        assert lse_err <= 2e-3, "lse error %.3g" % lse_err
    return mx, mx / max(rms, 1e-30), lse_err
