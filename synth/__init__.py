"""Seeded synthetic inputs (host numpy or device torch), shared by tests, the
benchmark and the smoke check. Holds none of the method's arithmetic; see
synth.h for the generator definition. Host and device fills of the same block
are bit-identical.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))

T_IDX_KEY, T_IDX_Q, T_IDX_W, T_ATT_Q, T_KV = 1, 2, 3, 4, 5
IDX_HEADS, IDX_DIM, ATT_HEADS, KV_DIM = 32, 128, 64, 576

_p = ctypes.c_void_p
_u64, _u32, _i32, _i64 = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int32, ctypes.c_int64

_host = ctypes.CDLL(os.path.join(HERE, "libsynth_host.so"))
_host.synth_host_fp8_rows.argtypes = [_u64, _u32, _u32, _i64, _i32, _u32, _i32, _i32, _i64, _i64,
                                      _p, _p]
_host.synth_host_bf16_rows.argtypes = [_u64, _u32, _u32, _i32, _i32, _i32, _i64, _i64, _p]
_host.synth_host_uniform_rows.argtypes = [_u64, _u32, _u32, _i32, _i32, _i32, _i64, _i64, _p]
_host.synth_host_planted.argtypes = [_u64, _u32, _i32, _i64, _u32, _i64, _i64, _p]
_host.synth_host_e4m3.argtypes = [ctypes.c_double]
_host.synth_host_e4m3.restype = ctypes.c_uint8
_host.synth_host_bf16.argtypes = [ctypes.c_float]
_host.synth_host_bf16.restype = ctypes.c_uint16
for _f in ("synth_host_fp8_rows", "synth_host_bf16_rows", "synth_host_uniform_rows",
           "synth_host_planted"):
    getattr(_host, _f).restype = ctypes.c_int

_dev = None


def _devlib():
    global _dev
    if _dev is None:
        import torch  # noqa: F401  (one HIP runtime per process: torch's, loaded first)
        _dev = ctypes.CDLL(os.path.join(HERE, "libsynth_dev.so"))
        _dev.synth_dev_fp8_rows.argtypes = [_u64, _u32, _u32, _i64, _i32, _u32, _i32, _i32, _i64,
                                            _i64, _p, _p, _p]
        _dev.synth_dev_bf16_rows.argtypes = [_u64, _u32, _u32, _i32, _i32, _i32, _i64, _i64, _p,
                                             _p]
        _dev.synth_dev_uniform_rows.argtypes = [_u64, _u32, _u32, _i32, _i32, _i32, _i64, _i64,
                                                _p, _p]
    return _dev


def _ok(rc, what):
    if rc != 0:
        raise RuntimeError("%s failed (%d)" % (what, rc))


# ---------------------------------------------------------------- host fills
def host_fp8_rows(seed, tensor, layer, R, D, permyriad, b0, nb, r0, nr):
    codes = np.empty((nb, nr, D), np.uint8)
    scales = np.empty((nb, nr), np.float32)
    _ok(_host.synth_host_fp8_rows(seed, tensor, layer, R, D, permyriad, b0, nb, r0, nr,
                                  codes.ctypes.data, scales.ctypes.data), "host fp8 fill")
    return codes, scales


def host_bf16_rows(seed, tensor, layer, D, b0, nb, r0, nr):
    out = np.empty((nb, nr, D), np.uint16)
    _ok(_host.synth_host_bf16_rows(seed, tensor, layer, D, b0, nb, r0, nr, out.ctypes.data),
        "host bf16 fill")
    return out


def host_uniform_rows(seed, tensor, layer, D, b0, nb, r0, nr):
    out = np.empty((nb, nr, D), np.float32)
    _ok(_host.synth_host_uniform_rows(seed, tensor, layer, D, b0, nb, r0, nr, out.ctypes.data),
        "host uniform fill")
    return out


def host_planted(seed, layer, b, R, permyriad, r0=0, nr=None):
    nr = R - r0 if nr is None else nr
    out = np.empty(nr, np.uint8)
    _host.synth_host_planted(seed, layer, b, R, permyriad, r0, nr, out.ctypes.data)
    return out


def e4m3_encode(v):
    return int(_host.synth_host_e4m3(float(v)))


def bf16_round(f):
    return int(_host.synth_host_bf16(float(f)))


# -------------------------------------------------------------- device fills
def _s(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream


def dev_fp8_rows(seed, tensor, layer, R, D, permyriad, b0, nb, r0, nr, codes, scales,
                 stream=None):
    assert codes.numel() == nb * nr * D and scales.numel() == nb * nr
    _ok(_devlib().synth_dev_fp8_rows(seed, tensor, layer, R, D, permyriad, b0, nb, r0, nr,
                                     codes.data_ptr(), scales.data_ptr(), _s(stream)),
        "device fp8 fill")


def dev_bf16_rows(seed, tensor, layer, D, b0, nb, r0, nr, out, stream=None):
    assert out.numel() == nb * nr * D
    _ok(_devlib().synth_dev_bf16_rows(seed, tensor, layer, D, b0, nb, r0, nr, out.data_ptr(),
                                      _s(stream)), "device bf16 fill")


def dev_uniform_rows(seed, tensor, layer, D, b0, nb, r0, nr, out, stream=None):
    assert out.numel() == nb * nr * D
    _ok(_devlib().synth_dev_uniform_rows(seed, tensor, layer, D, b0, nb, r0, nr, out.data_ptr(),
                                         _s(stream)), "device uniform fill")
