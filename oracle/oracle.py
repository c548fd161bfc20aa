"""ctypes binding of the CPU oracle (TEST INFRASTRUCTURE ONLY).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this module. It takes and returns numpy arrays; W and X are passed as fp32
arrays holding the exact values of the stored inputs.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# AWQ_ORACLE_LIB points at another build of this same source; the mutation test
# uses it to load copies with a planted mistake and check that the pins fail.
LIB_PATH = os.environ.get("AWQ_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")

SYM, ASYM = 0, 1
_MODES = {"sym": SYM, "asym": ASYM, SYM: SYM, ASYM: ASYM}

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _build  # noqa: F401  (package-relative when imported as oracle.oracle)
        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
    f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
    i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
    u32p = np.ctypeslib.ndpointer(np.uint32, flags="C_CONTIGUOUS")
    u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
    i64, cint = ctypes.c_int64, ctypes.c_int
    lib.awq_ref_act_stats.argtypes = [f32p, i64, i64, f32p]
    lib.awq_ref_act_stats.restype = None
    lib.awq_ref_s_table.argtypes = [f32p, i64, cint, f32p]
    lib.awq_ref_s_table.restype = cint
    lib.awq_ref_quant_group.argtypes = [f32p, i64, cint, cint, i32p, ctypes.POINTER(ctypes.c_float),
                                        ctypes.POINTER(ctypes.c_int32), f32p]
    lib.awq_ref_quant_group.restype = cint
    lib.awq_ref_fake_quant.argtypes = [f32p, i64, i64, f32p, cint, cint, cint, f64p]
    lib.awq_ref_fake_quant.restype = cint
    lib.awq_ref_output_mse.argtypes = [f32p, f64p, f32p, i64, i64, i64, cint]
    lib.awq_ref_output_mse.restype = ctypes.c_double
    lib.awq_ref_search.argtypes = [f32p, f32p, i64, i64, i64, f32p, cint, cint, cint, cint,
                                   f64p, ctypes.POINTER(ctypes.c_int32), f32p, cint]
    lib.awq_ref_search.restype = cint
    lib.awq_ref_quantize_pack.argtypes = [f32p, i64, i64, f32p, cint, cint, cint, u32p, f32p, u8p]
    lib.awq_ref_quantize_pack.restype = cint
    lib.awq_ref_clip_ratio.argtypes = [cint, cint, ctypes.c_float]
    lib.awq_ref_clip_ratio.restype = ctypes.c_float
    lib.awq_ref_quant_group_clip.argtypes = [f32p, i64, cint, cint, ctypes.c_float, i32p,
                                             ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int32),
                                             f32p]
    lib.awq_ref_quant_group_clip.restype = cint
    lib.awq_ref_clip_search.argtypes = [f32p, f32p, i64, i64, i64, f32p, cint, cint, cint, cint,
                                        ctypes.c_float, f32p, f64p, cint]
    lib.awq_ref_clip_search.restype = cint
    lib.awq_ref_quantize_pack_clip.argtypes = [f32p, i64, i64, f32p, ctypes.c_void_p, cint, cint, cint,
                                               u32p, f32p, u8p]
    lib.awq_ref_quantize_pack_clip.restype = cint
    lib.awq_ref_f32_to_f16.argtypes = [ctypes.c_float]
    lib.awq_ref_f32_to_f16.restype = ctypes.c_uint16
    lib.awq_ref_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.awq_ref_f32_to_bf16.restype = ctypes.c_uint16
    lib.awq_ref_fold_rows.argtypes = [f32p, i64, i64, f32p, cint, ctypes.c_void_p]
    lib.awq_ref_fold_rows.restype = cint
    lib.awq_ref_scale_cols.argtypes = [f32p, i64, i64, f32p, cint, ctypes.c_void_p]
    lib.awq_ref_scale_cols.restype = cint
    lib.awq_ref_qgemm.argtypes = [f32p, i64, i64, u32p, f32p, u8p, i64, cint, cint, f64p]
    lib.awq_ref_qgemm.restype = cint
    lib.awq_ref_unpack_code.argtypes = [u32p, i64, cint]
    lib.awq_ref_unpack_code.restype = ctypes.c_uint32
    _lib = lib
    return lib


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def act_stats(X):
    X = _f32(X)
    T, n_in = X.shape
    xmag = np.empty(n_in, np.float32)
    _load().awq_ref_act_stats(X, T, n_in, xmag)
    return xmag


def s_table(xmag, grid):
    xmag = _f32(xmag)
    out = np.empty((grid + 1, xmag.shape[0]), np.float32)
    st = _load().awq_ref_s_table(xmag, xmag.shape[0], grid, out)
    if st != 0:
        raise ValueError(f"awq_ref_s_table status {st}")
    return out


def quant_group(v, bits, mode):
    """Returns (codes int32[g], scale float, zero int, dequantized float32[g])."""
    v = _f32(v)
    g = v.shape[0]
    code = np.empty(g, np.int32)
    what = np.empty(g, np.float32)
    scale = ctypes.c_float()
    zero = ctypes.c_int32()
    st = _load().awq_ref_quant_group(v, g, bits, _MODES[mode], code, ctypes.byref(scale),
                                     ctypes.byref(zero), what)
    if st != 0:
        raise ValueError(f"awq_ref_quant_group status {st}")
    return code, np.float32(scale.value), int(zero.value), what


def fake_quant(W, s, bits, group, mode):
    W = _f32(W)
    out, n_in = W.shape
    wq = np.empty((out, n_in), np.float64)
    st = _load().awq_ref_fake_quant(W, out, n_in, _f32(s), bits, group, _MODES[mode], wq)
    if st != 0:
        raise ValueError(f"awq_ref_fake_quant status {st}")
    return wq


def output_mse(W, wq, X, nthreads=0):
    W, X = _f32(W), _f32(X)
    wq = np.ascontiguousarray(wq, dtype=np.float64)
    out, n_in = W.shape
    return float(_load().awq_ref_output_mse(W, wq, X, out, n_in, X.shape[0], nthreads))


def search(W, X, xmag, bits, group, grid, mode, nthreads=0):
    """Returns (mse float64[grid+1], best int, s_best float32[in], status)."""
    W, X, xmag = _f32(W), _f32(X), _f32(xmag)
    out, n_in = W.shape
    mse = np.empty(grid + 1, np.float64)
    s_best = np.empty(n_in, np.float32)
    best = ctypes.c_int32()
    st = _load().awq_ref_search(W, X, out, n_in, X.shape[0], xmag, bits, group, grid,
                                _MODES[mode], mse, ctypes.byref(best), s_best, nthreads)
    if st not in (0, -4):
        raise ValueError(f"awq_ref_search status {st}")
    return mse, int(best.value), s_best, st


def words_per_row(n_in, bits):
    return (n_in * bits + 31) // 32


def quantize_pack(W, s, bits, group, mode):
    """Returns (qweight uint32[out][words], scales float32[out][in/group], zeros uint8[...])."""
    W = _f32(W)
    out, n_in = W.shape
    q = np.empty((out, words_per_row(n_in, bits)), np.uint32)
    sc = np.empty((out, n_in // group), np.float32)
    z = np.empty((out, n_in // group), np.uint8)
    st = _load().awq_ref_quantize_pack(W, out, n_in, _f32(s), bits, group, _MODES[mode], q, sc, z)
    if st != 0:
        raise ValueError(f"awq_ref_quantize_pack status {st}")
    return q, sc, z


def clip_ratio(i, n_clip, max_shrink):
    return np.float32(_load().awq_ref_clip_ratio(i, n_clip, max_shrink))


def quant_group_clip(v, bits, mode, ratio):
    """quant_group with the clipping range scaled by `ratio`."""
    v = _f32(v)
    g = v.shape[0]
    code = np.empty(g, np.int32)
    what = np.empty(g, np.float32)
    scale = ctypes.c_float()
    zero = ctypes.c_int32()
    st = _load().awq_ref_quant_group_clip(v, g, bits, _MODES[mode], float(ratio), code,
                                          ctypes.byref(scale), ctypes.byref(zero), what)
    if st != 0:
        raise ValueError(f"awq_ref_quant_group_clip status {st}")
    return code, np.float32(scale.value), int(zero.value), what


def clip_search(W, X, s, bits, group, mode, n_clip=20, max_shrink=0.5, nthreads=0):
    """Returns (clip float32[out][in/group], sse float64[out][in/group][n_clip])."""
    W, X = _f32(W), _f32(X)
    out, n_in = W.shape
    clip = np.empty((out, n_in // group), np.float32)
    sse = np.empty((out, n_in // group, n_clip), np.float64)
    st = _load().awq_ref_clip_search(W, X, out, n_in, X.shape[0], _f32(s), bits, group, _MODES[mode],
                                     n_clip, max_shrink, clip, sse, nthreads)
    if st != 0:
        raise ValueError(f"awq_ref_clip_search status {st}")
    return clip, sse


def quantize_pack_clip(W, s, clip, bits, group, mode):
    """quantize_pack with a clipping ratio per (row, group)."""
    W = _f32(W)
    out, n_in = W.shape
    q = np.empty((out, words_per_row(n_in, bits)), np.uint32)
    sc = np.empty((out, n_in // group), np.float32)
    z = np.empty((out, n_in // group), np.uint8)
    clip = _f32(clip)
    st = _load().awq_ref_quantize_pack_clip(W, out, n_in, _f32(s), clip.ctypes.data_as(ctypes.c_void_p),
                                            bits, group, _MODES[mode], q, sc, z)
    if st != 0:
        raise ValueError(f"awq_ref_quantize_pack_clip status {st}")
    return q, sc, z


_STORE = {"f32": 0, "f16": 1, "bf16": 2}


def f32_to_f16_bits(x):
    """One fp32 value -> binary16 bit pattern (round half to even)."""
    return int(_load().awq_ref_f32_to_f16(float(np.float32(x))))


def f32_to_bf16_bits(x):
    """One fp32 value -> bfloat16 bit pattern (round half to even)."""
    return int(_load().awq_ref_f32_to_bf16(float(np.float32(x))))


def _folded(fn, A, s, storage):
    A = _f32(np.atleast_2d(A) if np.ndim(A) != 1 else A[:, None])
    rows, cols = A.shape
    out = np.empty((rows, cols), np.float32 if storage == "f32" else np.uint16)
    st = fn(A, rows, cols, _f32(s), _STORE[storage], out.ctypes.data_as(ctypes.c_void_p))
    if st != 0:
        raise ValueError(f"fold status {st}")
    return out


def fold_rows(A, s, storage="f32"):
    """store(A[r][c] / s[r]); A (rows, cols) or a vector (rows,) -> (rows, 1).
    Returns fp32 values or 16-bit patterns (uint16) for f16 / bf16 storage."""
    return _folded(_load().awq_ref_fold_rows, A, s, storage)


def scale_cols(W, s, storage="f32"):
    """store(W[o][j] * s[j])."""
    return _folded(_load().awq_ref_scale_cols, W, s, storage)


def qgemm(X, qweight, scales, zeros, bits, group):
    """Y (M, out) fp64 = X Wd^T with Wd = scale * (code - zero) from the packed layout."""
    X = _f32(np.atleast_2d(X))
    M, n_in = X.shape
    q = np.ascontiguousarray(qweight).view(np.uint32)
    out = q.shape[0]
    Y = np.empty((M, out), np.float64)
    st = _load().awq_ref_qgemm(X, M, n_in, np.ascontiguousarray(q), _f32(scales),
                               np.ascontiguousarray(zeros, dtype=np.uint8), out, bits, group, Y)
    if st != 0:
        raise ValueError(f"awq_ref_qgemm status {st}")
    return Y


def unpack_code(row_words, k, bits):
    return int(_load().awq_ref_unpack_code(np.ascontiguousarray(row_words, dtype=np.uint32), k, bits))
