"""Thin Python binding of libawq.so (include/awq.h) over torch device tensors.

Argument marshalling only: every step runs in the library's HIP kernels on
the caller's current torch stream. There is no CPU fallback: if the library
is not built, or a tensor is not on the GPU, these functions raise.
"""
import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libawq.so")

F32, F16, BF16 = 0, 1, 2
SYM, ASYM = 0, 1
OK, ERR_INVALID_ARG, ERR_WORKSPACE, ERR_HIP, ERR_NONFINITE, ERR_UNSUPPORTED = 0, -1, -2, -3, -4, -5
MAX_GRID = 1024
SEARCH_NOALLOC_MAX_BYTES = 24 << 20   # static per-GPU scratch of awq_search_noalloc
MAX_CLIP = 64

_DTYPE = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
_MODE = {"sym": SYM, "asym": ASYM, SYM: SYM, ASYM: ASYM}
_SEARCH_GROUPS = (32, 64, 128)
_PACK_GROUPS = (32, 64, 128, 256, 512, 1024, 2048)

_lib = None


class AwqError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                               "or python post_weight_quantization_30_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, cint, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        L.awq_act_stats.argtypes = [vp, cint, i64, i64, vp, vp, sz, vp]
        L.awq_act_stats.restype = cint
        L.awq_act_stats_workspace_size.argtypes = [i64, i64]
        L.awq_act_stats_workspace_size.restype = sz
        L.awq_s_table.argtypes = [vp, i64, cint, vp, vp]
        L.awq_s_table.restype = cint
        L.awq_search.argtypes = [vp, vp, cint, i64, i64, i64, vp, cint, cint, cint, cint,
                                 vp, vp, vp, vp, sz, vp]
        L.awq_search.restype = cint
        L.awq_search_noalloc.argtypes = [vp, vp, cint, i64, i64, i64, vp, cint, cint, cint, cint,
                                         vp, vp, vp, vp]
        L.awq_search_noalloc.restype = cint
        L.awq_search_prepare.argtypes = [vp, cint, vp, i64, i64, i64, cint, vp, sz, vp]
        L.awq_search_prepare.restype = cint
        L.awq_search_candidates.argtypes = [vp, vp, cint, i64, i64, i64, cint, cint, cint, cint,
                                            vp, sz, vp]
        L.awq_search_candidates.restype = cint
        L.awq_search_finish.argtypes = [i64, i64, i64, cint, vp, vp, vp, vp, sz, vp]
        L.awq_search_finish.restype = cint
        L.awq_search_workspace_size.argtypes = [i64, i64, i64, cint]
        L.awq_search_workspace_size.restype = sz
        L.awq_quantize_pack.argtypes = [vp, cint, i64, i64, vp, cint, cint, cint, vp, vp, vp, vp]
        L.awq_quantize_pack.restype = cint
        L.awq_clip_search.argtypes = [vp, vp, cint, i64, i64, i64, vp, cint, cint, cint, cint,
                                      ctypes.c_float, vp, vp, vp]
        L.awq_clip_search.restype = cint
        L.awq_quantize_pack_clip.argtypes = [vp, cint, i64, i64, vp, vp, cint, cint, cint, vp, vp,
                                             vp, vp]
        L.awq_quantize_pack_clip.restype = cint
        L.awq_fold_rows.argtypes = [vp, cint, i64, i64, vp, vp, vp]
        L.awq_fold_rows.restype = cint
        L.awq_scale_cols.argtypes = [vp, cint, i64, i64, vp, vp, vp]
        L.awq_scale_cols.restype = cint
        L.awq_qgemm.argtypes = [vp, cint, i64, i64, vp, vp, vp, i64, cint, cint, vp, cint, vp]
        L.awq_qgemm.restype = cint
        dbl = ctypes.c_double
        L.awq_gptq_hessian.argtypes = [vp, cint, i64, i64, dbl, vp, vp]
        L.awq_gptq_hessian.restype = cint
        L.awq_gptq_factor.argtypes = [vp, i64, vp, vp, sz, vp]
        L.awq_gptq_factor.restype = cint
        L.awq_gptq_quantize.argtypes = [vp, cint, i64, i64, vp, cint, cint, cint, vp, vp, vp, vp, sz, vp]
        L.awq_gptq_quantize.restype = cint
        L.awq_gptq.argtypes = [vp, vp, cint, i64, i64, i64, cint, cint, cint, dbl, vp, vp, vp, vp, sz, vp]
        L.awq_gptq.restype = cint
        for fn in ("awq_gptq_factor_workspace_size",):
            getattr(L, fn).argtypes = [i64]
            getattr(L, fn).restype = sz
        for fn in ("awq_gptq_quantize_workspace_size", "awq_gptq_workspace_size"):
            getattr(L, fn).argtypes = [i64, i64]
            getattr(L, fn).restype = sz
        L.awq_status_string.argtypes = [cint]
        L.awq_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status):
    return lib().awq_status_string(int(status)).decode()


def _check(fn, status):
    if status != OK:
        raise AwqError(fn, status)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, name, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _need(t, name, shape):
    """A caller-supplied tensor must have exactly this shape (checked before any
    launch: an undersized output would be written past its end)."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _dtype_code(t):
    if t.dtype not in _DTYPE:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DTYPE[t.dtype]


def words_per_row(n_in, bits):
    return (n_in * bits + 31) // 32


def act_stats_workspace_size(tokens, n_in):
    return int(lib().awq_act_stats_workspace_size(tokens, n_in))


def search_workspace_size(out, n_in, tokens, grid):
    return int(lib().awq_search_workspace_size(out, n_in, tokens, grid))


def _workspace(nbytes, device, ws):
    if ws is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError("workspace too small")
    return ws


def act_stats(X, xmag=None, workspace=None):
    """xmag[j] = mean_t |X[t, j]| + 1e-8 (fp32)."""
    T, n_in = X.shape
    if xmag is None:
        xmag = torch.empty(n_in, dtype=torch.float32, device=X.device)
    _need(xmag, "xmag", (n_in,))
    ws = _workspace(act_stats_workspace_size(T, n_in), X.device, workspace)
    _check("awq_act_stats", lib().awq_act_stats(
        _dev(X, "X"), _dtype_code(X), T, n_in, _dev(xmag, "xmag", torch.float32),
        _dev(ws, "workspace"), ws.numel() * ws.element_size(), _stream()))
    return xmag


def s_table(xmag, grid, out=None):
    n_in = xmag.shape[0]
    if out is None:
        out = torch.empty((grid + 1, n_in), dtype=torch.float32, device=xmag.device)
    _need(out, "s_table", (grid + 1, n_in))
    _check("awq_s_table", lib().awq_s_table(_dev(xmag, "xmag", torch.float32), n_in, grid,
                                            _dev(out, "s_table", torch.float32), _stream()))
    return out


def _check_search_io(n_in, grid, xmag, mse, best, s_best):
    _need(xmag, "xmag", (n_in,))
    _need(mse, "mse", (grid + 1,))
    _need(best, "best", (1,))
    _need(s_best, "s_best", (n_in,))


def search(W, X, xmag, bits, group, grid, mode, mse=None, best=None, s_best=None, workspace=None):
    """Returns device tensors (mse fp64[grid+1], best int32[1], s_best fp32[in])."""
    out, n_in = W.shape
    T = X.shape[0]
    if X.shape[1] != n_in or X.dtype != W.dtype:
        raise ValueError("W (out, in) and X (tokens, in) must share in and dtype")
    dev = W.device
    mse = torch.empty(grid + 1, dtype=torch.float64, device=dev) if mse is None else mse
    best = torch.empty(1, dtype=torch.int32, device=dev) if best is None else best
    s_best = torch.empty(n_in, dtype=torch.float32, device=dev) if s_best is None else s_best
    _check_search_io(n_in, grid, xmag, mse, best, s_best)
    ws = _workspace(search_workspace_size(out, n_in, T, grid), dev, workspace)
    _check("awq_search", lib().awq_search(
        _dev(W, "W"), _dev(X, "X"), _dtype_code(W), out, n_in, T, _dev(xmag, "xmag", torch.float32),
        bits, group, grid, _MODE[mode], _dev(mse, "mse", torch.float64),
        _dev(best, "best", torch.int32), _dev(s_best, "s_best", torch.float32),
        _dev(ws, "workspace"), ws.numel() * ws.element_size(), _stream()))
    return mse, best, s_best


def search_noalloc(W, X, xmag, bits, group, grid, mode, mse, best, s_best):
    """awq_search on the library's static per-GPU scratch: the C call allocates
    nothing. The outputs (mse fp64[grid+1], best int32[1], s_best fp32[in])
    are the caller's. Calls that overlap on one GPU race on the scratch."""
    out, n_in = W.shape
    T = X.shape[0]
    if X.shape[1] != n_in or X.dtype != W.dtype:
        raise ValueError("W (out, in) and X (tokens, in) must share in and dtype")
    _check_search_io(n_in, grid, xmag, mse, best, s_best)
    _check("awq_search_noalloc", lib().awq_search_noalloc(
        _dev(W, "W"), _dev(X, "X"), _dtype_code(W), out, n_in, T, _dev(xmag, "xmag", torch.float32),
        bits, group, grid, _MODE[mode], _dev(mse, "mse", torch.float64),
        _dev(best, "best", torch.int32), _dev(s_best, "s_best", torch.float32), _stream()))
    return mse, best, s_best


def search_prepare(X, xmag, out, grid, workspace):
    """The s-table (and, for the 16-bit search, X in fragment order) into the workspace."""
    T, n_in = X.shape
    _need(xmag, "xmag", (n_in,))
    _check("awq_search_prepare", lib().awq_search_prepare(
        _dev(X, "X"), _dtype_code(X), _dev(xmag, "xmag", torch.float32), out, n_in, T, grid,
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream()))


def search_candidates(W, X, bits, group, grid, mode, workspace):
    out, n_in = W.shape
    _check("awq_search_candidates", lib().awq_search_candidates(
        _dev(W, "W"), _dev(X, "X"), _dtype_code(W), out, n_in, X.shape[0], bits, group, grid,
        _MODE[mode], _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream()))


def search_finish(out, n_in, tokens, grid, mse, best, s_best, workspace):
    _need(mse, "mse", (grid + 1,))
    _need(best, "best", (1,))
    _need(s_best, "s_best", (n_in,))
    _check("awq_search_finish", lib().awq_search_finish(
        out, n_in, tokens, grid, _dev(mse, "mse", torch.float64), _dev(best, "best", torch.int32),
        _dev(s_best, "s_best", torch.float32), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream()))


def clip_search(W, X, s, bits, group, mode, n_clip=20, max_shrink=0.5, clip=None, sse=None,
                want_sse=False):
    """Clipping-range search on W diag(s). Returns (clip fp32 [out][in/group],
    sse fp64 [out][in/group][n_clip] or None)."""
    out, n_in = W.shape
    T = X.shape[0]
    if X.shape[1] != n_in or X.dtype != W.dtype:
        raise ValueError("W (out, in) and X (tokens, in) must share in and dtype")
    dev = W.device
    if clip is None:
        clip = torch.empty((out, n_in // group), dtype=torch.float32, device=dev)
    if sse is None and want_sse:
        sse = torch.empty((out, n_in // group, n_clip), dtype=torch.float64, device=dev)
    _need(s, "s", (n_in,))
    _need(clip, "clip", (out, n_in // group))
    if sse is not None:
        _need(sse, "sse", (out, n_in // group, n_clip))
    _check("awq_clip_search", lib().awq_clip_search(
        _dev(W, "W"), _dev(X, "X"), _dtype_code(W), out, n_in, T, _dev(s, "s", torch.float32),
        bits, group, _MODE[mode], n_clip, float(max_shrink), _dev(clip, "clip", torch.float32),
        None if sse is None else _dev(sse, "sse", torch.float64), _stream()))
    return clip, sse


def quantize_pack(W, s, bits, group, mode, qweight=None, scales=None, zeros=None, clip=None):
    """Returns device tensors (qweight int32 view of uint32 words [out][words],
    scales fp32 [out][in/group], zeros uint8 [out][in/group]). With `clip`
    (fp32 [out][in/group] ratios) each group's range is clipped first."""
    out, n_in = W.shape
    dev = W.device
    if qweight is None:
        qweight = torch.empty((out, words_per_row(n_in, bits)), dtype=torch.int32, device=dev)
    if scales is None:
        scales = torch.empty((out, n_in // group), dtype=torch.float32, device=dev)
    if zeros is None:
        zeros = torch.empty((out, n_in // group), dtype=torch.uint8, device=dev)
    _need(s, "s", (n_in,))
    _need(qweight, "qweight", (out, words_per_row(n_in, bits)))
    _need(scales, "scales", (out, n_in // group))
    _need(zeros, "zeros", (out, n_in // group))
    if clip is not None:
        _need(clip, "clip", (out, n_in // group))
    if clip is None:
        _check("awq_quantize_pack", lib().awq_quantize_pack(
            _dev(W, "W"), _dtype_code(W), out, n_in, _dev(s, "s", torch.float32), bits, group,
            _MODE[mode], _dev(qweight, "qweight"), _dev(scales, "scales", torch.float32),
            _dev(zeros, "zeros", torch.uint8), _stream()))
    else:
        _check("awq_quantize_pack_clip", lib().awq_quantize_pack_clip(
            _dev(W, "W"), _dtype_code(W), out, n_in, _dev(s, "s", torch.float32),
            _dev(clip, "clip", torch.float32), bits, group, _MODE[mode], _dev(qweight, "qweight"),
            _dev(scales, "scales", torch.float32), _dev(zeros, "zeros", torch.uint8), _stream()))
    return qweight, scales, zeros


def _rows_cols(A):
    if A.dim() == 1:
        return A.shape[0], 1
    if A.dim() != 2:
        raise ValueError("expected a vector or a matrix")
    return A.shape[0], A.shape[1]


def fold_rows(A, s, out=None):
    """The producer of a searched layer's input absorbs 1/s: out[r] = A[r] / s[r]
    for a norm weight or bias (vector) or the output rows of the previous
    linear layer (matrix). out=A folds in place."""
    rows, cols = _rows_cols(A)
    if s.numel() != rows:
        raise ValueError(f"the producer has {rows} output channels but s has {s.numel()}: it "
                         "cannot absorb these scales (e.g. v_proj under grouped-query attention)")
    out = torch.empty_like(A) if out is None else out
    if out.shape != A.shape or out.dtype != A.dtype:
        raise ValueError("out must match A")
    _check("awq_fold_rows", lib().awq_fold_rows(
        _dev(A, "A"), _dtype_code(A), rows, cols, _dev(s, "s", torch.float32), _dev(out, "out"),
        _stream()))
    return out


def scale_cols(W, s, out=None):
    """The searched layer's weight scaled: out[o][j] = W[o][j] * s[j]."""
    rows, cols = _rows_cols(W)
    if W.dim() != 2 or s.numel() != cols:
        raise ValueError("W must be (out, in) and s of length in")
    out = torch.empty_like(W) if out is None else out
    if out.shape != W.shape or out.dtype != W.dtype:
        raise ValueError("out must match W")
    _check("awq_scale_cols", lib().awq_scale_cols(
        _dev(W, "W"), _dtype_code(W), rows, cols, _dev(s, "s", torch.float32), _dev(out, "out"),
        _stream()))
    return out


def qgemm(X, qweight, scales, zeros, bits, group, y=None, y_f32=False):
    """Y (M, out) = X Wd^T with Wd = scale * (code - zero) read from the packed
    layout (X: fp16 / bf16 (M, in) with 1/s folded upstream). Y is fp32 when
    y_f32, else X's dtype."""
    M, n_in = X.shape
    out = qweight.shape[0]
    if scales.shape != (out, n_in // group) or zeros.shape != scales.shape:
        raise ValueError("scales / zeros must be (out, in / group)")
    if qweight.shape[1] != words_per_row(n_in, bits):
        raise ValueError("qweight has the wrong number of words per row")
    ydt = torch.float32 if y_f32 else X.dtype
    y = torch.empty((M, out), dtype=ydt, device=X.device) if y is None else y
    _need(y, "y", (M, out))
    _check("awq_qgemm", lib().awq_qgemm(
        _dev(X, "X"), _dtype_code(X), M, n_in, _dev(qweight, "qweight"),
        _dev(scales, "scales", torch.float32), _dev(zeros, "zeros", torch.uint8), out, bits, group,
        _dev(y, "y", ydt), _DTYPE[ydt], _stream()))
    return y


def _packed_outputs(out, n_in, bits, group, dev):
    return (torch.empty((out, words_per_row(n_in, bits)), dtype=torch.int32, device=dev),
            torch.empty((out, n_in // group), dtype=torch.float32, device=dev),
            torch.empty((out, n_in // group), dtype=torch.uint8, device=dev))


def gptq_hessian(X, damp=0.01, H=None):
    """H (in, in) fp64 = 2 X^T X plus damp * mean(diag) on the diagonal."""
    T, n_in = X.shape
    H = torch.empty((n_in, n_in), dtype=torch.float64, device=X.device) if H is None else H
    _need(H, "H", (n_in, n_in))
    _check("awq_gptq_hessian", lib().awq_gptq_hessian(
        _dev(X, "X"), _dtype_code(X), T, n_in, float(damp), _dev(H, "H", torch.float64), _stream()))
    return H


def gptq_factor(H, U=None, workspace=None):
    """U (in, in) fp64, upper, with H^-1 = U^T U."""
    n_in = H.shape[0]
    _need(H, "H", (n_in, n_in))
    U = torch.empty_like(H) if U is None else U
    _need(U, "U", (n_in, n_in))
    ws = _workspace(int(lib().awq_gptq_factor_workspace_size(n_in)), H.device, workspace)
    _check("awq_gptq_factor", lib().awq_gptq_factor(
        _dev(H, "H", torch.float64), n_in, _dev(U, "U", torch.float64), _dev(ws, "workspace"),
        ws.numel() * ws.element_size(), _stream()))
    return U


def gptq_quantize(W, U, bits, group, mode, workspace=None):
    """The column loop on W with U; returns (qweight, scales, zeros)."""
    out, n_in = W.shape
    _need(U, "U", (n_in, n_in))
    q, sc, z = _packed_outputs(out, n_in, bits, group, W.device)
    ws = _workspace(int(lib().awq_gptq_quantize_workspace_size(out, n_in)), W.device, workspace)
    _check("awq_gptq_quantize", lib().awq_gptq_quantize(
        _dev(W, "W"), _dtype_code(W), out, n_in, _dev(U, "U", torch.float64), bits, group, _MODE[mode],
        _dev(q, "qweight"), _dev(sc, "scales", torch.float32), _dev(z, "zeros", torch.uint8),
        _dev(ws, "workspace"), ws.numel() * ws.element_size(), _stream()))
    return q, sc, z


def gptq(W, X, bits=4, group=128, mode="asym", damp=0.01, workspace=None):
    """GPTQ of one layer; returns (qweight, scales, zeros) in the packed layout."""
    out, n_in = W.shape
    if X.shape[1] != n_in or X.dtype != W.dtype:
        raise ValueError("W (out, in) and X (tokens, in) must share in and dtype")
    q, sc, z = _packed_outputs(out, n_in, bits, group, W.device)
    ws = _workspace(int(lib().awq_gptq_workspace_size(out, n_in)), W.device, workspace)
    _check("awq_gptq", lib().awq_gptq(
        _dev(W, "W"), _dev(X, "X"), _dtype_code(W), out, n_in, X.shape[0], bits, group, _MODE[mode],
        float(damp), _dev(q, "qweight"), _dev(sc, "scales", torch.float32), _dev(z, "zeros", torch.uint8),
        _dev(ws, "workspace"), ws.numel() * ws.element_size(), _stream()))
    return q, sc, z


def quantize_layer(W, X, bits=4, group=128, grid=20, mode="sym", n_clip=0, max_shrink=0.5):
    """The whole path for one layer (or one stacked group of layers that share
    X): statistics, search, final quantization and packing; with n_clip > 0 a
    clipping-range search on W diag(s_best) runs before the packing."""
    xmag = act_stats(X)
    mse, best, s_best = search(W, X, xmag, bits, group, grid, mode)
    clip = None
    if n_clip > 0:
        clip, _ = clip_search(W, X, s_best, bits, group, mode, n_clip, max_shrink)
    qweight, scales, zeros = quantize_pack(W, s_best, bits, group, mode, clip=clip)
    return {"xmag": xmag, "mse": mse, "best": best, "s_best": s_best, "clip": clip,
            "qweight": qweight, "scales": scales, "zeros": zeros}


def to_device(arr, dtype_name, device="cuda"):
    """numpy storage array from synth (fp32 / fp16 / bf16 bits) -> device tensor."""
    import numpy as np
    if dtype_name == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16))
        return t.to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)
