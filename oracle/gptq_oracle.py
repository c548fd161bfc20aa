"""CPU oracle for GPTQ as a second workload on the same layer inputs.

TEST INFRASTRUCTURE ONLY: the plain, slow statement of what the GPU GPTQ path
computes. Only the test suite, the smoke check and the benchmark's CPU
baseline may use it; it shares no code with the HIP library.

Source: "AWQ vs GPTQ Quantization Architectures Compared", section "GPTQ:
compensate the error you just made" (the gptq_layer, group_params and rtn
listing and the three production details after it), and "Advanced
Quantization Algorithms: AWQ and GPTQ Explained", section 3 (the inverse
Hessian update). In words, for W (out, in) and calibration inputs X:

  1. H = 2 X^T X over the tokens (the pages write 2 X X^T with X as
     (in, tokens)), in fp64;
  2. dampening: add damp * mean(diag H) to the diagonal (damp = 0.01);
  3. U = the upper Cholesky factor of H^-1 (transpose of the lower factor);
  4. columns in order i = 0 .. in-1, all rows at once: at the start of each
     group fit the group parameters on the current (already corrected)
     weights of the group's columns; round column i with them; divide its
     rounding error by U[i, i] and subtract that times row i of U from the
     later columns.

Readings (the pages leave these open):
  - the quantizer is the one the packed format stores: asymmetric (the
    listing's group_params / rtn: range widened to contain 0, maxq = 2^b - 1,
    zero = rne(-lo / scale)) or symmetric (L = 2^(b-1) - 1, codes q + 2^(b-1));
    the range and the scale are computed in fp64 and the scale is rounded
    once to fp32, the precision it is stored in, and that fp32 scale is the
    one used for the rounding and the error (so the stored codes, scales and
    zeros reproduce exactly the weights GPTQ compensated for); divisions in
    fp64, ties to even (numpy's round);
  - act-order (desc_act) is not part of this path: group membership would
    then follow the permuted order and the packed format has no g_idx.
Steps 1-3 use numpy's matrix product, inverse and Cholesky as library steps.
"""
import numpy as np


def hessian(X):
    """H = 2 X^T X (fp64), X (tokens, in) given as exact fp32 values."""
    X = np.asarray(X, np.float64)
    return 2.0 * (X.T @ X)


def dampen(H, damp=0.01):
    H = H.copy()
    H[np.diag_indices_from(H)] += damp * np.mean(np.diag(H))
    return H


def inverse_cholesky_upper(H):
    """U with H^-1 = U^T U, U upper: the Cholesky factor of the inverse, transposed."""
    return np.linalg.cholesky(np.linalg.inv(H)).T


def group_params(Wg, bits, mode):
    """Scale (fp32 value) and zero for each row of the group's current weights."""
    if mode == "asym":
        maxq = (1 << bits) - 1
        lo = np.minimum(Wg.min(axis=1), 0.0)
        hi = np.maximum(Wg.max(axis=1), 0.0)
        scale = np.maximum((hi - lo) / maxq, 1e-8).astype(np.float32).astype(np.float64)
        zero = np.round(-lo / scale)
        return scale, zero
    L = (1 << (bits - 1)) - 1
    a = np.abs(Wg).max(axis=1)
    scale = np.maximum(a / L, 1e-8).astype(np.float32).astype(np.float64)
    return scale, np.full_like(scale, float(1 << (bits - 1)))


def quantize_column(w, scale, zero, bits, mode):
    """Codes (stored form) and the dequantized values of one column."""
    if mode == "asym":
        maxq = (1 << bits) - 1
        q = np.clip(np.round(w / scale) + zero, 0, maxq)
        return q, scale * (q - zero)
    L = (1 << (bits - 1)) - 1
    q = np.clip(np.round(w / scale), -L - 1, L)
    return q + (1 << (bits - 1)), scale * q


def gptq(W, X=None, bits=4, group=128, mode="asym", damp=0.01, U=None, corrected=False):
    """Returns (codes int64 (out, in), scales float32 (out, in/group),
    zeros uint8 (out, in/group), Wq fp64 (out, in) the dequantized weights)
    and, with corrected=True, the weights each column had when it was rounded.
    U may be passed (computed once for all rows); rows are independent given U."""
    W = np.array(W, np.float64)
    out, n_in = W.shape
    if n_in % group:
        raise ValueError("in must be a multiple of group")
    if U is None:
        U = inverse_cholesky_upper(dampen(hessian(X), damp))
    codes = np.zeros((out, n_in), np.int64)
    Wq = np.zeros((out, n_in))
    scales = np.zeros((out, n_in // group), np.float32)
    zeros = np.zeros((out, n_in // group), np.uint8)
    for i in range(n_in):
        if i % group == 0:
            scale, zero = group_params(W[:, i:i + group], bits, mode)
            scales[:, i // group] = scale
            zeros[:, i // group] = zero
        q, wq = quantize_column(W[:, i], scale, zero, bits, mode)
        codes[:, i] = q
        Wq[:, i] = wq
        err = (W[:, i] - wq) / U[i, i]
        W[:, i + 1:] -= np.outer(err, U[i, i + 1:])
    if corrected:
        return codes, scales, zeros, Wq, W       # column i is no longer changed after step i
    return codes, scales, zeros, Wq


def pack(codes, bits):
    """The packed layout of the GPU library and the AWQ oracle: code i of a row
    at bits [i*bits, (i+1)*bits) of the row's little-endian 32-bit words."""
    out, n_in = codes.shape
    words = (n_in * bits + 31) // 32
    q = np.zeros((out, words), np.uint64)
    for i in range(n_in):
        w, sh = divmod(i * bits, 32)
        c = codes[:, i].astype(np.uint64)
        q[:, w] |= (c << np.uint64(sh)) & np.uint64(0xFFFFFFFF)
        if sh + bits > 32:
            q[:, w + 1] |= c >> np.uint64(32 - sh)
    return q.astype(np.uint32)


def output_sse(W, Wq, X):
    """sum over tokens and rows of (X Wq^T - X W^T)^2, fp64."""
    X = np.asarray(X, np.float64)
    D = np.asarray(Wq, np.float64) - np.asarray(W, np.float64)
    E = X @ D.T
    return float((E * E).sum())
