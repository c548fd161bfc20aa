"""CPU oracle for GPTQ as a second workload on the same layer inputs.

TEST INFRASTRUCTURE ONLY: the plain, slow statement of what the GPU GPTQ path
computes. Only the test suite, the smoke check and the benchmark's CPU
baseline may use it; it shares no code with the HIP library.

Sources: "AWQ vs GPTQ Quantization Architectures Compared", section "GPTQ:
compensate the error you just made" (the error-compensation idea, the damped
Hessian and the group quantizer), and "Advanced Quantization Algorithms: AWQ
and GPTQ Explained", section 3 (the Optimal Brain Surgeon step and the
inverse-Hessian update after each weight is fixed).

The method, as this module states it. Each output row is quantised on its
own, weight by weight in column order, against the quadratic form of the
layer's inputs, H = 2 X^T X (X as (tokens, in)) plus damp * mean(diag H) on
the diagonal. Once weight i of a row is fixed at its quantised value, the
remaining free weights F = {i+1, ...} move to minimise (w' - w)^T H (w' - w)
given the fixed ones. Optimal Brain Surgeon gives that move in terms of the
inverse Hessian of the weights still free before the step, G = (H_FF)^-1
over F = {i, i+1, ...}:

    w_j  <-  w_j - (w_i - q_i) * G[i, j] / G[i, i]      for j > i,

and the inverse Hessian of the next free set follows by eliminating index i
from G (a rank-one update). Writing the rows of these successive inverses as
V[i, j] = G_i[i, j] / sqrt(G_i[i, i]) (j >= i) turns the move into
w_j -= ((w_i - q_i) / V[i, i]) * V[i, j]; V is upper triangular with
V^T V = H^-1, which is how the GPU path factors it. The group parameters of
a group are fitted when its first column is reached, on the weights as the
earlier steps have moved them.

Readings (the pages leave these open):
  - the quantizer is the one the packed format stores: asymmetric (range
    widened to contain 0, maxq = 2^b - 1, zero = rne(-lo / scale)) or
    symmetric (L = 2^(b-1) - 1, codes q + 2^(b-1)); the range and the scale
    are computed in fp64 and the scale is rounded once to fp32, the precision
    it is stored in, and that fp32 scale is the one used for the rounding and
    the error (so the stored codes, scales and zeros reproduce exactly the
    weights GPTQ compensated for); divisions in fp64, ties to even;
  - the per-weight step evaluates (w_i - q_i) / V[i, i] once and multiplies
    it by V[i, j], the same two roundings the GPU's column loop makes;
  - act-order (desc_act) is not part of this path: group membership would
    then follow the permuted order and the packed format has no g_idx.
numpy's matrix product and inverse serve as library steps.
"""
import numpy as np


def hessian(X):
    """H = 2 X^T X (fp64), X (tokens, in) given as exact fp32 values."""
    X = np.asarray(X, np.float64)
    return 2.0 * (X.T @ X)


def dampen(H, damp=0.01):
    """H + damp * mean(diag H) * I."""
    mean_diag = float(np.trace(H)) / H.shape[0]
    return H + np.diag(np.full(H.shape[0], damp * mean_diag))


def obs_factor(H):
    """V (in, in), upper triangular: row i is the row of weight i in the
    inverse Hessian of the weights still free when weight i is fixed,
    divided by the square root of its diagonal element. Computed by fixing
    the weights one at a time and eliminating each from the inverse."""
    n = H.shape[0]
    G = np.linalg.inv(np.asarray(H, np.float64))
    V = np.zeros((n, n))
    for i in range(n):
        pivot = G[i, i]
        V[i, i:] = G[i, i:] / np.sqrt(pivot)
        # weight i leaves the free set: Schur complement of its pivot
        G[i + 1:, i + 1:] -= np.outer(G[i + 1:, i], G[i, i + 1:]) / pivot
    return V


def group_params(Wg, bits, mode):
    """Scale (an fp32 value, held in fp64) and zero of each row of a group's weights."""
    Wg = np.asarray(Wg, np.float64)
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


def round_weight(w, scale, zero, bits, mode):
    """The stored code of one weight and the value it stands for."""
    if mode == "asym":
        code = min(max(np.round(w / scale) + zero, 0.0), float((1 << bits) - 1))
        return code, scale * (code - zero)
    L = (1 << (bits - 1)) - 1
    level = min(max(np.round(w / scale), float(-L - 1)), float(L))
    return level + (1 << (bits - 1)), scale * level


def gptq(W, X=None, bits=4, group=128, mode="asym", damp=0.01, U=None, corrected=False):
    """Returns (codes int64 (out, in), scales float32 (out, in/group),
    zeros uint8 (out, in/group), Wq fp64 (out, in) the dequantized weights)
    and, with corrected=True, the value each weight had when it was fixed.
    U, the factor obs_factor() returns, may be passed (it depends on X only)."""
    W0 = np.array(W, np.float64)
    out, n_in = W0.shape
    if n_in % group:
        raise ValueError("in must be a multiple of group")
    V = obs_factor(dampen(hessian(X), damp)) if U is None else np.asarray(U, np.float64)
    codes = np.zeros((out, n_in), np.int64)
    Wq = np.zeros((out, n_in))
    Wfix = np.zeros((out, n_in))
    scales = np.zeros((out, n_in // group), np.float32)
    zeros = np.zeros((out, n_in // group), np.uint8)
    for r in range(out):
        w = W0[r].copy()                       # the row's weights as the steps move them
        for g in range(n_in // group):
            cols = range(g * group, (g + 1) * group)
            sc, zr = group_params(w[None, cols.start:cols.stop], bits, mode)
            scale, zero = float(sc[0]), float(zr[0])
            scales[r, g], zeros[r, g] = scale, zero
            for i in cols:
                code, value = round_weight(w[i], scale, zero, bits, mode)
                codes[r, i], Wq[r, i], Wfix[r, i] = code, value, w[i]
                step = (w[i] - value) / V[i, i]
                w[i + 1:] = w[i + 1:] - step * V[i, i + 1:]
    if corrected:
        return codes, scales, zeros, Wq, Wfix
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
