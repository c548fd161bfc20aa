"""Pins of the GPTQ oracle (CPU only).

The oracle states GPTQ as Optimal Brain Surgeon steps ("Advanced
Quantization Algorithms: AWQ and GPTQ Explained", section 3; "AWQ vs GPTQ
Quantization Architectures Compared", "GPTQ: compensate the error you just
made"): weights fixed one at a time, the free ones moved by the row of the
current inverse Hessian, that inverse updated by eliminating the fixed
weight. The pins tie it to facts that do not go through that route:
  - the compensation is the exact least-squares correction: after the
    columns before j are fixed at their rounded values, the weights left free
    are the minimisers of ||X (W' - W)||^2 (the Optimal Brain Surgeon step the
    page starts from), computed here with a plain linear solve on H;
  - a hand-worked two-column case, and a hand-worked factor;
  - the factor of the successive inverses is the upper Cholesky factor of
    H^-1 (V^T V = H^-1, V upper), checked against the library's Cholesky;
  - with a diagonal Hessian there is nothing to compensate: the codes are the
    nearest levels of a brute-force search over every code;
  - GPTQ's output error on the calibration data is below RTN's on the
    layer recipes (the purpose of the method, [A] section 3).
"""
import importlib.util
import os

import numpy as np
import pytest

if os.environ.get("AWQ_GPTQ_ORACLE"):          # a copy with a planted mistake (mutation tests)
    _spec = importlib.util.spec_from_file_location("gptq_oracle_copy", os.environ["AWQ_GPTQ_ORACLE"])
    G = importlib.util.module_from_spec(_spec)
    _spec.loader.exec_module(G)
else:
    from oracle import gptq_oracle as G


def _layer(out, n_in, T, seed, outliers=0):
    r = np.random.default_rng(seed)
    W = (r.standard_normal((out, n_in)) * 0.02).astype(np.float32)
    X = r.standard_normal((T, n_in))
    if outliers:
        X[:, r.permutation(n_in)[:outliers]] *= 10.0
    return W, X.astype(np.float32)


@pytest.mark.parametrize("mode,bits,group", [("asym", 4, 8), ("sym", 3, 16), ("asym", 2, 4)])
def test_compensation_is_the_least_squares_correction(mode, bits, group):
    W, X = _layer(3, 16, 40, 1 + bits)
    H = G.dampen(G.hessian(X), 0.01)
    codes, scales, zeros, Wq, Wc = G.gptq(W, X, bits, group, mode, corrected=True)
    W64 = W.astype(np.float64)
    for j in range(1, 16):
        C, F = np.arange(j), np.arange(j, 16)
        # minimise (w' - w)^T H (w' - w) over the free columns F, w'_C = Wq_C
        rhs = H[np.ix_(F, C)] @ (W64[:, C] - Wq[:, C]).T
        free = W64[:, F] + np.linalg.solve(H[np.ix_(F, F)], rhs).T
        np.testing.assert_allclose(Wc[:, j], free[:, 0], rtol=1e-9, atol=1e-12)
        if j % group == 0:
            # group parameters are fitted on the corrected weights of the group
            s, z = G.group_params(free[:, :group], bits, mode)
            np.testing.assert_allclose(scales[:, j // group], s, rtol=1e-6)
            np.testing.assert_array_equal(zeros[:, j // group], z)


def test_dampening_hand_example():
    # mean of the diagonal 7, one per cent of it added to the diagonal
    H = G.dampen(np.array([[4.0, 2.0], [2.0, 10.0]]), 0.01)
    np.testing.assert_allclose(H, [[4.07, 2.0], [2.0, 10.07]], rtol=0, atol=1e-15)


def test_factor_hand_example():
    # H = [[4, 2], [2, 10]]: H^-1 = [[10, -2], [-2, 4]] / 36. Row 0 is row 0 of
    # H^-1 over sqrt(10/36); eliminating index 0 leaves 4/36 - (2/36)^2 / (10/36).
    U = G.obs_factor(np.array([[4.0, 2.0], [2.0, 10.0]]))
    want = np.array([[np.sqrt(10) / 6, -2 / (6 * np.sqrt(10))], [0.0, np.sqrt(4 / 36 - 4 / 360)]])
    np.testing.assert_allclose(U, want, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("n,seed", [(5, 0), (33, 1), (128, 2)])
def test_factor_is_the_cholesky_factor_of_the_inverse(n, seed):
    r = np.random.default_rng(seed)
    A = r.standard_normal((3 * n, n))
    H = G.dampen(2.0 * A.T @ A, 0.01)
    V = G.obs_factor(H)
    assert np.all(np.tril(V, -1) == 0.0) and np.all(np.diag(V) > 0)
    Hinv = np.linalg.inv(H)
    np.testing.assert_allclose(V.T @ V, Hinv, rtol=0, atol=1e-10 * np.abs(Hinv).max())
    # a library route to the same factor: Cholesky of H^-1, transposed
    np.testing.assert_allclose(V, np.linalg.cholesky(Hinv).T, rtol=0, atol=1e-9 * np.abs(V).max())


def test_hand_worked_two_columns():
    # X rows (1, 1), (1, 0), (0, 2): X^T X = [[2, 1], [1, 5]], H = [[4, 2], [2, 10]] (no damping)
    X = np.array([[1, 1], [1, 0], [0, 2]], np.float32)
    W = np.array([[0.16, 0.25]], np.float32)
    codes, scales, zeros, Wq, Wc = G.gptq(W, X, bits=2, group=2, mode="asym", damp=0.0, corrected=True)
    # group of both columns: lo 0, hi 0.25, scale = fp32(0.25 / 3), zero 0
    s = float(np.float32(0.25 / 3))
    assert scales[0, 0] == np.float32(0.25 / 3) and zeros[0, 0] == 0
    # column 0: 0.16 / s = 1.92 -> code 2, value 2 s
    assert codes[0, 0] == 2 and Wq[0, 0] == 2 * s
    # column 1 absorbs (w0 - 2 s) * H01 / H11 = (0.16 - 2 s) * 0.2
    w1 = float(np.float32(0.25)) + (float(np.float32(0.16)) - 2 * s) * 0.2
    assert abs(Wc[0, 1] - w1) < 1e-15
    assert abs(Wc[0, 1] - 0.248666666) < 1e-8
    assert codes[0, 1] == 3 and Wq[0, 1] == 3 * s


@pytest.mark.parametrize("mode,bits", [("asym", 4), ("sym", 4), ("asym", 3)])
def test_diagonal_hessian_gives_nearest_levels(mode, bits):
    """Orthogonal input columns: nothing to compensate; every code is the
    nearest level (ties to even), found by trying every code."""
    r = np.random.default_rng(bits)
    n_in, group = 24, 8
    X = np.zeros((n_in, n_in), np.float32)
    X[np.arange(n_in), np.arange(n_in)] = r.uniform(0.5, 2.0, n_in)
    W = (r.standard_normal((5, n_in)) * 0.02).astype(np.float32)
    codes, scales, zeros, Wq = G.gptq(W, X, bits, group, mode)
    maxq = (1 << bits) - 1
    for o in range(5):
        for j in range(n_in):
            s = float(scales[o, j // group])
            z = float(zeros[o, j // group])
            levels = s * (np.arange(maxq + 1) - z)
            if mode == "sym":
                levels = s * (np.arange(maxq + 1) - (1 << (bits - 1)))
            d = np.abs(levels - float(W[o, j]))
            best = np.flatnonzero(d == d.min())
            assert codes[o, j] in best
            assert Wq[o, j] == levels[codes[o, j]]


@pytest.mark.parametrize("mode", ["asym", "sym"])
def test_gptq_beats_rtn_on_the_calibration_error(mode):
    W, X = _layer(32, 256, 512, 7, outliers=4)
    _, _, _, Wq = G.gptq(W, X, 4, 64, mode)
    # RTN: the same quantizer without compensation (diagonal U)
    U0 = np.eye(256)
    _, _, _, Wr = G.gptq(W, None, 4, 64, mode, U=U0)
    assert G.output_sse(W, Wq, X) < 0.8 * G.output_sse(W, Wr, X)


def test_pack_layout():
    codes = np.array([[1, 2, 3, 4, 5, 6, 7, 0, 15, 14]], np.int64)
    q = G.pack(codes, 4)
    big = sum(int(c) << (4 * i) for i, c in enumerate(codes[0]))
    assert q[0].tolist() == [big & 0xFFFFFFFF, big >> 32]
    c3 = np.array([[5, 2, 7, 1, 0, 6, 3, 4, 7, 7, 1]], np.int64)
    big3 = sum(int(c) << (3 * i) for i, c in enumerate(c3[0]))
    assert G.pack(c3, 3)[0].tolist() == [big3 & 0xFFFFFFFF, big3 >> 32]
