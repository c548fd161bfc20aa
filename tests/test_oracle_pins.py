"""Pins of the CPU oracle to facts fixed outside itself (CPU only).

Each test checks the oracle against a value printed on the pages, a closed
form, an invariant the pages state, a brute-force enumeration, or a library
routine on a special case, chosen so that a dropped term, a wrong sign or
index, or a transposed operand anywhere in the oracle fails at least one.
"""
import math

import numpy as np
import pytest
import torch

from conftest import read_golden
from post_weight_quantization_30_amd import synth


def _rng(seed):
    return np.random.default_rng(seed)


def _unpack_rows(qweight, n_in, bits):
    """Independent bit-stream reader: code i of a row sits at bits [i*bits, (i+1)*bits)."""
    out = qweight.shape[0]
    words = qweight.astype(np.uint64)
    codes = np.zeros((out, n_in), np.int64)
    for i in range(n_in):
        bit = i * bits
        w, sh = divmod(bit, 32)
        val = words[:, w] >> np.uint64(sh)
        if sh + bits > 32:
            val = val | (words[:, w + 1] << np.uint64(32 - sh))
        codes[:, i] = (val & np.uint64((1 << bits) - 1)).astype(np.int64)
    return codes


# ---------------------------------------------------------------------------
# P1: the two-channel worked example (printed values)
# ---------------------------------------------------------------------------
def test_worked_example_two_channels(ref):
    g = read_golden("two_channel_worked_example.txt")
    w = np.array([g["w"]], np.float32)
    abar = np.array(g["abar"], np.float32)
    bits = int(g["bits"][0])
    X = abar[None, :]                       # one token whose |x| are the printed averages
    xmag = ref.act_stats(X)
    np.testing.assert_allclose(xmag, abar, rtol=1e-6)
    st = ref.s_table(xmag, 20)
    k = int(round(g["alpha"][0] * 20))
    s = st[k]

    # codes of the scaled weights and of plain RTN
    code, scale, zero, _ = ref.quant_group(w[0] * s, bits, "sym")
    assert list(code - zero) == [int(c) for c in g["awq_signed_codes"]]
    code0, scale0, zero0, _ = ref.quant_group(w[0], bits, "sym")
    assert list(code0 - zero0) == [int(c) for c in g["rtn_signed_codes"]]
    assert math.isclose(scale0, 2.0 / 3.0, rel_tol=1e-6)

    weff = ref.fake_quant(w, s, bits, 2, "sym")[0]
    np.testing.assert_allclose(weff, g["awq_w_eff"], atol=5e-4)
    np.testing.assert_allclose(np.abs(w[0] - weff) * abar, g["awq_weighted_error"], atol=5e-4)
    weff0 = ref.fake_quant(w, st[0], bits, 2, "sym")[0]
    np.testing.assert_allclose(weff0, g["rtn_w_eff"], atol=5e-4)
    np.testing.assert_allclose(np.abs(w[0] - weff0) * abar, g["rtn_weighted_error"], atol=5e-3)

    # The page normalises by the largest magnitude instead of sqrt(max*min);
    # its s = (abar/max)^alpha gives the same effective weights.
    s_page = np.array([1.0, 0.1], np.float32)
    np.testing.assert_allclose(ref.fake_quant(w, s_page, bits, 2, "sym")[0], weff, rtol=1e-6)

    # One-token output error follows from the printed weighted errors:
    # AWQ (-0.0333)^2 and RTN (1.667)^2.
    mse, best, s_best, status = ref.search(w, X, xmag, bits, 2, 20, "sym")
    assert status == 0
    assert math.isclose(mse[k], (0.1 * (2.0 - 5.0 / 3.0)) ** 2, rel_tol=1e-4)
    assert math.isclose(mse[0], (10.0 * (2.0 / 3.0 - 0.5)) ** 2, rel_tol=1e-4)
    assert mse[best] <= mse[k]


# ---------------------------------------------------------------------------
# P2: alpha = 0 is plain RTN
# ---------------------------------------------------------------------------
def _torch_rtn(w, bits, group):
    """Symmetric group RTN ("Output MSE vs bit width" of "GPTQ and AWQ weight
    quantisation") as a nearest-level search in torch: each group's step is
    its largest magnitude over the 2^(b-1) - 1 positive levels (floored at
    1e-8); every weight takes the level k in [-2^(b-1), 2^(b-1) - 1] nearest
    to w / step (fp32 quotient, as the method computes it), ties to the even
    k; the value is k * step in fp32."""
    out_f, in_f = w.shape
    top = (1 << (bits - 1)) - 1
    wg = torch.from_numpy(w).reshape(out_f, in_f // group, group).to(torch.float32)
    step = torch.maximum(wg.abs().max(dim=-1, keepdim=True).values / top,
                         torch.tensor(1e-8, dtype=torch.float32))
    t = (wg / step).to(torch.float64).unsqueeze(-1)          # exact in fp64
    ks = torch.arange(-top - 1, top + 1, dtype=torch.float64)
    dist = (t - ks).abs()
    near = dist == dist.min(dim=-1, keepdim=True).values
    # among equally near levels, the even one
    pick = torch.where(near & (ks.remainder(2) == 0), 1, 0) + near.to(torch.int64) * 2
    k = ks[pick.argmax(dim=-1)]
    value = (k.to(torch.float32) * step)
    return value.reshape(out_f, in_f).numpy(), k.reshape(out_f, in_f).numpy().astype(np.int64)


@pytest.mark.parametrize("bits,group", [(4, 128), (3, 64), (2, 32)])
def test_alpha_zero_is_rtn(ref, bits, group):
    r = _rng(1)
    out, n_in, T = 24, 256, 40
    W = (r.standard_normal((out, n_in)) * 0.02).astype(np.float32)
    X = r.standard_normal((T, n_in)).astype(np.float32)
    X[:, [3, 77]] *= 6
    xmag = ref.act_stats(X)
    st = ref.s_table(xmag, 20)
    assert np.all(st[0] == np.float32(1.0))
    w_rtn, q_rtn = _torch_rtn(W, bits, group)
    qw, sc, z = ref.quantize_pack(W, st[0], bits, group, "sym")
    codes = _unpack_rows(qw, n_in, bits)
    assert np.array_equal(codes - (1 << (bits - 1)), q_rtn)
    mse, best, _, _ = ref.search(W, X, xmag, bits, group, 20, "sym")
    X64 = X.astype(np.float64)
    rtn_mse = np.mean((X64 @ w_rtn.astype(np.float64).T - X64 @ W.astype(np.float64).T) ** 2)
    assert math.isclose(mse[0], rtn_mse, rel_tol=1e-12)


# ---------------------------------------------------------------------------
# P3: the chosen error is never above RTN's; on the notebook's own setup it is below
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", ["sym", "asym"])
def test_awq_never_worse_than_rtn(ref, mode):
    for seed in range(4):
        r = _rng(10 + seed)
        out, n_in, T = 16, 128, 24
        W = (r.standard_normal((out, n_in)) * 0.02).astype(np.float32)
        X = r.standard_normal((T, n_in)).astype(np.float32)
        X[:, r.choice(n_in, 3, replace=False)] *= 20
        xmag = ref.act_stats(X)
        mse, best, s_best, st = ref.search(W, X, xmag, 4, 64, 10, mode)
        assert st == 0
        assert mse[best] <= mse[0]
        assert mse[best] == mse.min()
        assert best == int(np.argmin(mse))


def test_awq_beats_rtn_on_notebook_setup(ref):
    # The notebook's 4096x4096 / 256-token / g128 int4 layer with 64 outlier
    # channels x6, on its first 128 output rows (rows are independent).
    spec = synth.with_shape(synth.HEADLINE, out=128)
    lay = synth.make_layer(spec)
    W = synth.storage_to_f32(lay["W"], spec.dtype)
    X = synth.storage_to_f32(lay["X"], spec.dtype)
    xmag = ref.act_stats(X)
    mse, best, _, st = ref.search(W, X, xmag, 4, 128, 20, "sym")
    assert st == 0 and best > 0
    assert mse[best] < mse[0]
    assert np.isfinite(mse).all() and mse[best] > 0


# ---------------------------------------------------------------------------
# P4: the error functional itself (closed forms, library routine)
# ---------------------------------------------------------------------------
def test_scaling_identity_gives_zero_error(ref):
    r = _rng(2)
    out, n_in, T = 9, 40, 13
    W = r.standard_normal((out, n_in)).astype(np.float32)
    X = r.standard_normal((T, n_in)).astype(np.float32)
    s = np.exp(r.uniform(-3, 3, n_in))
    wq = (W.astype(np.float64) * s) / s       # (W s)(x / s) = W x before rounding
    ref_out = X.astype(np.float64) @ W.astype(np.float64).T
    assert ref.output_mse(W, wq, X) <= 1e-24 * np.mean(ref_out ** 2)


def test_output_error_single_perturbation_closed_form(ref):
    r = _rng(3)
    out, n_in, T = 7, 12, 5                  # all different: a transposed operand fails
    W = r.standard_normal((out, n_in)).astype(np.float32)
    X = r.standard_normal((T, n_in)).astype(np.float32)
    for (o, i, d) in [(0, 0, 0.5), (6, 11, -0.25), (3, 7, 2.0)]:
        wq = W.astype(np.float64).copy()
        wq[o, i] += d
        expect = d * d * np.sum(X[:, i].astype(np.float64) ** 2) / (T * out)
        assert math.isclose(ref.output_mse(W, wq, X), expect, rel_tol=1e-12)


def test_output_error_matches_numpy_matmul(ref):
    r = _rng(4)
    out, n_in, T = 11, 32, 6
    W = r.standard_normal((out, n_in)).astype(np.float32)
    X = r.standard_normal((T, n_in)).astype(np.float32)
    wq = W.astype(np.float64) + r.standard_normal((out, n_in)) * 1e-2
    X64 = X.astype(np.float64)
    expect = np.mean((X64 @ wq.T - X64 @ W.astype(np.float64).T) ** 2)
    assert math.isclose(ref.output_mse(W, wq, X), expect, rel_tol=1e-12)


# ---------------------------------------------------------------------------
# P5: flat activations reduce AWQ to RTN, and ties keep the lowest alpha
# ---------------------------------------------------------------------------
def test_flat_activations_tie_to_rtn(ref):
    r = _rng(5)
    out, n_in, T = 8, 64, 10
    W = (r.standard_normal((out, n_in)) * 0.02).astype(np.float32)
    X = np.where(r.random((T, n_in)) < 0.5, -0.75, 0.75).astype(np.float32)
    xmag = ref.act_stats(X)
    assert np.all(xmag == xmag[0])
    st = ref.s_table(xmag, 20)
    assert np.all(st == np.float32(1.0))
    mse, best, s_best, _ = ref.search(W, X, xmag, 4, 32, 20, "sym")
    assert np.all(mse == mse[0]) and best == 0
    assert np.all(s_best == 1.0)


# ---------------------------------------------------------------------------
# P6: centring only changes rounding: a power-of-two factor on s changes nothing
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", ["sym", "asym"])
def test_power_of_two_rescale_is_exact(ref, mode):
    r = _rng(6)
    for bits in (2, 3, 4, 8):
        v = (r.standard_normal(64) * 0.3).astype(np.float32)
        c0, s0, z0, _ = ref.quant_group(v, bits, mode)
        for m in (-3, -1, 2, 5):
            c1, s1, z1, _ = ref.quant_group(v * np.float32(2.0 ** m), bits, mode)
            assert np.array_equal(c0, c1) and z0 == z1
            assert s1 == np.float32(s0 * np.float32(2.0 ** m))


# ---------------------------------------------------------------------------
# P7, P8, P10: the group quantizer against its error bound, brute force, ranges
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", ["sym", "asym"])
def test_quantizer_error_bound_and_ranges(ref, mode):
    r = _rng(7)
    for bits in range(2, 9):
        for _ in range(20):
            g = int(r.choice([8, 32, 64, 128]))
            v = (r.standard_normal(g) * r.uniform(1e-3, 10)).astype(np.float32)
            if mode == "asym" and r.random() < 0.3:
                v = np.abs(v) + np.float32(r.uniform(0, 1))    # same-sign group: range still holds 0
            if r.random() < 0.5:
                v[r.integers(g)] = 0.0
            code, scale, zero, what = ref.quant_group(v, bits, mode)
            maxc = (1 << bits) - 1
            assert 0 <= zero <= maxc
            assert code.min() >= (1 if mode == "sym" else 0) and code.max() <= maxc
            err = np.abs(v.astype(np.float64) - what.astype(np.float64))
            assert np.all(err <= scale / 2 * (1 + 1e-6) + 1e-12)
            assert np.all(what[v == 0] == 0.0)        # zero is exactly representable
            if mode == "sym":
                lv = (1 << (bits - 1)) - 1
                assert abs(code[np.argmax(np.abs(v))] - zero) == lv   # the group max gets the top level
            else:
                if v.min() < 0:
                    assert code[np.argmin(v)] == 0
                assert code[np.argmax(v)] >= maxc - 1


def test_quantizer_ties_round_half_to_even(ref):
    # np.round (the awq() listing) and torch.round (the notebook) round half to even.
    code, scale, zero, what = ref.quant_group(np.array([7.0, 2.5, -1.5, 0.5, -0.5, 3.5], np.float32), 4, "sym")
    assert scale == 1.0 and zero == 8
    assert list(code - zero) == [7, 2, -2, 0, 0, 4]
    # asym: range [-0.5, 7] over 15 levels gives scale 0.5; v/scale = 5 and 1.5 -> 2 (even)
    code, scale, zero, _ = ref.quant_group(np.array([-0.5, 7.0, 0.75, 2.5], np.float32), 4, "asym")
    assert scale == 0.5 and zero == 1
    assert list(code) == [0, 15, 3, 6]


@pytest.mark.parametrize("mode", ["sym", "asym"])
def test_all_zero_group_uses_scale_floor(ref, mode):
    code, scale, zero, what = ref.quant_group(np.zeros(16, np.float32), 4, mode)
    assert scale == np.float32(1e-8)
    assert np.all(what == 0.0) and np.all(code == zero)
    assert zero == (8 if mode == "sym" else 0)


def test_asym_range_always_holds_zero(ref):
    # group_params on the comparison page widens [min, max] to include 0
    v = np.array([0.2, 0.5, 1.7, 3.2], np.float32)          # all positive: lo -> 0
    code, scale, zero, what = ref.quant_group(v, 4, "asym")
    assert zero == 0 and scale == np.float32(np.float32(3.2) / np.float32(15))
    code, scale, zero, what = ref.quant_group(-v, 4, "asym")  # all negative: hi -> 0
    assert zero == 15 and code[3] == 0


@pytest.mark.parametrize("mode", ["sym", "asym"])
def test_quantizer_codes_brute_force(ref, mode):
    """Each code is the representable level nearest to v (enumerated), except
    where fp32 division lands within 1e-5 of a half-way point (excluded)."""
    r = _rng(8)
    checked = 0
    for bits in range(2, 9):
        for _ in range(10):
            g = int(r.choice([4, 16, 128]))
            v = (r.standard_normal(g) * 0.05).astype(np.float32)
            code, scale, zero, _ = ref.quant_group(v, bits, mode)
            levels = np.arange(1 << bits)
            recon = np.float64(scale) * (levels - zero)
            for i in range(g):
                x = np.float64(v[i]) / np.float64(scale)
                if abs(abs(x - np.floor(x)) - 0.5) < 1e-5:
                    continue
                dist = np.abs(np.float64(v[i]) - recon)
                assert code[i] == int(np.argmin(dist))
                checked += 1
    assert checked > 1000


# ---------------------------------------------------------------------------
# P9: packing round trip and the storage arithmetic printed on the pages
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("bits,group,mode", [(4, 128, "sym"), (3, 64, "sym"), (4, 32, "asym"),
                                             (5, 96, "asym"), (8, 48, "sym"), (2, 160, "asym")])
def test_pack_round_trip(ref, bits, group, mode):
    r = _rng(9)
    out, n_in = 5, group * 3
    W = (r.standard_normal((out, n_in)) * 0.02).astype(np.float32)
    s = np.exp(r.uniform(-1, 1, n_in)).astype(np.float32)
    qw, sc, z = ref.quantize_pack(W, s, bits, group, mode)
    assert qw.shape == (out, (n_in * bits + 31) // 32)
    codes = _unpack_rows(qw, n_in, bits)
    for o in range(out):
        for gi in range(n_in // group):
            sl = slice(gi * group, (gi + 1) * group)
            c, scale, zero, _ = ref.quant_group(W[o, sl] * s[sl], bits, mode)
            assert np.array_equal(codes[o, sl], c)
            assert sc[o, gi] == scale and z[o, gi] == zero
    # bits beyond the last code of each row are zero
    tail = qw.shape[1] * 32 - n_in * bits
    if tail:
        assert np.all((qw[:, -1].astype(np.uint64) >> np.uint64(32 - tail)) == 0)


def test_storage_math_matches_pages(ref):
    g = read_golden("storage_math.txt")
    out, n_in, group = int(g["layer_out"][0]), int(g["layer_in"][0]), int(g["group"][0])
    W = np.zeros((out, n_in), np.float32)
    qw, sc, z = ref.quantize_pack(W, np.ones(n_in, np.float32), 4, group, "sym")
    mib = 1024.0 ** 2
    assert out * n_in * 2 / mib == g["fp16_layer_mib"][0]
    assert qw.nbytes / mib == g["int4_weight_mib"][0]
    fp16_scales = sc.size * 2 / mib
    assert fp16_scales == g["fp16_scale_mib"][0]
    assert qw.nbytes / mib + fp16_scales == g["total_mib"][0]
    ratio = g["fp16_layer_mib"][0] / g["total_mib"][0]
    assert abs(ratio - g["compression_target"][0]) <= g["compression_rtol"][0] * g["compression_target"][0]
    # 4-bit code + 16-bit scale + 4-bit zero per 128 weights
    bpw = 8 * qw.nbytes / (out * n_in) + (16 + 4) / group
    assert abs(bpw - g["bits_per_weight"][0]) < 0.005
    # this library stores fp32 scales and byte zeros: 4 + (32 + 8)/128 bits
    assert 8 * (qw.nbytes + sc.nbytes + z.nbytes) / (out * n_in) == 4 + 40 / group


# ---------------------------------------------------------------------------
# P11, P12 and the statistics / s-table closed forms
# ---------------------------------------------------------------------------
def test_s_table_centring_and_closed_form(ref):
    r = _rng(11)
    xmag = np.exp(r.uniform(-4, 4, 300)).astype(np.float32)
    grid = 20
    st = ref.s_table(xmag, grid)
    x64 = xmag.astype(np.float64)
    for k in range(grid + 1):
        a = k / grid
        prod = np.float64(st[k].max()) * np.float64(st[k].min())
        assert abs(prod - 1.0) < 4 * 2.0 ** -23
        expect = (x64 / np.sqrt(x64.max() * x64.min())) ** a
        np.testing.assert_allclose(st[k], expect, rtol=2e-7)
    # two channels: s = [(a/b)^(alpha/2), (b/a)^(alpha/2)]
    two = np.array([9.0, 0.25], np.float32)
    st2 = ref.s_table(two, 4)
    for k in range(5):
        a = k / 4
        np.testing.assert_allclose(st2[k], [(36.0) ** (a / 2), (1 / 36.0) ** (a / 2)], rtol=1e-7)
    # alpha = 1 over the grid's end: s proportional to xmag
    np.testing.assert_allclose(st[grid] / st[grid][0], x64 / x64[0], rtol=3e-7)


def test_act_stats_exact_for_fp16_and_ragged_tokens(ref):
    r = _rng(12)
    for T in (1, 63, 64, 100, 257):
        X16 = (r.standard_normal((T, 48)) * 3).astype(np.float16)
        X16[:, 5] = 0
        X = X16.astype(np.float32)
        xmag = ref.act_stats(X)
        # fp16 values are multiples of 2^-24 below 2^16: their fp64 sum is exact in any order
        exact = np.abs(X16.astype(np.float64)).sum(0) / T
        assert np.array_equal(xmag, (exact + 1e-8).astype(np.float32))
        assert xmag[5] == np.float32(1e-8)


def test_act_stats_close_to_exact_mean_fp32(ref):
    r = _rng(13)
    X = (r.standard_normal((333, 20)) * np.exp(r.uniform(-5, 5, 20))).astype(np.float32)
    xmag = ref.act_stats(X)
    exact = np.array([math.fsum(abs(float(v)) for v in X[:, j]) / 333 + 1e-8 for j in range(20)])
    np.testing.assert_allclose(xmag, exact, rtol=2 ** -23)


def test_zero_channels_keep_finite_scales(ref):
    spec = synth.with_shape(synth.CONFIGS[4], out=16, tokens=64, inn=1024)
    lay = synth.make_layer(spec)
    assert len(lay["zeros"]) >= 1
    W = synth.storage_to_f32(lay["W"], spec.dtype)
    X = synth.storage_to_f32(lay["X"], spec.dtype)
    xmag = ref.act_stats(X)
    assert np.all(xmag[lay["zeros"]] == np.float32(1e-8))
    st = ref.s_table(xmag, spec.grid)
    assert np.isfinite(st).all() and (st > 0).all()
    mse, best, s_best, status = ref.search(W, X, xmag, spec.bits, spec.group, spec.grid, spec.mode)
    assert status == 0 and np.isfinite(mse).all() and np.isfinite(s_best).all()


# ---------------------------------------------------------------------------
# the search loop against an independent loop on tiny inputs
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode,bits,group", [("sym", 4, 16), ("asym", 3, 8), ("asym", 4, 48)])
def test_search_matches_independent_loop(ref, mode, bits, group):
    r = _rng(14)
    out, n_in, T, grid = 6, 96 if group != 48 else 144, 9, 8
    W = (r.standard_normal((out, n_in)) * 0.05).astype(np.float32)
    X = r.standard_normal((T, n_in)).astype(np.float32)
    X[:, 2] *= 30
    xmag = ref.act_stats(X)
    st = ref.s_table(xmag, grid)
    X64 = X.astype(np.float64)
    ref_out = X64 @ W.astype(np.float64).T
    errs = []
    for k in range(grid + 1):
        wq = ref.fake_quant(W, st[k], bits, group, mode)
        errs.append(np.mean((X64 @ wq.T - ref_out) ** 2))
    best, best_err = -1, math.inf
    for k, e in enumerate(errs):
        if e < best_err:
            best, best_err = k, e
    mse, b, s_best, status = ref.search(W, X, xmag, bits, group, grid, mode)
    np.testing.assert_allclose(mse, errs, rtol=1e-12)
    assert b == best and np.array_equal(s_best, st[best])


def test_nonfinite_input_gives_no_choice(ref):
    W = np.ones((2, 32), np.float32) * 0.1
    X = np.ones((3, 32), np.float32)
    X[1, 4] = np.nan
    xmag = ref.act_stats(X)
    mse, best, s_best, status = ref.search(W, X, xmag, 4, 32, 4, "sym")
    assert status == -4 and best == -1
    assert np.isnan(mse).all() and np.all(s_best == 1.0)
