"""Pins of the oracle's clipping-range search and clipped pack (CPU only).

The pages describe the clipping search in prose only ("AWQ (activation-aware
weight quantization)", "Simplifications"; "AWQ vs GPTQ Quantization
Architectures Compared", "AWQ: move the error away from what matters"), so
these pins fix the readings stated in the oracle's header: the ratio grid,
the clipped quantizer and the per-group output-error objective. They are
checked against hand-worked values and properties, not against the oracle's
own formulas.
"""
import numpy as np
import pytest


def test_ratio_grid(ref):
    # r_i = 1 - i * max_shrink / n_clip, rounded once to fp32; r_0 = 1 exactly.
    assert ref.clip_ratio(0, 20, 0.5) == np.float32(1.0)
    assert ref.clip_ratio(19, 20, 0.5) == np.float32(0.525)
    assert ref.clip_ratio(3, 4, 0.75) == np.float32(0.4375)
    assert ref.clip_ratio(1, 4, 0.75) == np.float32(0.8125)


@pytest.mark.parametrize("mode", ["sym", "asym"])
@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_ratio_one_is_plain_rtn(ref, mode, bits):
    r = np.random.default_rng(bits)
    for _ in range(20):
        v = (r.standard_normal(64) * r.uniform(0.01, 10)).astype(np.float32)
        c0, s0, z0, w0 = ref.quant_group(v, bits, mode)
        c1, s1, z1, w1 = ref.quant_group_clip(v, bits, mode, 1.0)
        assert np.array_equal(c0, c1) and s0 == s1 and z0 == z1 and np.array_equal(w0, w1)


def test_clipped_quantizer_hand_example(ref):
    # 3-bit symmetric (L = 3), r = 0.5: range [-0.5, 0.5], scale = 0.5/3.
    # Clamped values [0.5, 0.5, -0.25, 0.1] / scale = [3, 3, -1.5, 0.6]
    # -> rne [3, 3, -2, 1] -> dequantized [0.5, 0.5, -1/3, 1/6].
    v = np.array([1.0, 0.5, -0.25, 0.1], np.float32)
    code, scale, zero, what = ref.quant_group_clip(v, 3, "sym", 0.5)
    assert scale == np.float32(np.float32(0.5) / np.float32(3.0))
    assert np.array_equal(code - zero, [3, 3, -2, 1])
    np.testing.assert_allclose(what, [0.5, 0.5, -1 / 3, 1 / 6], rtol=1e-6)
    # asymmetric 2-bit (maxq = 3), r = 0.5 on v in [-1, 2]: range [-0.5, 1],
    # scale = 1.5/3 = 0.5, zero = rne(0.5/0.5) = 1; clamped [-0.5, 1, 0.2]
    # -> rne(x/0.5) + 1 = [0, 3, 1 (0.4 -> 0, +1)].
    v = np.array([-1.0, 2.0, 0.2], np.float32)
    code, scale, zero, what = ref.quant_group_clip(v, 2, "asym", 0.5)
    assert scale == np.float32(0.5) and zero == 1
    assert np.array_equal(code, [0, 3, 1])
    np.testing.assert_allclose(what, [-0.5, 1.0, 0.0], atol=1e-7)


def _designed_case(s_value):
    # One group of 4 columns; column 0 carries a large weight but its
    # activations are all zero, so clipping it costs nothing in output error.
    # X picks out columns 1..3 one token at a time, so a choice's error is
    # sum_{j=1..3} (wq_j - w_j)^2 exactly.
    W = np.array([[1.0, 0.29, 0.15, 0.05]], np.float32)
    X = np.array([[0, 1, 0, 0], [0, 0, 1, 0], [0, 0, 0, 1]], np.float32)
    s = np.full(4, s_value, np.float32)
    return W, X, s


@pytest.mark.parametrize("s_value", [1.0, 2.0])
def test_search_hand_worked_example(ref, s_value):
    # 4-bit symmetric (L = 7), ratios {1, 0.8125, 0.625, 0.4375} (n_clip = 4,
    # max_shrink = 0.75); the range max is r * 1.0 (times s, which cancels).
    #   r = 1:      scale 1/7:      codes 2, 1, 0 -> errors -0.004286, -0.007143, -0.05
    #   r = 0.8125: scale 0.116071: codes 2, 1, 0 -> errors -0.057857, -0.033929, -0.05
    #   r = 0.625:  scale 0.089286: codes 3, 2, 1 -> errors -0.022143, +0.028571, +0.039286
    #   r = 0.4375: scale 0.0625:   codes 5, 2, 1 -> errors +0.0225,   -0.025,    +0.0125
    # Sums of squares: 2.5694e-3, 6.9986e-3, 2.8500e-3, 1.2875e-3 -> the
    # smallest ratio wins although it clips column 0 from 1.0 to 0.4375.
    W, X, s = _designed_case(s_value)
    clip, sse = ref.clip_search(W, X, s, 4, 4, "sym", n_clip=4, max_shrink=0.75)
    assert clip[0, 0] == np.float32(0.4375)
    want = [
        (1 / 7 * 2 - 0.29) ** 2 + (1 / 7 - 0.15) ** 2 + 0.05 ** 2,
        (0.8125 / 7 * 2 - 0.29) ** 2 + (0.8125 / 7 - 0.15) ** 2 + 0.05 ** 2,
        (0.625 / 7 * 3 - 0.29) ** 2 + (0.625 / 7 * 2 - 0.15) ** 2 + (0.625 / 7 - 0.05) ** 2,
        (0.0625 * 5 - 0.29) ** 2 + (0.0625 * 2 - 0.15) ** 2 + (0.0625 - 0.05) ** 2,
    ]
    np.testing.assert_allclose(sse[0, 0], want, rtol=2e-6)


def test_search_never_worse_than_no_clip_and_ties_keep_first(ref):
    r = np.random.default_rng(7)
    W = (r.standard_normal((6, 128)) * 0.02).astype(np.float32)
    X = r.standard_normal((24, 128)).astype(np.float32)
    s = np.exp(r.uniform(-1, 1, 128)).astype(np.float32)
    for mode in ("sym", "asym"):
        clip, sse = ref.clip_search(W, X, s, 4, 32, mode)
        best = sse.argmin(-1)        # numpy argmin keeps the first minimum too
        ratios = np.array([ref.clip_ratio(i, 20, 0.5) for i in range(20)], np.float32)
        assert np.array_equal(clip, ratios[best])
        assert np.all(sse.min(-1) <= sse[..., 0])
    # all-zero weights: every ratio gives the same (zero) error -> ratio 1
    clip, sse = ref.clip_search(np.zeros((2, 64), np.float32), X[:, :64], s[:64], 4, 32, "sym")
    assert np.all(clip == 1.0) and np.all(sse == 0.0)


@pytest.mark.parametrize("mode", ["sym", "asym"])
def test_clipped_pack_matches_groupwise_quantizer(ref, mode):
    r = np.random.default_rng(11)
    W = (r.standard_normal((5, 256)) * 0.02).astype(np.float32)
    s = np.exp(r.uniform(-1, 1, 256)).astype(np.float32)
    clip = np.array([[ref.clip_ratio(int(k), 20, 0.5) for k in row] for row in r.integers(0, 20, (5, 4))],
                    np.float32)
    q, sc, z = ref.quantize_pack_clip(W, s, clip, 3, 64, mode)
    # ratio 1 everywhere is the plain pack
    q1, sc1, z1 = ref.quantize_pack_clip(W, s, np.ones_like(clip), 3, 64, mode)
    q0, sc0, z0 = ref.quantize_pack(W, s, 3, 64, mode)
    assert np.array_equal(q1, q0) and np.array_equal(sc1, sc0) and np.array_equal(z1, z0)
    # each group's codes, scale and zero are the clipped group quantizer's
    bits_all = np.unpackbits(q.view(np.uint8), bitorder="little").reshape(5, -1)
    for o in range(5):
        for g in range(4):
            v = (W[o, g * 64:(g + 1) * 64] * s[g * 64:(g + 1) * 64]).astype(np.float32)
            code, scale, zero, _ = ref.quant_group_clip(v, 3, mode, clip[o, g])
            got = bits_all[o, g * 64 * 3:(g + 1) * 64 * 3].reshape(64, 3) @ (1 << np.arange(3))
            assert np.array_equal(got, code) and sc[o, g] == scale and z[o, g] == zero
