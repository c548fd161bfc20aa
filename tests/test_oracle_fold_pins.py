"""Pins of the oracle's scale folding (CPU only).

Folding ([G] "How it works" step 5 and the transformer paragraph; [C] "AWQ:
move the error away from what matters") rests on W x = (W diag(s)) (x / s):
the searched layer's weight is multiplied by s, and whatever produces x (a
norm weight, or the previous linear layer's output rows) is divided by s.
The pins: the two storage conversions against numpy's and torch's own
round-half-to-even conversions; exact results for power-of-two scales;
a hand example; and the identity itself on a Llama-style block, where a
transposed or misplaced fold (columns instead of rows, the wrong producer)
breaks the block's output.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as ref


def _special_f32():
    r = np.random.default_rng(0)
    vals = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 65536.0, 1e30, -1e30,
            np.inf, -np.inf, 2.0 ** -14, 2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001,
            3 * 2.0 ** -26, 2.0 ** -26, 1e-45, 3.4e38, 5.96e-8, 6.1e-5, 6.09e-5]
    # exact half-way points of fp16 and bf16 in several binades, and their neighbours
    for e in (-20, -14, -5, 0, 7, 15):
        for k in range(8):
            base = (1024 + k) * 2.0 ** (e - 10)
            vals += [base + 2.0 ** (e - 11), np.nextafter(np.float32(base + 2.0 ** (e - 11)), np.float32(0))]
            b2 = (128 + k) * 2.0 ** (e - 7)
            vals += [b2 + 2.0 ** (e - 8)]
    vals += list(r.standard_normal(3000) * np.exp(r.uniform(-30, 12, 3000)))
    vals += list(r.uniform(-70000, 70000, 500))
    bits = r.integers(0, 2 ** 32, 3000, dtype=np.uint64).astype(np.uint32)
    rnd = bits.view(np.float32)
    vals += list(rnd[np.isfinite(rnd)])
    return np.array(vals, np.float64).astype(np.float32)


def test_f16_conversion_matches_numpy():
    x = _special_f32()
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    got = np.array([ref.f32_to_f16_bits(v) for v in x], np.uint16)
    assert np.array_equal(got, want), x[got != want][:5]
    nan = ref.f32_to_f16_bits(np.float32(np.nan))
    assert (nan & 0x7c00) == 0x7c00 and (nan & 0x3ff) != 0


def test_bf16_conversion_matches_torch():
    x = _special_f32()
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([ref.f32_to_bf16_bits(v) for v in x], np.uint16)
    assert np.array_equal(got, want), x[got != want][:5]
    nan = ref.f32_to_bf16_bits(np.float32(np.nan))
    assert (nan & 0x7f80) == 0x7f80 and (nan & 0x7f) != 0


def test_hand_example():
    gamma = np.array([1.0, 2.0, 3.0, -1.5], np.float32)
    s = np.array([2.0, 0.5, 3.0, 0.25], np.float32)
    assert ref.fold_rows(gamma, s).ravel().tolist() == [0.5, 4.0, 1.0, -6.0]
    W = np.array([[1.0, 2.0, 3.0, 4.0], [-1.0, 0.5, 0.0, 2.0]], np.float32)
    assert ref.scale_cols(W, s).tolist() == [[2.0, 1.0, 9.0, 1.0], [-2.0, 0.25, 0.0, 0.5]]
    # a previous linear layer (3 x 2): row r divided by s[r]
    P = np.array([[2.0, 4.0], [1.0, -3.0], [6.0, 9.0]], np.float32)
    assert ref.fold_rows(P, s[:3]).tolist() == [[1.0, 2.0], [2.0, -6.0], [2.0, 3.0]]


@pytest.mark.parametrize("storage", ["f32", "f16", "bf16"])
def test_power_of_two_scales_are_exact(storage):
    r = np.random.default_rng(1)
    A = (r.standard_normal((24, 40)) * 0.05).astype(np.float32)
    if storage == "f16":
        A = A.astype(np.float16).astype(np.float32)
    elif storage == "bf16":
        A = torch.from_numpy(A).to(torch.bfloat16).float().numpy()
    k = r.integers(-3, 4, 24)
    s_rows = np.ldexp(np.ones(24), k).astype(np.float32)
    s_cols = np.ldexp(np.ones(40), r.integers(-3, 4, 40)).astype(np.float32)
    # the fp32 results are exact (ldexp); storing them rounds once, as the
    # library conversions do (fp16 may underflow into subnormals here)
    want_rows = np.ldexp(A, -k[:, None]).astype(np.float32)
    want_cols = np.ldexp(A, np.log2(s_cols).astype(int)[None, :]).astype(np.float32)
    got_rows = ref.fold_rows(A, s_rows, storage)
    got_cols = ref.scale_cols(A, s_cols, storage)
    if storage == "f16":
        want_rows, want_cols = (w.astype(np.float16).view(np.uint16) for w in (want_rows, want_cols))
    elif storage == "bf16":
        want_rows, want_cols = (torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
                                for w in (want_rows, want_cols))
    assert np.array_equal(got_rows, want_rows)
    assert np.array_equal(got_cols, want_cols)
    ones = np.ones(24, np.float32)
    same = ref.fold_rows(A, ones, "f32")
    assert np.array_equal(same, A)


def test_fold_rounds_once_per_element():
    """fp16 storage: the fp32 quotient rounded half to even to fp16, element
    by element (numpy does the same two steps)."""
    r = np.random.default_rng(2)
    A = r.standard_normal((16, 33)).astype(np.float16).astype(np.float32)
    s = np.exp(r.uniform(-3, 3, 16)).astype(np.float32)
    want = (A / s[:, None]).astype(np.float32).astype(np.float16).view(np.uint16)
    assert np.array_equal(ref.fold_rows(A, s, "f16"), want)


def _rmsnorm(h, gamma, eps=1e-6):
    return h / np.sqrt((h * h).mean(axis=1, keepdims=True) + eps) * gamma[None, :]


def _silu(x):
    return x / (1.0 + np.exp(-x))


def test_block_identity_mlp_and_attention_inputs():
    """A Llama-style block (fp32 storage, forward in fp64): the norm before the
    MLP absorbs 1/s1 of gate/up, up_proj absorbs 1/s2 of down_proj, the norm
    before attention absorbs 1/s0 of q/k/v, and v_proj absorbs 1/s3 of o_proj
    (as many KV heads as query heads, so the shapes line up). The block's
    outputs are unchanged up to fp32 rounding of the folded weights."""
    r = np.random.default_rng(3)
    T, H, I = 12, 64, 160
    h = r.standard_normal((T, H))
    g_attn = (1 + 0.1 * r.standard_normal(H)).astype(np.float32)
    g_mlp = (1 + 0.1 * r.standard_normal(H)).astype(np.float32)
    Wq, Wk, Wv, Wo = [(r.standard_normal((H, H)) * 0.1).astype(np.float32) for _ in range(4)]
    Wg, Wu = [(r.standard_normal((I, H)) * 0.1).astype(np.float32) for _ in range(2)]
    Wd = (r.standard_normal((H, I)) * 0.1).astype(np.float32)
    s0, s1, s3 = [np.exp(r.uniform(-1, 1, H)).astype(np.float32) for _ in range(3)]
    s2 = np.exp(r.uniform(-1, 1, I)).astype(np.float32)

    def block(ga, q, k, v, o, gm, g, u, d):
        f = lambda a: np.asarray(a, np.float64)
        n = _rmsnorm(h, f(ga))
        Q, K, V = n @ f(q).T, n @ f(k).T, n @ f(v).T
        att = Q @ K.T / np.sqrt(H)
        att = np.exp(att - att.max(axis=1, keepdims=True))
        att /= att.sum(axis=1, keepdims=True)
        x1 = h + (att @ V) @ f(o).T
        m = _rmsnorm(x1, f(gm))
        y = x1 + (_silu(m @ f(g).T) * (m @ f(u).T)) @ f(d).T
        return Q, K, V, x1, y

    base = block(g_attn, Wq, Wk, Wv, Wo, g_mlp, Wg, Wu, Wd)
    fold = block(ref.fold_rows(g_attn, s0).ravel(),
                 ref.scale_cols(Wq, s0), ref.scale_cols(Wk, s0),
                 ref.fold_rows(ref.scale_cols(Wv, s0), s3),      # v_proj rows absorb o_proj's 1/s3
                 ref.scale_cols(Wo, s3),
                 ref.fold_rows(g_mlp, s1).ravel(),
                 ref.scale_cols(Wg, s1),
                 ref.fold_rows(ref.scale_cols(Wu, s1), s2),      # up_proj rows absorb down_proj's 1/s2
                 ref.scale_cols(Wd, s2))
    # q and k are unchanged; v is divided by s3 column-wise (o_proj undoes it);
    # the attention output and the block output are unchanged
    for a, b in ((base[0], fold[0]), (base[1], fold[1]), (base[2] / s3[None, :], fold[2]),
                 (base[3], fold[3]), (base[4], fold[4])):
        np.testing.assert_allclose(b, a, rtol=0, atol=1e-5 * np.abs(a).max())
    # without the folds the scaled weights change the block
    broken = block(g_attn, ref.scale_cols(Wq, s0), Wk, Wv, Wo, g_mlp, Wg, Wu, Wd)
    assert np.abs(broken[0] - base[0]).max() > 1e-2 * np.abs(base[0]).max()
