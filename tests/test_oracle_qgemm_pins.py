"""Pins of the oracle's deployment product Y = X Wd^T over the packed layout
(CPU only). Wd = scale * (code - zero) per group ([C] "What lands on disk";
the product is what a serving kernel computes, "From checkpoint to kernel").

The pins: a hand-worked row; the bit order of a 3-bit stream built with
Python integers; the round trip through the oracle's own pack (the identity
matrix as X returns the quantizer's dequantized values bit for bit); a
random X against numpy on those values; and the deployment identity
(X / s) Wd^T = X (Q(W diag(s)) / s)^T that ties the product to the search.
"""
import numpy as np
import pytest

from oracle import oracle as ref


def test_hand_worked_row():
    # eight 4-bit codes 0..7 in one word (code i at bits 4i), scale 0.5, zero 8:
    # Wd = 0.5 * (i - 8) = -4, -3.5, ..., -0.5; X = 1..8:
    # sum (i + 1) * (i - 8) over i = 0..7 = 140 - 196 - 64 = -120, times 0.5 = -60
    q = np.array([[0x76543210]], np.uint32)
    Y = ref.qgemm(np.arange(1, 9, dtype=np.float32)[None, :], q, np.array([[0.5]], np.float32),
                  np.array([[8]], np.uint8), 4, 8)
    assert Y.tolist() == [[-60.0]]


def test_three_bit_stream_order():
    codes = [5, 2, 7, 1, 0, 6, 3, 4, 7, 7, 1, 2, 3, 4, 5, 6, 0, 1, 2, 3, 7, 6, 5, 4]
    big = sum(c << (3 * i) for i, c in enumerate(codes))
    words = np.array([(big >> (32 * w)) & 0xFFFFFFFF for w in range(3)], np.uint32)
    assert [ref.unpack_code(words, k, 3) for k in range(len(codes))] == codes


@pytest.mark.parametrize("bits,group,mode", [(4, 128, "sym"), (4, 32, "asym"), (3, 64, "sym"),
                                             (8, 64, "asym"), (2, 32, "asym"), (5, 128, "sym")])
def test_round_trip_through_the_pack(bits, group, mode):
    r = np.random.default_rng(bits * group)
    out, n_in = 6, 256
    W = (r.standard_normal((out, n_in)) * 0.02).astype(np.float32)
    s = np.exp(r.uniform(-1, 1, n_in)).astype(np.float32)
    q, sc, z = ref.quantize_pack(W, s, bits, group, mode)
    # dequantized values from the quantizer itself, group by group
    what = np.empty((out, n_in), np.float32)
    for o in range(out):
        for g in range(n_in // group):
            cols = slice(g * group, (g + 1) * group)
            what[o, cols] = ref.quant_group((W[o, cols] * s[cols]).astype(np.float32), bits, mode)[3]
    eye = np.eye(n_in, dtype=np.float32)
    Y = ref.qgemm(eye, q, sc, z, bits, group)
    assert np.array_equal(Y.T.astype(np.float32), what)
    # random X: `what` is the fp32 rounding of the exact Wd, so each product
    # differs by at most 2^-24 of |x * what| (plus fp64 summation noise)
    X = r.standard_normal((9, n_in)).astype(np.float32)
    Xd, Wh = X.astype(np.float64), what.astype(np.float64)
    diff = np.abs(ref.qgemm(X, q, sc, z, bits, group) - Xd @ Wh.T)
    assert np.all(diff <= 2.0 ** -24 * (np.abs(Xd) @ np.abs(Wh).T) * 1.001 + 1e-15)


def test_deployment_identity():
    """Feeding X / s through the packed weights gives the search's fake-quantized
    product X (Q(W diag(s)) / s)^T, up to the fp32 rounding of X / s."""
    r = np.random.default_rng(4)
    out, n_in, T = 16, 256, 12
    W = (r.standard_normal((out, n_in)) * 0.02).astype(np.float32)
    X = r.standard_normal((T, n_in)).astype(np.float32)
    s = np.exp(r.uniform(-1, 1, n_in)).astype(np.float32)
    q, sc, z = ref.quantize_pack(W, s, 4, 64, "asym")
    Y = ref.qgemm((X / s[None, :]).astype(np.float32), q, sc, z, 4, 64)
    want = X.astype(np.float64) @ ref.fake_quant(W, s, 4, 64, "asym").T
    np.testing.assert_allclose(Y, want, rtol=0, atol=1e-6 * np.abs(want).max())
