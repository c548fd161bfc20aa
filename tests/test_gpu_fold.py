"""Scale folding on the GPU against the oracle: bitwise for every storage type
and shape class (vector, matrix with a multiple of 8 columns, other widths,
ragged tails, misaligned and in-place buffers), and end to end: the deployed
layer -- its input produced by a folded norm weight, its weight the packed
codes -- reproduces the error that the search reported.
Each test prints the case it runs (flushed) before touching the GPU.
"""
import sys

import numpy as np
import pytest
import torch

from post_weight_quantization_30_amd import synth

pytestmark = pytest.mark.gpu

TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def awq():
    from post_weight_quantization_30_amd import awq as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


def stored(arr32, dt):
    """fp32 values -> storage array (numpy) and the exact fp32 values it holds."""
    st = synth.to_storage(arr32.astype(np.float64), dt)
    return st, synth.storage_to_f32(st, dt)


def bits_of(t, dt):
    a = t.cpu()
    if dt == "f32":
        return a.numpy().view(np.uint32)
    return a.view(torch.int16).numpy().view(np.uint16)


def want_bits(arr, dt):
    return arr.view(np.uint32) if dt == "f32" else arr


def values(r, shape):
    a = r.standard_normal(shape) * 0.02
    flat = a.reshape(-1)
    n = flat.size
    k = max(1, n // 50)
    flat[:k] = 0.0
    flat[k:2 * k] = -0.0
    flat[2 * k:3 * k] *= 1e-4            # fp16 subnormal results after the fold
    flat[3 * k:4 * k] *= 3e5             # fp16 overflow after division by a small s
    return a.astype(np.float32)


def scales(r, n):
    s = np.exp(r.uniform(-4, 4, n)).astype(np.float32)
    a = max(1, n // 20)
    b = max(a, n // 10)
    s[:a] = 1.0
    s[a:b] = 2.0 ** r.integers(-6, 7, b - a)
    return s


SHAPES = [(4096, 1), (4099, 1), (7, 1), (64, 4096), (37, 100), (16, 4104), (3, 8), (1, 1)]


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("rows,cols", SHAPES)
def test_fold_rows_bitwise(awq, ref, dt, rows, cols):
    say("fold rows", dt, rows, cols)
    r = np.random.default_rng(rows * 7 + cols)
    A_st, A32 = stored(values(r, (rows, cols)), dt)
    s = scales(r, rows)
    want = want_bits(ref.fold_rows(A32, s, dt), dt)
    Ad = awq.to_device(A_st, dt)
    sd = torch.from_numpy(s).cuda()
    got = awq.fold_rows(Ad.reshape(-1) if cols == 1 else Ad, sd)     # a vector, or a matrix
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(got, dt).reshape(rows, cols), want)
    # in place gives the same bits
    awq.fold_rows(Ad, sd, out=Ad)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(Ad, dt).reshape(rows, cols), want)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("rows,cols", [(64, 4096), (33, 512), (5, 100), (2, 8), (17, 1)])
def test_scale_cols_bitwise(awq, ref, dt, rows, cols):
    say("scale cols", dt, rows, cols)
    r = np.random.default_rng(rows * 11 + cols)
    W_st, W32 = stored(values(r, (rows, cols)), dt)
    s = scales(r, cols)
    want = want_bits(ref.scale_cols(W32, s, dt), dt)
    got = awq.scale_cols(awq.to_device(W_st, dt), torch.from_numpy(s).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(got, dt), want)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_fold_misaligned_buffers(awq, ref, dt):
    """Views starting one element into an allocation take the scalar path."""
    rows, cols = 24, 64
    say("fold misaligned", dt)
    r = np.random.default_rng(5)
    A_st, A32 = stored(values(r, (rows, cols)), dt)
    s = scales(r, rows)
    buf = torch.zeros(rows * cols + 1, dtype=TORCH[dt], device="cuda")
    flat = awq.to_device(A_st.reshape(-1), dt)
    buf[1:] = flat
    A = buf[1:].view(rows, cols)
    out_buf = torch.zeros_like(buf)
    out = out_buf[1:].view(rows, cols)
    awq.fold_rows(A, torch.from_numpy(s).cuda(), out=out)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(out, dt), want_bits(ref.fold_rows(A32, s, dt), dt))
    assert out_buf[0].item() == 0


def test_fold_refuses_mismatched_producer(awq, ref):
    """Grouped-query attention: v_proj has fewer output channels than o_proj has
    inputs, so it cannot absorb o_proj's scales."""
    v_proj = torch.zeros((1024, 4096), dtype=torch.float16, device="cuda")
    s = torch.ones(4096, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        awq.fold_rows(v_proj, s)


def test_folded_norm_and_packed_codes_reproduce_the_search_error(awq, ref):
    """gate/up-shaped layer fed by an RMSNorm: search s on X = norm(h) * gamma,
    fold 1/s into gamma, pack W diag(s). The deployed layer -- input
    norm(h) * gamma', weight dequantized from the codes -- has the output error
    the search reported for its choice (up to fp16 rounding of the folded input)."""
    r = np.random.default_rng(9)
    T, H, O = 256, 512, 1024
    h = r.standard_normal((T, H))
    h[:, r.permutation(H)[:8]] *= 20.0                  # a few outlier channels
    gamma = (1 + 0.2 * r.standard_normal(H)).astype(np.float16)
    nrm = h / np.sqrt((h * h).mean(axis=1, keepdims=True) + 1e-6)
    X = (nrm * gamma.astype(np.float64)).astype(np.float16)
    W = (r.standard_normal((O, H)) * 0.02).astype(np.float16)
    say("folded norm end to end")
    Xd, Wd = torch.from_numpy(X).cuda(), torch.from_numpy(W).cuda()
    res = awq.quantize_layer(Wd, Xd, bits=4, group=128, grid=20, mode="sym")
    g2 = awq.fold_rows(torch.from_numpy(gamma).cuda(), res["s_best"])
    torch.cuda.synchronize()
    best = int(res["best"].item())
    mse_best = float(res["mse"].cpu().numpy()[best])
    # deployed input: the same norm with the folded weight, stored as fp16
    Xf = (nrm * g2.cpu().numpy().astype(np.float64)).astype(np.float16).astype(np.float64)
    # deployed weight: scale * (code - zero) per group, unpacked on the host
    bits, g = 4, 128
    words = res["qweight"].cpu().numpy().view(np.uint32)
    codes = np.zeros((O, H), np.int64)
    for i in range(H):
        w, sh = divmod(i * bits, 32)
        codes[:, i] = (words[:, w] >> sh) & 0xF
    sc = np.repeat(res["scales"].cpu().numpy().astype(np.float64), g, axis=1)
    z = np.repeat(res["zeros"].cpu().numpy().astype(np.float64), g, axis=1)
    What = sc * (codes - z)
    y_dep = Xf @ What.T
    y_ref = X.astype(np.float64) @ W.astype(np.float64).T
    mse_dep = float(((y_dep - y_ref) ** 2).mean())
    assert abs(mse_dep - mse_best) <= 0.02 * mse_best, (mse_dep, mse_best)
    assert best > 0 and mse_best < float(res["mse"].cpu().numpy()[0])
    # folding the wrong way (multiplying gamma) is far off
    Xw = (nrm * (gamma.astype(np.float64) * res["s_best"].cpu().numpy())).astype(np.float64)
    assert ((Xw @ What.T - y_ref) ** 2).mean() > 10 * mse_best
