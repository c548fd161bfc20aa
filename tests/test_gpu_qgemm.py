"""The deployment product Y = X Wd^T over the packed layout, GPU against the
oracle's exact fp64 value.

Bar, per output element (the kernel's arithmetic: code - zero exact in the
16-bit operand, products exact in fp32, at most one rounding per product in
the fp32 group sum, one per group when scaled into the total, 8 more for the
reduction over waves; u = 2^-24):
    |Y_gpu - Y| <= (group + ngroups + 8) u sum_k |X[m][k] Wd[n][k]|
plus half an ulp of the output type when Y is stored in 16 bits.
Each test prints the case it runs (flushed) before touching the GPU.
"""
import sys

import numpy as np
import pytest
import torch

from post_weight_quantization_30_amd import synth

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def awq():
    from post_weight_quantization_30_amd import awq as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


def abs_wd(q, sc, z, n_in, bits, group):
    """|Wd| for the error bound only (the expected values come from the oracle)."""
    words = q.view(np.uint32).astype(np.uint64)
    codes = np.zeros((q.shape[0], n_in), np.float64)
    for i in range(n_in):
        w, sh = divmod(i * bits, 32)
        codes[:, i] = ((words[:, w] >> np.uint64(sh)) & np.uint64((1 << bits) - 1)).astype(np.float64)
    scr = np.repeat(sc.astype(np.float64), group, axis=1)
    zr = np.repeat(z.astype(np.float64), group, axis=1)
    return np.abs(scr * (codes - zr))


def layer(ref, out, n_in, bits, group, mode, seed, dt):
    r = np.random.default_rng(seed)
    W = (r.standard_normal((out, n_in)) * 0.02).astype(np.float32)
    s = np.exp(r.uniform(-1.5, 1.5, n_in)).astype(np.float32)
    q, sc, z = ref.quantize_pack(W, s, bits, group, mode)
    return q, sc, z


def acts(M, n_in, dt, seed):
    r = np.random.default_rng(seed + 1)
    X = r.standard_normal((M, n_in))
    X[:, r.permutation(n_in)[: max(1, n_in // 100)]] *= 20.0
    st = synth.to_storage(X, dt)
    return st, synth.storage_to_f32(st, dt)


def check(Y_gpu, Y_ref, X32, q, sc, z, n_in, bits, group, y16_dtype=None, label=""):
    ng = n_in // group
    bound = (group + ng + 8) * U * (np.abs(X32.astype(np.float64)) @ abs_wd(q, sc, z, n_in, bits, group).T)
    if y16_dtype is not None:
        eps = 2.0 ** -11 if y16_dtype == "f16" else 2.0 ** -8
        bound = bound * (1 + eps) + eps * np.abs(Y_ref) + 2.0 ** -24   # half ulp (plus fp16 subnormal spacing)
    err = np.abs(Y_gpu.astype(np.float64) - Y_ref)
    say(label, "max err/bound", float((err / np.maximum(bound, 1e-300)).max()))
    assert np.all(err <= bound), f"{label}: {(err > bound).sum()} elements outside the bound"


def to_dev(awq, q, sc, z):
    return (torch.from_numpy(q.view(np.int32)).cuda(), torch.from_numpy(sc).cuda(),
            torch.from_numpy(z).cuda())


def y_numpy(Y, dt):
    if Y.dtype == torch.float32:
        return Y.cpu().numpy()
    if dt == "bf16":
        return Y.float().cpu().numpy()
    return Y.cpu().numpy().astype(np.float32)


CASES = [
    # (dt, bits, group, mode, M, out, in)
    ("f16", 4, 128, "sym", 1, 300, 512),
    ("f16", 4, 128, "asym", 5, 64, 1024),
    ("f16", 4, 128, "sym", 16, 48, 256),
    ("f16", 4, 128, "asym", 17, 40, 384),       # the 32-token x 64-row tile path, ragged tokens
    ("f16", 4, 64, "sym", 100, 33, 512),
    ("bf16", 4, 64, "asym", 3, 130, 512),
    ("bf16", 4, 32, "sym", 70, 20, 256),
    ("f16", 8, 32, "asym", 2, 64, 256),
    ("bf16", 8, 128, "sym", 33, 16, 640),
    ("bf16", 8, 64, "asym", 1, 1, 64),          # a single output row and token
    ("f16", 4, 128, "asym", 3, 8200, 256),      # tall layer: 32-row decode blocks, ragged rows
    ("bf16", 8, 64, "sym", 16, 8192, 128),
    # decode batches of four groups: a ragged last batch (5 groups), several
    # batches per wave (in = 14336: 28 batches over 8 waves; 8-bit g32: 36)
    ("f16", 4, 128, "asym", 4, 100, 640),
    ("bf16", 4, 128, "sym", 8, 40, 14336),
    ("f16", 8, 32, "sym", 1, 70, 4608),
    # the persistent decode grid walking several row tiles per block (the
    # register sets rotate across tile boundaries), the last tile moved back
    ("f16", 4, 128, "asym", 1, 40000, 1024),
    ("bf16", 4, 128, "sym", 2, 30001, 512),
    ("f16", 8, 64, "asym", 3, 20007, 1024),
    # the 64-token x 128-row prefill tile (at least 256 blocks, in a multiple of 128)
    ("bf16", 4, 128, "sym", 1000, 4000, 256),    # ragged token and row tiles
    ("f16", 8, 64, "asym", 1100, 3900, 128),
    # the 32 x 32 prefill tile with two 32-row tiles per wave (4-bit, group 128,
    # 512-row blocks): ragged token and row tiles in both input types
    ("bf16", 4, 128, "asym", 2100, 4100, 256),
    ("f16", 4, 128, "sym", 2050, 4097, 128),
    # one 32-row tile per wave (groups of 64), three K chunks, ragged edges
    ("bf16", 4, 64, "sym", 1030, 4100, 384),
    ("f16", 4, 32, "sym", 2048, 2048, 128),
    # more than 32 tokens, fewer blocks or in not a multiple of 128: the 32-token tile
    ("bf16", 4, 128, "sym", 200, 130, 1024),
    ("f16", 4, 32, "asym", 40, 50, 96),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("y_f32", [True, False])
def test_qgemm_matches_oracle(awq, ref, case, y_f32):
    dt, bits, group, mode, M, out, n_in = CASES[case]
    q, sc, z = layer(ref, out, n_in, bits, group, mode, 100 + case, dt)
    Xs, X32 = acts(M, n_in, dt, 200 + case)
    Y_ref = ref.qgemm(X32, q, sc, z, bits, group)
    say("qgemm", CASES[case], "y_f32" if y_f32 else "y16")
    Y = awq.qgemm(awq.to_device(Xs, dt), *to_dev(awq, q, sc, z), bits, group, y_f32=y_f32)
    torch.cuda.synchronize()
    check(y_numpy(Y, dt), Y_ref, X32, q, sc, z, n_in, bits, group, None if y_f32 else dt,
          f"{CASES[case]}")
    Y2 = awq.qgemm(awq.to_device(Xs, dt), *to_dev(awq, q, sc, z), bits, group, y_f32=y_f32)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2)                       # bitwise reproducible


@pytest.mark.parametrize("M", [1, 16, 256, 2048])
def test_qgemm_full_size_layer(awq, ref, M):
    """The 4096x4096 fp16 int4 g128 layer packed from its own search; sampled
    output rows against the oracle (all rows when M is small). 2048 tokens
    (the calibration tokens repeated) take the prefill tile."""
    spec = synth.HEADLINE
    lay = synth.make_layer(spec)
    say("qgemm full size", M)
    Wd = awq.to_device(lay["W"], spec.dtype)
    Xd = awq.to_device(lay["X"], spec.dtype)
    res = awq.quantize_layer(Wd, Xd, spec.bits, spec.group, spec.grid, spec.mode)
    Xin = awq.fold_rows(Xd.t().contiguous(), res["s_best"]).t().contiguous()       # X / s
    Xin = Xin.repeat((M + Xin.shape[0] - 1) // Xin.shape[0], 1)[:M].contiguous()
    Y = awq.qgemm(Xin, res["qweight"], res["scales"], res["zeros"], spec.bits, spec.group, y_f32=True)
    torch.cuda.synchronize()
    q = res["qweight"].cpu().numpy().view(np.uint32)
    sc, z = res["scales"].cpu().numpy(), res["zeros"].cpu().numpy()
    X32 = Xin.float().cpu().numpy()
    rows = np.arange(spec.out) if M <= 16 else np.r_[0:64, 2048:2112, 4032:4096]
    Y_ref = ref.qgemm(X32, q[rows], sc[rows], z[rows], spec.bits, spec.group)
    check(Y.cpu().numpy()[:, rows], Y_ref, X32, q[rows], sc[rows], z[rows], spec.inn, spec.bits,
          spec.group, None, f"full size M={M}")


def test_deployed_layer_reproduces_the_searched_error(awq, ref):
    """X / s through the packed weights reproduces the error the search
    measured for its choice: mean((qgemm(X / s) - X W^T)^2) = mse[best]."""
    spec = synth.with_shape(synth.HEADLINE, out=512, inn=1024, tokens=256)
    lay = synth.make_layer(spec)
    say("deployed layer", spec)
    Wd, Xd = awq.to_device(lay["W"], spec.dtype), awq.to_device(lay["X"], spec.dtype)
    res = awq.quantize_layer(Wd, Xd, spec.bits, spec.group, spec.grid, spec.mode)
    Xin = (Xd.float() / res["s_best"][None, :]).contiguous()          # fp32 X / s, then fp16
    Y = awq.qgemm(Xin.half(), res["qweight"], res["scales"], res["zeros"], spec.bits, spec.group,
                  y_f32=True)
    torch.cuda.synchronize()
    Xf = synth.storage_to_f32(lay["X"], spec.dtype).astype(np.float64)
    Wf = synth.storage_to_f32(lay["W"], spec.dtype).astype(np.float64)
    mse_dep = float(((Y.cpu().numpy().astype(np.float64) - Xf @ Wf.T) ** 2).mean())
    mse = res["mse"].cpu().numpy()
    best = int(res["best"].item())
    assert abs(mse_dep - mse[best]) <= 0.02 * mse[best], (mse_dep, mse[best])
