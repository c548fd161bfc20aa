"""A Llama-style block through the library on the GPU, step by step against
the oracle ("AWQ (activation-aware weight quantization)", "How it works"
step 5 and the transformer paragraph; "AWQ vs GPTQ Quantization
Architectures Compared", "AWQ: move the error away from what matters").

The block (fp16 storage, one attention head as wide as the model, as many
KV heads as query heads): four searches -- the stacked q/k/v on the
attention norm's output (s0), o_proj on the attention output (s3), the
stacked gate/up on the MLP norm's output (s1), down_proj on the MLP's hidden
activations (s2) -- then the folds: the attention norm absorbs 1/s0, the MLP
norm 1/s1, v_proj's rows 1/s3 and up_proj's rows 1/s2; the packs of W diag(s)
for all four; and the folded block run through awq_qgemm. Bars:
  * searches: every per-candidate error within 1e-3 relative of the oracle,
    the oracle's choice unless its errors at the two choices are that close,
    s_best bitwise;
  * folds and packs: bitwise;
  * each qgemm output against the oracle's fp64 product of the same packed
    weights and the same 16-bit input, within the kernel's rounding bound
    (test_gpu_qgemm.py): (group + ngroups + 8) 2^-24 sum_k |x_k w_k|.
A v_proj with fewer rows than o_proj has inputs (grouped-query attention)
cannot absorb o_proj's scales: the fold is refused.
Each test prints the case it runs (flushed) before touching the GPU.
"""
import sys

import numpy as np
import pytest
import torch

from post_weight_quantization_30_amd import synth

pytestmark = pytest.mark.gpu

H, I, T = 256, 512, 64
BITS, GROUP, GRID, MODE = 4, 128, 20, "sym"
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


def f16(a):
    """fp64 values rounded to fp16 storage, as fp32 numpy (exact)."""
    return np.asarray(a, np.float64).astype(np.float32).astype(np.float16).astype(np.float32)


def rmsnorm(h, gamma, eps=1e-6):
    h = np.asarray(h, np.float64)
    return h / np.sqrt((h * h).mean(axis=1, keepdims=True) + eps) * np.asarray(gamma, np.float64)[None, :]


def silu(x):
    return x / (1.0 + np.exp(-x))


def attention(Q, K, V):
    att = Q @ K.T / np.sqrt(Q.shape[1])
    att = np.exp(att - att.max(axis=1, keepdims=True))
    att /= att.sum(axis=1, keepdims=True)
    return att @ V


def gpu16(t):
    return torch.from_numpy(np.ascontiguousarray(t, np.float32)).cuda().half()


def from_bits16(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float32)


def check_search(awq, ref, W, X, label):
    say("block search", label, W.shape, X.shape)
    Wd, Xd = gpu16(W), gpu16(X)
    xmag_g = awq.act_stats(Xd)
    mse, best, sb = awq.search(Wd, Xd, xmag_g, BITS, GROUP, GRID, MODE)
    torch.cuda.synchronize()
    xmag_o = ref.act_stats(X)
    assert np.array_equal(xmag_g.cpu().numpy(), xmag_o), label
    mse_o, best_o, _, _ = ref.search(W, X, xmag_o, BITS, GROUP, GRID, MODE)
    stab = ref.s_table(xmag_o, GRID)
    m, b = mse.cpu().numpy(), int(best.item())
    rel = np.abs(m - mse_o) / np.abs(mse_o)
    assert np.all(rel <= 1e-3), (label, float(rel.max()))
    if b != best_o:
        assert mse_o[b] <= (1 + 1e-3) * mse_o[best_o], (label, b, best_o)
    s = sb.cpu().numpy()
    assert np.array_equal(s, stab[b]), label
    return s


def check_fold_rows(awq, ref, A, s, label):
    got = awq.fold_rows(gpu16(A), torch.from_numpy(s).cuda()).cpu().numpy()
    want = from_bits16(ref.fold_rows(A, s, "f16")).reshape(got.shape)
    assert np.array_equal(got.astype(np.float32), want), label
    return want


def check_pack(awq, ref, W, s, label):
    q, sc, z = awq.quantize_pack(gpu16(W), torch.from_numpy(s).cuda(), BITS, GROUP, MODE)
    torch.cuda.synchronize()
    q_o, sc_o, z_o = ref.quantize_pack(W, s, BITS, GROUP, MODE)
    assert np.array_equal(q.cpu().numpy().view(np.uint32), q_o), label
    assert np.array_equal(sc.cpu().numpy(), sc_o), label
    assert np.array_equal(z.cpu().numpy(), z_o), label
    return (q, sc, z), (q_o, sc_o, z_o)


def abs_wd(q, sc, z, n_in):
    words = q.astype(np.uint64)
    codes = np.zeros((q.shape[0], n_in), np.float64)
    for i in range(n_in):
        w, sh = divmod(i * BITS, 32)
        codes[:, i] = ((words[:, w] >> np.uint64(sh)) & np.uint64((1 << BITS) - 1)).astype(np.float64)
    return np.abs(np.repeat(sc.astype(np.float64), GROUP, 1) * (codes - np.repeat(z.astype(np.float64), GROUP, 1)))


def check_qgemm(awq, ref, X, packed_g, packed_o, label):
    q, sc, z = packed_g
    say("block qgemm", label, X.shape)
    Y = awq.qgemm(gpu16(X), q, sc, z, BITS, GROUP, y_f32=True).cpu().numpy().astype(np.float64)
    Yo = ref.qgemm(X, *packed_o, BITS, GROUP)
    n_in = X.shape[1]
    bound = (GROUP + n_in // GROUP + 8) * U * (np.abs(X.astype(np.float64)) @ abs_wd(packed_o[0], packed_o[1], packed_o[2], n_in).T)
    assert np.all(np.abs(Y - Yo) <= bound + 1e-30), (label, float(np.max(np.abs(Y - Yo) - bound)))
    return Yo


def test_llama_block_through_the_library(awq, ref):
    r = np.random.default_rng(11)
    h = f16(r.standard_normal((T, H)))
    h[:, r.permutation(H)[:4]] *= 8.0                      # a few outlier channels
    h = f16(h)
    g_attn, g_mlp = (f16(1 + 0.1 * r.standard_normal(H)) for _ in range(2))
    Wq, Wk, Wv, Wo = (f16(r.standard_normal((H, H)) * 0.05) for _ in range(4))
    Wg, Wu = (f16(r.standard_normal((I, H)) * 0.05) for _ in range(2))
    Wd = f16(r.standard_normal((H, I)) * 0.05)

    # calibration inputs of the four searches (the unquantized block, fp16 storage)
    X0 = f16(rmsnorm(h, g_attn))
    Q, K, V = (X0.astype(np.float64) @ W.T.astype(np.float64) for W in (Wq, Wk, Wv))
    X3 = f16(attention(Q, K, V))
    x1 = h + X3.astype(np.float64) @ Wo.T.astype(np.float64)
    X1 = f16(rmsnorm(x1, g_mlp))
    X2 = f16(silu(X1.astype(np.float64) @ Wg.T) * (X1.astype(np.float64) @ Wu.T))

    s0 = check_search(awq, ref, np.vstack([Wq, Wk, Wv]), X0, "q/k/v")
    s3 = check_search(awq, ref, Wo, X3, "o_proj")
    s1 = check_search(awq, ref, np.vstack([Wg, Wu]), X1, "gate/up")
    s2 = check_search(awq, ref, Wd, X2, "down_proj")

    # folds: norms, v_proj rows (o_proj's 1/s3), up_proj rows (down_proj's 1/s2)
    g_attn_f = check_fold_rows(awq, ref, g_attn, s0, "attention norm").ravel()
    g_mlp_f = check_fold_rows(awq, ref, g_mlp, s1, "MLP norm").ravel()
    Wv_f = check_fold_rows(awq, ref, Wv, s3, "v_proj rows")
    Wu_f = check_fold_rows(awq, ref, Wu, s2, "up_proj rows")

    # packs of W diag(s)
    p_qkv = check_pack(awq, ref, np.vstack([Wq, Wk, Wv_f]), s0, "q/k/v")
    p_o = check_pack(awq, ref, Wo, s3, "o_proj")
    p_gu = check_pack(awq, ref, np.vstack([Wg, Wu_f]), s1, "gate/up")
    p_d = check_pack(awq, ref, Wd, s2, "down_proj")

    # the folded, quantized block through awq_qgemm, each product against the oracle
    n_f = f16(rmsnorm(h, g_attn_f))                       # = n / s0 up to fp16 rounding
    QKV = check_qgemm(awq, ref, n_f, *p_qkv, "q/k/v")
    a_f = f16(attention(QKV[:, :H], QKV[:, H:2 * H], QKV[:, 2 * H:]))   # = attention out / s3
    x1_q = h + check_qgemm(awq, ref, a_f, *p_o, "o_proj")
    m_f = f16(rmsnorm(x1_q, g_mlp_f))                     # = m / s1
    GU = check_qgemm(awq, ref, m_f, *p_gu, "gate/up")
    z_f = f16(silu(GU[:, :I]) * GU[:, I:])                # = hidden / s2
    y_q = x1_q + check_qgemm(awq, ref, z_f, *p_d, "down_proj")

    # the quantized block stays near the original one (int4 with the folded scales)
    y = x1 + X2.astype(np.float64) @ Wd.T.astype(np.float64)
    assert np.all(np.isfinite(y_q))
    rel = np.linalg.norm(y_q - y) / np.linalg.norm(y)
    say("block output relative error", rel)
    assert rel < 0.1


def test_gqa_producer_is_refused(awq, ref):
    """Grouped-query attention: v_proj has fewer output rows than o_proj has
    inputs, so o_proj's per-input scales have no v_proj row to live in."""
    r = np.random.default_rng(12)
    Wv_gqa = gpu16(f16(r.standard_normal((H // 4, H)) * 0.05))
    s3 = torch.from_numpy(np.exp(r.uniform(-1, 1, H)).astype(np.float32)).cuda()
    say("GQA producer")
    with pytest.raises(ValueError):
        awq.fold_rows(Wv_gqa, s3)
