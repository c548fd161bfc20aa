"""Seeded synthetic layers for the AWQ scale search.

Draws a weight matrix W (out, in) and calibration activations X (tokens, in)
shaped like the layers on the pages: a 4096x4096 fp16 linear with 256 tokens
and 64 outlier channels scaled by 6 ("GPTQ and AWQ weight quantisation",
section "Setup: a linear layer and some calibration data"), and Llama-3-8B
shaped q/k/v, gate/up and down_proj layer groups ("AWQ vs GPTQ Quantization
Architectures Compared", "Worked example: an 8B model both ways"), with the
outlier fractions of "AWQ (activation-aware weight quantization)", "The idea"
(0.1-1 % of channels) and the 20-100x magnitudes of "Advanced Quantization
Algorithms: AWQ and GPTQ Explained", section 1.

This module holds none of the method's arithmetic: it only draws numbers and
converts storage formats. Both the oracle and the GPU library receive the
arrays it returns.

Recipe: numpy Philox bit generators, one independent stream each for W, X
and the channel selection (SeedSequence(seed).spawn(3)); normals and
Student-t draws in fp64; outlier and all-zero channels are the first n (then
the next n0) entries of one seeded permutation of range(in), n = round(frac*in);
values are formed in fp64 and rounded to the storage type (fp16 directly,
bf16 through fp32, both round-half-to-even).
"""
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class LayerSpec:
    name: str
    out: int
    inn: int
    tokens: int
    dtype: str                 # "f32" | "f16" | "bf16"
    bits: int
    group: int
    grid: int
    mode: str                  # "sym" | "asym"
    seed: int
    w_std: float = 0.02
    x_dist: str = "normal"     # "normal" | "student_t3"
    outlier_n: int = 0
    outlier_factor: tuple = ("const", 1.0)   # ("const", c) or ("loguniform", lo, hi)
    zero_n: int = 0
    note: str = field(default="", compare=False)

    @property
    def n_alpha(self):
        return self.grid + 1

    @property
    def alpha_macs(self):
        return self.n_alpha * self.tokens * self.out * self.inn


def _rnd(frac, n):
    return int(round(frac * n))


# The five workloads, in order: tiny, single linear (the headline), q/k/v group,
# gate/up group, wide-input down_proj.
CONFIGS = [
    LayerSpec("tiny_64x256_t32", 64, 256, 32, "f32", 4, 128, 20, "sym", 1000,
              outlier_n=4, outlier_factor=("const", 6.0)),
    LayerSpec("linear_4096x4096_t256", 4096, 4096, 256, "f16", 4, 128, 20, "sym", 1001,
              outlier_n=64, outlier_factor=("const", 6.0)),
    LayerSpec("qkv_12288x4096_t512", 12288, 4096, 512, "bf16", 4, 128, 20, "asym", 1002,
              outlier_n=_rnd(0.01, 4096), outlier_factor=("const", 20.0)),
    LayerSpec("gateup_28672x4096_t2048", 28672, 4096, 2048, "bf16", 4, 128, 20, "asym", 1003,
              x_dist="student_t3", outlier_n=_rnd(0.005, 4096),
              outlier_factor=("loguniform", 20.0, 100.0)),
    LayerSpec("down_4096x14336_t4096", 4096, 14336, 4096, "bf16", 3, 64, 40, "sym", 1004,
              outlier_n=_rnd(0.01, 14336), outlier_factor=("loguniform", 5.0, 100.0),
              zero_n=_rnd(0.001, 14336)),
]
BY_NAME = {c.name: c for c in CONFIGS}
HEADLINE = CONFIGS[1]


def with_shape(spec: LayerSpec, out=None, tokens=None, inn=None, seed=None, **kw) -> LayerSpec:
    """Same recipe at another size (outlier counts rescaled by the same fractions)."""
    inn2 = spec.inn if inn is None else inn
    scale_n = lambda n: n if inn is None else max(1 if n else 0, int(round(n * inn2 / spec.inn)))
    d = dict(spec.__dict__)
    d.update(out=spec.out if out is None else out,
             tokens=spec.tokens if tokens is None else tokens,
             inn=inn2,
             seed=spec.seed if seed is None else seed,
             outlier_n=scale_n(spec.outlier_n),
             zero_n=scale_n(spec.zero_n) if spec.zero_n else 0)
    d.update(kw)
    return LayerSpec(**d)


# ----------------------------------------------------------------------------
# storage formats
# ----------------------------------------------------------------------------
def f64_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 (RNE) -> bf16 (RNE), returned as uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_storage(a64: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(a64, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(a64, dtype=np.float16)
    if dtype == "bf16":
        return f64_to_bf16_bits(a64)
    raise ValueError(dtype)


def storage_to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of stored values to fp32 (what the oracle consumes)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a)
    return np.ascontiguousarray(a, dtype=np.float32)


# ----------------------------------------------------------------------------
# drawing
# ----------------------------------------------------------------------------
def _streams(seed):
    ss = np.random.SeedSequence(seed)
    return [np.random.Generator(np.random.Philox(s)) for s in ss.spawn(3)]


def draw_x64(spec: LayerSpec, rng_x, rng_c):
    if spec.x_dist == "normal":
        X = rng_x.standard_normal((spec.tokens, spec.inn))
    elif spec.x_dist == "student_t3":
        X = rng_x.standard_t(3, size=(spec.tokens, spec.inn))
    else:
        raise ValueError(spec.x_dist)
    perm = rng_c.permutation(spec.inn)
    outl = perm[: spec.outlier_n]
    zero = perm[spec.outlier_n: spec.outlier_n + spec.zero_n]
    kind = spec.outlier_factor[0]
    if spec.outlier_n:
        if kind == "const":
            fac = np.full(spec.outlier_n, float(spec.outlier_factor[1]))
        elif kind == "loguniform":
            lo, hi = spec.outlier_factor[1], spec.outlier_factor[2]
            fac = np.exp(rng_c.uniform(np.log(lo), np.log(hi), size=spec.outlier_n))
        else:
            raise ValueError(kind)
        X[:, outl] *= fac[None, :]
    if spec.zero_n:
        X[:, zero] = 0.0
    return X, outl, zero


def make_layer(spec: LayerSpec):
    """Returns dict(W, X) in storage format plus the outlier / zero channel lists."""
    rng_w, rng_x, rng_c = _streams(spec.seed)
    W = to_storage(rng_w.standard_normal((spec.out, spec.inn)) * spec.w_std, spec.dtype)
    X64, outl, zero = draw_x64(spec, rng_x, rng_c)
    X = to_storage(X64, spec.dtype)
    del X64
    return {"W": W, "X": X, "outliers": np.sort(outl), "zeros": np.sort(zero), "spec": spec}

