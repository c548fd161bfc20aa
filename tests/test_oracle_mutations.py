"""Planted mistakes in the CPU oracle must make its pins fail (CPU only).

Each case copies the oracle source, plants one plausible mistake (a dropped
term, a wrong sign, index, constant or rounding rule), builds the copy with
gcc and runs the pin tests against it in a subprocess. A case that still
passes every pin would mean the pins cannot see that part of the oracle.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "awq_oracle.c")

MUTATIONS = [
 ("stats drop guard", "xmag[j] = (float)(mean + 1e-8);", "xmag[j] = (float)(mean);"),
 ("stats T-1", "double mean = total / (double)tokens;", "double mean = total / (double)(tokens > 1 ? tokens - 1 : 1);"),
 ("alpha k/(grid+1)", "double alpha = (double)k / (double)grid;", "double alpha = (double)k / (double)(grid + 1);"),
 ("centre drop min", "double centre = sqrt(pmax * pmin);", "double centre = sqrt(pmax);"),
 ("sym levels", "const float levels = (float)((1 << (bits - 1)) - 1);", "const float levels = (float)((1 << (bits - 1)));"),
 ("sym round away", "float q = rintf(v[i] / scale);", "float q = roundf(v[i] / scale);"),
 ("asym zero sign", "float zero = rintf(-lo / scale);", "float zero = rintf(lo / scale);"),
 ("asym no zero in range", "if (lo > 0.0f) lo = 0.0f;", ";"),
 ("fq multiply", "wq[o * in + g0 + i] = (double)what[i] / (double)s[g0 + i];", "wq[o * in + g0 + i] = (double)what[i] * (double)s[g0 + i];"),
 ("err sign", "double e = y - ref[o * tokens + t];", "double e = y + ref[o * tokens + t];"),
 ("err index", "double e = y - ref[o * tokens + t];", "double e = y - ref[t * out + o];"),
 ("tie rule", "if (err < best_err) {", "if (err <= best_err) {"),
 ("pack shift", "rowq[word] |= c << shift;", "rowq[word] |= c << (32 - bits - shift);"),
 ("mse norm", "err = output_sse(x64, ref, wq, out, in, tokens, row, nthreads) /\n                     ((double)tokens * (double)out);", "err = output_sse(x64, ref, wq, out, in, tokens, row, nthreads) /\n                     ((double)tokens);"),
 ("v uses w only", "v[i] = W[o * in + g0 + i] * s[g0 + i];\n                    awq_ref_quant_group(v, group, bits, mode, NULL", "v[i] = W[o * in + g0 + i];\n                    awq_ref_quant_group(v, group, bits, mode, NULL"),
 ("sym clamp hi", "if (q > levels) q = levels;", "if (q > levels - 1.0f) q = levels - 1.0f;"),
 ("stats chunk reset", "double chunk = 0.0;", "double chunk = total;"),
 ("dot drops last", "for (int64_t i = 0; i < n; ++i)\n        acc += a[i] * b[i];", "for (int64_t i = 0; i + 1 < n; ++i)\n        acc += a[i] * b[i];"),
 ("asym dequant", "if (what) what[i] = scale * (q - zero);", "if (what) what[i] = scale * q;"),
 ("sym scale floor", "if (scale < 1e-8f) scale = 1e-8f;\n        for (int64_t i = 0; i < g; ++i) {\n            float q = rintf(v[i] / scale);\n            if (q < -levels", "for (int64_t i = 0; i < g; ++i) {\n            float q = rintf(v[i] / scale);\n            if (q < -levels"),
]
# Mistakes in the clipping-range search, checked against its own pins.
CLIP_MUTATIONS = [
 ("clip ratio i+1", "return (float)(1.0 - (double)i * (double)max_shrink / (double)n_clip);",
  "return (float)(1.0 - (double)(i + 1) * (double)max_shrink / (double)n_clip);"),
 ("clip err without 1/s", "d[j] = (double)what[j] / (double)s[g0 + j] - (double)W[o * in + g0 + j];",
  "d[j] = (double)what[j] - (double)W[o * in + g0 + j];"),
 ("clip sym range unscaled", "const float mx = ratio * amax;", "const float mx = amax;"),
 ("clip asym only hi", "lo = ratio * lo;", ";"),
 ("clip tie last", "if (e < best_e) {", "if (e <= best_e) {"),
 ("clip pack ignores clip", "if (clip)\n                awq_ref_quant_group_clip(", "if (0)\n                awq_ref_quant_group_clip("),
]


# Mistakes in the scale folding and the storage conversions.
FOLD_MUTATIONS = [
 ("fold multiplies", "store_one(out, r * cols + c, storage, A[r * cols + c] / s[r]);",
  "store_one(out, r * cols + c, storage, A[r * cols + c] * s[r]);"),
 ("fold column index", "store_one(out, r * cols + c, storage, A[r * cols + c] / s[r]);",
  "store_one(out, r * cols + c, storage, A[r * cols + c] / s[c % rows]);"),
 ("scale divides", "store_one(out, r * cols + c, storage, W[r * cols + c] * s[c]);",
  "store_one(out, r * cols + c, storage, W[r * cols + c] / s[c]);"),
 ("f16 truncates", "if (rem > half || (rem == half && (q & 1u)))\n        q += 1;",
  "if (0)\n        q += 1;"),
 ("f16 ties away", "if (rem > half || (rem == half && (q & 1u)))", "if (rem >= half)"),
 ("f16 flushes subnormals", "if (shift > 24)\n            return (uint16_t)sign;",
  "if (shift > 0)\n            return (uint16_t)sign;"),
 ("bf16 ties up", "if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))",
  "if (lower >= 0x8000u)"),
]

# Mistakes in the deployment product over the packed layout.
QGEMM_MUTATIONS = [
 ("unpack bit order", "code |= ((row[bit / 32] >> (bit % 32)) & 1u) << b;",
  "code |= ((row[bit / 32] >> (31 - bit % 32)) & 1u) << b;"),
 ("unpack stride", "const uint64_t bit = (uint64_t)k * (uint64_t)bits + (uint64_t)b;",
  "const uint64_t bit = (uint64_t)k * 4u + (uint64_t)b;"),
 ("qgemm no zero", "wd[k] = (double)scales[n * ngroups + g] * (code - (double)zeros[n * ngroups + g]);",
  "wd[k] = (double)scales[n * ngroups + g] * code;"),
 ("qgemm group index", "const int64_t g = k / group;", "const int64_t g = k % ngroups;"),
 ("qgemm scale transposed", "wd[k] = (double)scales[n * ngroups + g] *",
  "wd[k] = (double)scales[(g * out + n) % (out * ngroups)] *"),
]

# Mistakes in the GPTQ oracle (a Python module): run against its own pins.
GPTQ_SRC = os.path.join(ROOT, "oracle", "gptq_oracle.py")
GPTQ_MUTATIONS = [
 ("gptq no division by V_ii", "step = (w[i] - value) / V[i, i]", "step = (w[i] - value)"),
 ("gptq column of V", "w[i + 1:] = w[i + 1:] - step * V[i, i + 1:]",
  "w[i + 1:] = w[i + 1:] - step * V[i + 1:, i]"),
 ("gptq update sign", "w[i + 1:] = w[i + 1:] - step * V[i, i + 1:]",
  "w[i + 1:] = w[i + 1:] + step * V[i, i + 1:]"),
 ("gptq no elimination", "G[i + 1:, i + 1:] -= np.outer(G[i + 1:, i], G[i, i + 1:]) / pivot",
  "pass"),
 ("gptq unnormalised factor row", "V[i, i:] = G[i, i:] / np.sqrt(pivot)", "V[i, i:] = G[i, i:]"),
 ("gptq params on original weights", "sc, zr = group_params(w[None, cols.start:cols.stop], bits, mode)",
  "sc, zr = group_params(W0[r, None, cols.start:cols.stop], bits, mode)"),
 ("gptq absolute damping", "np.full(H.shape[0], damp * mean_diag)", "np.full(H.shape[0], damp)"),
 ("gptq zero sign", "zero = np.round(-lo / scale)", "zero = np.round(lo / scale)"),
]


@pytest.mark.parametrize("name,before,after", GPTQ_MUTATIONS, ids=[m[0] for m in GPTQ_MUTATIONS])
def test_planted_gptq_mistake_is_caught(tmp_path, name, before, after):
    src = open(GPTQ_SRC).read()
    assert before in src, f"pattern for '{name}' no longer in the GPTQ oracle"
    mutated = src.replace(before, after, 1)
    path = tmp_path / "gptq_oracle.py"
    path.write_text(mutated)
    env = dict(os.environ, AWQ_GPTQ_ORACLE=str(path))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_gptq_pins.py")],
                       env=env, capture_output=True, text=True, cwd=ROOT, timeout=600)
    assert r.returncode != 0, f"planted mistake '{name}' passed every pin:\n{r.stdout[-500:]}"


CASES = ([(n, b, a, "test_oracle_pins.py") for n, b, a in MUTATIONS] +
         [(n, b, a, "test_oracle_clip_pins.py") for n, b, a in CLIP_MUTATIONS] +
         [(n, b, a, "test_oracle_fold_pins.py") for n, b, a in FOLD_MUTATIONS] +
         [(n, b, a, "test_oracle_qgemm_pins.py") for n, b, a in QGEMM_MUTATIONS])


@pytest.mark.parametrize("name,before,after,pins", CASES, ids=[m[0] for m in CASES])
def test_planted_mistake_is_caught(tmp_path, name, before, after, pins):
    src = open(SRC).read()
    assert before in src, f"pattern for '{name}' no longer in the oracle source"
    (tmp_path / "awq_oracle.c").write_text(src.replace(before, after, 1))
    shutil.copy(os.path.join(ROOT, "oracle", "awq_oracle.h"), tmp_path / "awq_oracle.h")
    lib = tmp_path / "liboracle.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-o", str(lib), str(tmp_path / "awq_oracle.c"), "-lm"], check=True)
    env = dict(os.environ, AWQ_ORACLE_LIB=str(lib), OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", pins)],
                       env=env, capture_output=True, text=True, cwd=ROOT, timeout=600)
    assert r.returncode != 0, f"planted mistake '{name}' passed every pin:\n{r.stdout[-500:]}"
