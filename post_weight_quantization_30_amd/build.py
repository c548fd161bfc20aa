"""Builds libawq.so (hand-written HIP kernels for gfx950 + the C ABI) in-tree.

hipcc flags: gfx950 only; -O3; -ffp-contract=off (the exact quantizer and the
fixed-order fp64 sums must not be contracted; the search kernel asks for its
fused multiply-adds explicitly); packed fp32 instructions disabled on the
device side.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libawq.so")
SOURCES = ["abi.hip", "k_stats.hip", "k_search.hip", "k_pack.hip", "k_clip.hip", "k_fold.hip", "k_qgemm.hip", "k_gptq.hip"]
# k_search16.hip is compiled once per (operand type, group size), in parallel:
# (source, extra flags, object name).
VARIANTS = [("k_search16.hip", [f"-DAWQ_S16_T={t}", f"-DAWQ_S16_G={g}"], f"k_search16_{t}_g{g}.o")
            for t in ("f16", "bf16") for g in (32, 64, 128)]
# Standalone measurement programs: the attainable MFMA peak (bench.py runs
# it) and the microbenchmarks behind the kernel design (mb_gfx950).
PROBES = [("mfma_peak.hip", os.path.join(PKG, "mfma_peak")),
          ("mb_gfx950.hip", os.path.join(PKG, "mb_gfx950"))]
ARCH = "gfx950"

CFLAGS = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-ffp-contract=off",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}"]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(job, verbose):
    src, extra, objname = job if isinstance(job, tuple) else (job, [], os.path.splitext(job)[0] + ".o")
    obj = os.path.join(BUILD, objname)
    cmd = [_hipcc(), *CFLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    return obj, out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = VARIANTS + SOURCES   # the slowest first
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 8)) as ex:
        results = list(ex.map(lambda s: _compile(s, verbose), jobs))
    for _, out in results:
        if out and verbose:
            print(out)
    objs = [o for o, _ in results]
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", LIB + ".tmp", *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    for src, exe in PROBES:
        cmd = [_hipcc(), *[f for f in CFLAGS if f != "-fPIC"], os.path.join(CSRC, src), "-o", exe + ".tmp"]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}{r.stderr}")
        os.replace(exe + ".tmp", exe)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
