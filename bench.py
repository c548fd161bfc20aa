"""Benchmark of the AWQ per-layer scale search and pack on one MI355X.

One step = the whole path for one layer with its inputs resident in HBM:
activation statistics, candidate scales (with X's matrix-fragment copy in
the same launch), the fused error search over every alpha, the reduction
and argmin, and the final quantize-and-pack. The workload
is the 4096x4096 fp16 linear layer with 256 calibration tokens, int4
symmetric, group 128, grid 20 (21 alpha candidates), on seeded synthetic data.

Prints one JSON line. Timing: HIP events recorded on the stream the library
launches on (torch's current stream). `value` is alpha-candidate MACs per
second over K whole steps timed back to back; a second run of K steps with
events between the stages gives the per-stage times and the search kernel's
time for the roofline.
"""
import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_F16_TFLOPS = 2500.0       # MI355X dense fp16/bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0
METRIC = "AWQ search: α-candidate·MACs/s + ms per layer (4096×4096, 256 tok, g128, 21 α)"
SEARCH_SRC = os.path.join(ROOT, "post_weight_quantization_30_amd", "csrc", "k_search16.hip")
MFMA_PROBE = os.path.join(ROOT, "post_weight_quantization_30_amd", "mfma_peak")
PMC_FILE = os.path.join(ROOT, "profiles", "k_search16_linear_4096x4096_t256_hbm_counters.json")
CLIP_SRC = os.path.join(ROOT, "post_weight_quantization_30_amd", "csrc", "k_clip.hip")
CLIP_PMC_FILE = os.path.join(ROOT, "profiles", "k_clip_search_linear_4096x4096_t256_hbm_counters.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", default="linear_4096x4096_t256",
                   help="workload name (one of synth.CONFIGS)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--copy-calib", action="store_true",
                   help="also run a plain device copy of known size (HBM counter calibration)")
    p.add_argument("--no-launch-cost", action="store_true",
                   help="skip the search kernel's launch-cost record (other shapes of the same kernel)")
    p.add_argument("--no-mfma-peak", action="store_true",
                   help="skip the attainable-MFMA-peak probe")
    p.add_argument("--no-clip", action="store_true",
                   help="skip the clipping-range search measurement")
    p.add_argument("--no-gptq", action="store_true", help="skip the GPTQ measurement")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the per-workload records of the other layers")
    p.add_argument("--clip-steps", type=int, default=10,
                   help="timed launches of the clipping-range search")
    p.add_argument("--decode-only", action="store_true",
                   help="only the decode product on the 28672 x 4096 int4 g128 layer, hot and cold "
                        "(a short run for the profiler)")
    return p.parse_args()


def source_hash(path):
    """Hash of a kernel source's code: comments and blank lines left out, so a
    comment edit does not orphan counters taken from the same code."""
    import re
    with open(path) as f:
        text = f.read()
    text = re.sub(r"//[^\n]*", "", text)
    code = "\n".join(l.rstrip() for l in text.splitlines() if l.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def traffic_from_profile(config, pmc_file=PMC_FILE, src=SEARCH_SRC):
    """HBM bytes per launch of a kernel from committed rocprofv3 counters, or
    None when none are committed for this workload and the current kernel source."""
    if not os.path.exists(pmc_file):
        return None
    with open(pmc_file) as f:
        d = json.load(f)
    sha = d.get("source_sha256_16", d.get("k_search_source_sha256_16"))
    if d.get("config") != config or sha != source_hash(src):
        return None
    return d.get("hbm_bytes_per_launch")


def measured_mfma_peak():
    """Attainable dense 16x16x32 MFMA throughput from the standalone probe
    program (a child process; None if it is not built or fails)."""
    if not os.path.exists(MFMA_PROBE):
        return None
    try:
        r = subprocess.run([MFMA_PROBE], capture_output=True, text=True, timeout=120)
        return json.loads(r.stdout.strip().splitlines()[-1]) if r.returncode == 0 else None
    except (subprocess.SubprocessError, ValueError, IndexError):
        return None


def cpu_baseline(spec, lay, target_s):
    """The oracle as it stands, on the first R rows of the same layer (all tokens,
    all columns, every candidate), R grown until the run takes ~target_s.
    Returns the timing record and the oracle's results for the R rows."""
    import numpy as np
    from oracle import oracle as ref
    from post_weight_quantization_30_amd import synth
    Xf = synth.storage_to_f32(lay["X"], spec.dtype)
    cores = len(os.sched_getaffinity(0))
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    rows = 8
    while True:
        Wf = synth.storage_to_f32(lay["W"][:rows], spec.dtype)
        t0 = time.perf_counter()
        xmag = ref.act_stats(Xf)
        mse, best, s_best, _ = ref.search(Wf, Xf, xmag, spec.bits, spec.group, spec.grid, spec.mode)
        packed = ref.quantize_pack(Wf, s_best, spec.bits, spec.group, spec.mode)
        dt = time.perf_counter() - t0
        if dt >= target_s / 3 or rows >= spec.out:
            break
        rows = min(spec.out, int(rows * max(2.0, min(8.0, target_s / max(dt, 1e-3)))))
    macs = spec.n_alpha * spec.tokens * rows * spec.inn
    rec = {"value": macs / dt, "unit": "alpha-candidate MAC/s", "cores": threads, "kind": "oracle",
           "sample": f"{rows} of {spec.out} rows, all {spec.tokens} tokens and {spec.inn} columns, "
                     f"{spec.n_alpha} candidates; stats + search + pack; {dt:.2f} s"}
    return rec, {"rows": rows, "xmag": xmag, "mse": np.asarray(mse), "best": int(best),
                 "s_best": np.asarray(s_best, np.float32), "packed": packed}


MSE_RTOL = 1e-3


def parity_record(awq, torch, spec, W, X, xmag, full, o):
    """The GPU's results on the oracle's rows against the oracle's: statistics
    bitwise, every candidate error within 1e-3 relative, the same choice unless
    the oracle's errors at the two choices lie within 1e-3 relative, and the
    packed codes, scales and zeros bitwise for the oracle's s."""
    import numpy as np
    rows = o["rows"]
    if rows == spec.out:
        mse_g, best_g = full
    else:
        m, b, _ = awq.search(W[:rows].contiguous(), X, xmag, spec.bits, spec.group, spec.grid, spec.mode)
        mse_g, best_g = m.cpu().numpy(), int(b.item())
    mse_o, best_o = o["mse"], o["best"]
    rel = float(np.max(np.abs(mse_g - mse_o) / np.abs(mse_o)))
    same_choice = best_g == best_o or bool(mse_o[best_g] <= (1 + MSE_RTOL) * mse_o[best_o])
    s_o = torch.from_numpy(np.ascontiguousarray(o["s_best"])).to(W.device)
    q, sc, z = awq.quantize_pack(W[:rows].contiguous(), s_o, spec.bits, spec.group, spec.mode)
    q_o, sc_o, z_o = o["packed"]
    codes = (np.array_equal(q.cpu().numpy().view(np.uint32), q_o) and
             np.array_equal(sc.cpu().numpy(), sc_o) and np.array_equal(z.cpu().numpy(), z_o))
    stats = bool(np.array_equal(xmag.cpu().numpy(), o["xmag"]))
    ok = stats and rel <= MSE_RTOL and same_choice and codes
    return {"rows": rows, "of": spec.out, "xmag_bitwise": stats, "mse_max_rel_diff": rel,
            "best_gpu": best_g, "best_oracle": best_o, "same_choice": same_choice,
            "codes_scales_zeros_bitwise": codes, "pass": bool(ok)}


N_CLIP, MAX_SHRINK = 20, 0.5


def clip_measure(awq, torch, spec, W, X, s_best, args):
    """The clipping-range search on W diag(s_best) (the step after the alpha
    search) and the clipped pack: kernel times from HIP events on the launch
    stream, and the MFMA roofline of the search kernel. For 16-bit layers the
    kernel multiplies X by D split into 16-bit parts (two fp16 parts, three
    bf16 parts) on the 16-bit matrix cores: the roofline takes that dtype's
    peak with the algorithmic FLOP count, so at most 1/parts of it is
    reachable; `mfma_issued_frac` counts the parts."""
    out, n_in, T = spec.out, spec.inn, spec.tokens
    dev = W.device
    clip = torch.empty((out, n_in // spec.group), dtype=torch.float32, device=dev)
    sse = torch.empty((out, n_in // spec.group, N_CLIP), dtype=torch.float64, device=dev)
    qw = torch.empty((out, awq.words_per_row(n_in, spec.bits)), dtype=torch.int32, device=dev)
    sc = torch.empty((out, n_in // spec.group), dtype=torch.float32, device=dev)
    zr = torch.empty((out, n_in // spec.group), dtype=torch.uint8, device=dev)

    def search():
        awq.clip_search(W, X, s_best, spec.bits, spec.group, spec.mode, N_CLIP, MAX_SHRINK, clip=clip)

    def pack():
        awq.quantize_pack(W, s_best, spec.bits, spec.group, spec.mode, qw, sc, zr, clip=clip)

    def timed(fn, k):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(k):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / k

    for _ in range(2):
        search()
        pack()
    torch.cuda.synchronize()
    ms = timed(search, args.clip_steps)
    pack_ms = timed(pack, args.clip_steps)
    # the chosen ratios and their errors, for the record (untimed)
    awq.clip_search(W, X, s_best, spec.bits, spec.group, spec.mode, N_CLIP, MAX_SHRINK, clip=clip, sse=sse)
    torch.cuda.synchronize()
    e = sse.cpu()
    e_best = e.min(dim=-1).values
    macs = N_CLIP * T * out * n_in
    achieved = 2.0 * macs / (ms * 1e-3) / 1e12
    peak, parts = {"f16": (PEAK_F16_TFLOPS, 2), "bf16": (PEAK_F16_TFLOPS, 3)}.get(spec.dtype, (PEAK_F32_TFLOPS, 1))
    return {"n_clip": N_CLIP, "max_shrink": MAX_SHRINK, "ms": ms, "pack_ms": pack_ms,
            "ratio_macs_per_s": macs / (ms * 1e-3),
            "roofline": {"bound": "mfma", "kernel": "k_clip_search", "achieved": achieved,
                         "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
                         "mfma_parts": parts, "mfma_issued_frac": parts * achieved / peak,
                         "traffic": traffic_from_profile(spec.name, CLIP_PMC_FILE, CLIP_SRC)},
            "clipped_group_frac": float((clip < 1).float().mean().item()),
            "group_sse_vs_unclipped": float(e_best.sum() / e[..., 0].sum())}


def fold_measure(awq, torch, spec, W, s_best, args):
    """Folding s into the model: the previous linear layer's output rows / s
    (a producer of the headline layer's shape and dtype stands in for it), the
    layer's own columns * s, and a norm-weight vector. HBM roofline:
    read and write every element once, plus s."""
    out, n_in = spec.out, spec.inn
    esize = W.element_size()
    buf = torch.empty_like(W)
    # the producer has one output row per input channel of the layer
    prod = W if out == n_in else torch.ones((n_in, out), dtype=W.dtype, device=W.device)
    pbuf = buf if out == n_in else torch.empty_like(prod)
    gamma = torch.ones(n_in, dtype=W.dtype, device=W.device)
    gbuf = torch.empty_like(gamma)

    def timed(fn, k):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(k):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / k

    k = max(args.clip_steps, 10)
    rows_ms = timed(lambda: awq.fold_rows(prod, s_best, out=pbuf), k)
    cols_ms = timed(lambda: awq.scale_cols(W, s_best, out=buf), k)
    norm_ms = timed(lambda: awq.fold_rows(gamma, s_best, out=gbuf), k)
    nbytes = 2 * out * n_in * esize + 4 * n_in
    gbs = nbytes / (rows_ms * 1e-3) / 1e9
    return {"producer_shape": [n_in, out], "rows_ms": rows_ms, "cols_ms": cols_ms,
            "norm_vector_ms": norm_ms,
            "roofline": {"bound": "hbm", "kernel": "k_fold_vec (rows)", "achieved": gbs,
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                         "traffic": None},
            "cols_gbs": nbytes / (cols_ms * 1e-3) / 1e9}


def _graph_us(torch, launches, replays):
    """Average time of one launch, from a HIP graph of the given launches
    replayed back to back (the host's per-call overhead stays out)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for fn in launches:
            fn()
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (replays * len(launches))
    del g
    return us


COLD_BYTES = 600 * 2 ** 20      # > 2x the 256 MB last-level cache


def _decode_times(torch, awq, x, q, sc, z, bits, group, y, nbytes, replays):
    """Decode time with the packed weights read hot (the same copy every
    launch: after the first it is served from the last-level cache) and cold
    (launches rotate over copies totalling more than twice that cache, so
    every launch reads its weights from HBM). The cold one is the HBM figure."""
    hot = _graph_us(torch, [lambda: awq.qgemm(x, q, sc, z, bits, group, y=y)] * 20, replays)
    ncopy = max(2, COLD_BYTES // int(nbytes) + 1)
    copies = [(q.clone(), sc.clone(), z.clone()) for _ in range(ncopy)]
    cold = _graph_us(torch, [lambda c=c: awq.qgemm(x, c[0], c[1], c[2], bits, group, y=y) for c in copies],
                     max(1, replays // 3))
    del copies
    return hot, cold, ncopy


def qgemm_measure(awq, torch, spec, X, qweight, scales, zeros, s_best, args):
    """The deployment product over the layer's packed result: decode (1 and 16
    tokens, HBM-bound: the packed weights are read once), 256 tokens and a
    2048-token prefill (MFMA; the calibration tokens repeated). Launches are
    captured in a HIP graph so that the host's per-call overhead does not hide
    the kernel time; the graph's result is checked against an eager call.
    Decode is timed hot and cold (see _decode_times); its roofline uses the
    cold time."""
    out, n_in = spec.out, spec.inn
    Xin = (X.float() / s_best[None, :]).to(X.dtype).contiguous()      # 1/s folded upstream
    res = {}
    k = max(1, args.clip_steps // 2)
    for M in (1, 16, 256, 2048):
        xm = Xin.repeat((M + Xin.shape[0] - 1) // Xin.shape[0], 1)[:M].contiguous()
        y = torch.empty((M, out), dtype=X.dtype, device=X.device)
        awq.qgemm(xm, qweight, scales, zeros, spec.bits, spec.group, y=y)
        torch.cuda.synchronize()
        eager = y.clone()
        ng = n_in // spec.group
        nbytes = out * n_in * spec.bits / 8 + out * ng * 5 + M * n_in * 2 + M * out * 2
        flops = 2.0 * M * n_in * out
        rec = {}
        if M <= 16:
            us, cold, ncopy = _decode_times(torch, awq, xm, qweight, scales, zeros, spec.bits, spec.group, y,
                                            nbytes, k)
            gbs = nbytes / cold / 1e3
            rec = {"cold_us": cold, "cold_copies": ncopy, "hot_gbs": nbytes / us / 1e3}
            roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": gbs / PEAK_HBM_GBS, "traffic": None, "timing": "cold"}
        else:
            us = _graph_us(torch, [lambda: awq.qgemm(xm, qweight, scales, zeros, spec.bits, spec.group, y=y)] * 20,
                           k)
            gbs = nbytes / us / 1e3
            tfs = flops / us / 1e6
            roof = {"bound": "mfma", "achieved": tfs, "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                    "frac": tfs / PEAK_F16_TFLOPS, "traffic": None}
        if not torch.equal(y, eager):
            raise RuntimeError("qgemm graph replay differs from the eager result")
        res[f"M{M}"] = {"us": us, "bytes": nbytes, "gbs": nbytes / us / 1e3, "tflops": flops / us / 1e6,
                        **rec, "roofline": roof}
    res["M1_28672x4096"] = wide_decode(awq, torch, Xin[:1, :4096].to(torch.float16).contiguous())
    return res


def wide_decode(awq, torch, xw):
    """Decode on a wide layer (a gate/up-sized 28672 x 4096 int4 g128 stack,
    codes from a pack of seeded weights with s = 1): the transfer, not the
    launch and first round trip, dominates here."""
    wo, wi, gw = 28672, 4096, 128
    gen = torch.Generator(device=xw.device).manual_seed(7)
    Ww = (torch.randn((wo, wi), generator=gen, device=xw.device) * 0.02).to(torch.float16)
    qw, sw, zw = awq.quantize_pack(Ww, torch.ones(wi, dtype=torch.float32, device=xw.device), 4, gw, "sym")
    del Ww
    yw = torch.empty((1, wo), dtype=torch.float16, device=xw.device)
    nbytes = wo * wi / 2 + wo * (wi // gw) * 5 + wi * 2 + wo * 2
    us, cold, ncopy = _decode_times(torch, awq, xw, qw, sw, zw, 4, gw, yw, nbytes, 5)
    gbs = nbytes / cold / 1e3
    return {"us": us, "cold_us": cold, "cold_copies": ncopy, "bytes": nbytes, "gbs": nbytes / us / 1e3,
            "roofline": {"bound": "hbm", "kernel": "k_qgemv", "achieved": gbs, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS, "traffic": None, "timing": "cold"}}


def decode_only(awq, torch):
    gen = torch.Generator(device="cuda").manual_seed(3)
    xw = torch.randn((1, 4096), generator=gen, device="cuda").to(torch.float16)
    return {"workload": "qgemm decode, 28672 x 4096 int4 g128, 1 token", **wide_decode(awq, torch, xw)}


PEAK_F64_TFLOPS = 78.6          # MI355X fp64 matrix


def gptq_measure(awq, torch, spec, W, X, xmag_mse, args, awq_pack=None):
    """GPTQ on the same layer and quantizer (fp64 throughout): time per stage
    with HIP events, and the calibration error of its packed result next to
    RTN's and AWQ's (computed through the deployment product)."""
    out, n_in, T = spec.out, spec.inn, spec.tokens
    dev = W.device
    if n_in % 128 or spec.group not in (32, 64, 128) or spec.dtype == "f32":
        return None                      # outside the GPU GPTQ path or the fp16/bf16 product
    H = torch.empty((n_in, n_in), dtype=torch.float64, device=dev)
    U = torch.empty_like(H)
    wsf = torch.empty(awq.lib().awq_gptq_factor_workspace_size(n_in), dtype=torch.uint8, device=dev)
    wsq = torch.empty(awq.lib().awq_gptq_quantize_workspace_size(out, n_in), dtype=torch.uint8, device=dev)

    def run(ev=None):
        if ev: ev[0].record()
        awq.gptq_hessian(X, 0.01, H)
        if ev: ev[1].record()
        awq.gptq_factor(H, U, wsf)
        if ev: ev[2].record()
        res = awq.gptq_quantize(W, U, spec.bits, spec.group, spec.mode, wsq)
        if ev: ev[3].record()
        return res

    run()
    torch.cuda.synchronize()
    k = 5
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(k)]
    for e in evs:
        q, sc, z = run(e)
    torch.cuda.synchronize()
    st = {name: sorted(e[i].elapsed_time(e[i + 1]) for e in evs)[k // 2]
          for i, name in enumerate(("hessian", "factor", "quantize"))}
    total = sum(st.values())
    # calibration error of the packed result, through the deployment product (s = 1)
    y = awq.qgemm(X, q, sc, z, spec.bits, spec.group, y_f32=True)
    ref = X.float() @ W.float().t()
    mse = float(((y - ref) ** 2).mean())
    # held-out tokens of the same recipe (same outlier channels, a new activation
    # stream): RTN, AWQ (X / s through its packed weights) and GPTQ side by side
    import numpy as np
    from post_weight_quantization_30_amd import synth
    _, _, rng_c = synth._streams(spec.seed)
    rng_x2 = np.random.Generator(np.random.Philox(np.random.SeedSequence(spec.seed + 10_000)))
    X2_64, _, _ = synth.draw_x64(spec, rng_x2, rng_c)
    X2 = awq.to_device(synth.to_storage(X2_64, spec.dtype), spec.dtype)
    ref2 = X2.float() @ W.float().t()
    ones = torch.ones(n_in, dtype=torch.float32, device=dev)
    qr, sr, zr = awq.quantize_pack(W, ones, spec.bits, spec.group, spec.mode)
    held = {"rtn": float(((awq.qgemm(X2, qr, sr, zr, spec.bits, spec.group, y_f32=True) - ref2) ** 2).mean()),
            "gptq": float(((awq.qgemm(X2, q, sc, z, spec.bits, spec.group, y_f32=True) - ref2) ** 2).mean())}
    if awq_pack is not None:
        qa, sa, za, s_best = awq_pack
        X2s = (X2.float() / s_best[None, :]).to(X2.dtype).contiguous()
        held["awq"] = float(((awq.qgemm(X2s, qa, sa, za, spec.bits, spec.group, y_f32=True) - ref2) ** 2).mean())
    # algorithmic FLOPs: H is symmetric (one triangle, T in (in + 1)); a
    # Cholesky factor and a triangular inverse take in^3 / 3 each; the
    # compensation products sum out * (in - j) * 2 over the columns j
    flops = {"hessian": 1.0 * T * n_in * (n_in + 1),
             "factor": 2.0 * (n_in ** 3) / 3,
             "quantize": 1.0 * out * n_in * n_in}
    tf = {s: flops[s] / (st[s] * 1e-3) / 1e12 for s in st}
    return {"ms": total, "stages_ms": st, "tflops": tf,
            "roofline": {"bound": "mfma", "kernel": "GPTQ quantize stage (k_dgemm f64 + k_gptq_block)",
                         "achieved": tf["quantize"], "peak": PEAK_F64_TFLOPS, "unit": "TFLOP/s",
                         "frac": tf["quantize"] / PEAK_F64_TFLOPS, "traffic": None},
            "calibration_mse": {"gptq": mse, "awq": xmag_mse[0], "rtn": xmag_mse[1]},
            "heldout_mse": held}


def search_launch_cost(awq, torch, reps=10):
    """The error kernel's fixed cost per launch: the search (fp16, int4 sym
    g128, 21 candidates, 256 tokens) at 128 and 4096 input columns (1 and 32
    pipeline steps of 128 columns) for 4096 and 2048 rows (two blocks per
    compute unit and one). t(1 step) - (t(32) - t(1)) / 31 is what a launch
    costs beyond its steps: block start-up (staging, the first tile build,
    X prefetch), the epilogue and the launch itself. Seeded synthetic
    layers (W ~ N(0, 0.02), X ~ N(0, 1))."""
    g = torch.Generator(device="cuda")
    g.manual_seed(1234)
    res = {}
    for out in (4096, 2048):
        t = {}
        for n_in in (128, 4096):
            W = (torch.randn(out, n_in, device="cuda", generator=g) * 0.02).half()
            X = torch.randn(256, n_in, device="cuda", generator=g).half()
            xmag = awq.act_stats(X)
            ws = torch.empty(awq.search_workspace_size(out, n_in, 256, 20), dtype=torch.uint8, device="cuda")
            awq.search_prepare(X, xmag, out, 20, ws)
            for _ in range(3):
                awq.search_candidates(W, X, 4, 128, 20, "sym", ws)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                awq.search_candidates(W, X, 4, 128, 20, "sym", ws)
            e1.record()
            torch.cuda.synchronize()
            t[n_in] = e0.elapsed_time(e1) * 1e3 / reps
        step = (t[4096] - t[128]) / 31
        res[f"out{out}"] = {"us_1_step": t[128], "us_32_steps": t[4096], "us_per_step": step,
                            "us_fixed": t[128] - step, "blocks_per_cu": out // 16 * 2 // 256}
    return res


def measure_layer(awq, torch, synth, spec, steps, warmup, probe, cold_reps=5):
    """One workload: `steps` whole-path steps back to back (statistics, the
    single-call search, the pack), the same work again as separate stages with
    events between them, and cold-cache statistics and pack. Returns the
    record and the tensors the other measurements reuse."""
    lay = synth.make_layer(spec)
    W = awq.to_device(lay["W"], spec.dtype)
    X = awq.to_device(lay["X"], spec.dtype)
    out, n_in, T, grid = spec.out, spec.inn, spec.tokens, spec.grid
    dev = W.device
    ws_s = torch.empty(awq.act_stats_workspace_size(T, n_in), dtype=torch.uint8, device=dev)
    ws = torch.empty(awq.search_workspace_size(out, n_in, T, grid), dtype=torch.uint8, device=dev)
    xmag = torch.empty(n_in, dtype=torch.float32, device=dev)
    mse = torch.empty(grid + 1, dtype=torch.float64, device=dev)
    best = torch.empty(1, dtype=torch.int32, device=dev)
    s_best = torch.empty(n_in, dtype=torch.float32, device=dev)
    qweight = torch.empty((out, awq.words_per_row(n_in, spec.bits)), dtype=torch.int32, device=dev)
    scales = torch.empty((out, n_in // spec.group), dtype=torch.float32, device=dev)
    zeros = torch.empty((out, n_in // spec.group), dtype=torch.uint8, device=dev)

    stages = ["stats", "prepare", "search", "finish", "pack"]

    def step():
        # The path as a user runs it: statistics, the single-call search
        # (preparation with X's fragment copy, error kernel, finish), the
        # pack -- five launches back to back.
        awq.act_stats(X, xmag, ws_s)
        awq.search(W, X, xmag, spec.bits, spec.group, grid, spec.mode, mse, best, s_best, ws)
        awq.quantize_pack(W, s_best, spec.bits, spec.group, spec.mode, qweight, scales, zeros)

    def staged(ev):
        # The same work as separate stages, one launch each, with events
        # between them: the per-kernel times.
        ev[0].record()
        awq.act_stats(X, xmag, ws_s)
        ev[1].record()
        awq.search_prepare(X, xmag, out, grid, ws)
        ev[2].record()
        awq.search_candidates(W, X, spec.bits, spec.group, grid, spec.mode, ws)
        ev[3].record()
        awq.search_finish(out, n_in, T, grid, mse, best, s_best, ws)
        ev[4].record()
        awq.quantize_pack(W, s_best, spec.bits, spec.group, spec.mode, qweight, scales, zeros)
        ev[5].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K whole steps back to back, one event pair around them.
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record()
    for _ in range(steps):
        step()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = t_start.elapsed_time(t_end) / steps

    # Stage breakdown (and the search kernel's time for the roofline): the
    # same K steps again with events between the stages.
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    for k in range(steps):
        staged(events[k])
    torch.cuda.synchronize()
    per = {s: [] for s in stages}
    for ev in events:
        for i, s in enumerate(stages):
            per[s].append(ev[i].elapsed_time(ev[i + 1]))
    avg = {s: sum(v) / len(v) for s, v in per.items()}

    # Cold-cache statistics and pack: a 512 MiB write before each launch
    # evicts X and W from the 256 MiB Infinity Cache.
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = {"stats": [], "pack": []}
    for r in range(cold_reps):
        for name, fn in (("stats", lambda: awq.act_stats(X, xmag, ws_s)),
                         ("pack", lambda: awq.quantize_pack(W, s_best, spec.bits, spec.group, spec.mode,
                                                            qweight, scales, zeros))):
            flush.fill_(r)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            cold[name].append(e0.elapsed_time(e1))
    del flush
    cold_ms = {k: sorted(v)[len(v) // 2] for k, v in cold.items()}

    alpha_macs = spec.alpha_macs
    search_flops = 2.0 * alpha_macs
    fp32_ops = spec.dtype == "f32" or out < 256 or T < 16
    peak = PEAK_F32_TFLOPS if fp32_ops else PEAK_F16_TFLOPS
    achieved = search_flops / (avg["search"] * 1e-3) / 1e12
    measured = None
    if probe and not fp32_ops:
        measured = probe["mfma_16x16x32_f16_tflops" if spec.dtype == "f16" else "mfma_16x16x32_bf16_tflops"]
    esize = {"f32": 4, "f16": 2, "bf16": 2}[spec.dtype]
    stats_bytes = T * n_in * esize + 4 * n_in
    pack_bytes = out * n_in * esize + 4 * n_in + out * n_in * spec.bits / 8 + 5 * out * (n_in // spec.group)
    m = mse.cpu().numpy()
    b = int(best.item())
    core = {
        "ms_per_layer": ms_per_step,
        "wall_ms_per_layer": wall * 1e3 / steps,
        "alpha_macs_per_s": alpha_macs / (ms_per_step * 1e-3),
        "stages_ms": avg,
        "search_alpha_macs_per_s": alpha_macs / (avg["search"] * 1e-3),
        "roofline": {"bound": "mfma", "kernel": "k_search16" if not fp32_ops else "k_search",
                     "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
                     "peak_measured": measured,
                     "frac_of_measured": achieved / measured if measured else None},
        "stats_gbs": stats_bytes / (avg["stats"] * 1e-3) / 1e9,
        "pack_gbs": pack_bytes / (avg["pack"] * 1e-3) / 1e9,
        "stats_gbs_cold": stats_bytes / (cold_ms["stats"] * 1e-3) / 1e9,
        "pack_gbs_cold": pack_bytes / (cold_ms["pack"] * 1e-3) / 1e9,
        "result": {"best_index": b, "best_alpha": b / grid if b >= 0 else None,
                   "awq_mse": float(m[b]) if b >= 0 else None, "rtn_mse": float(m[0])},
    }
    tensors = {"lay": lay, "W": W, "X": X, "xmag": xmag, "s_best": s_best, "qweight": qweight,
               "scales": scales, "zeros": zeros, "mse": m, "best": b}
    return core, tensors


def oracle_rate(spec, lay, rows):
    """The oracle on the first `rows` rows of the layer: the statistics over
    all of X (timed on their own), then the search and the pack of those
    rows; the alpha-candidate MAC/s of the search and pack, and the whole
    layer's oracle time at that rate plus the statistics."""
    from oracle import oracle as ref
    from post_weight_quantization_30_amd import synth
    Xf = synth.storage_to_f32(lay["X"], spec.dtype)
    Wf = synth.storage_to_f32(lay["W"][:rows], spec.dtype)
    t0 = time.perf_counter()
    xmag = ref.act_stats(Xf)
    t1 = time.perf_counter()
    _, _, s_best, _ = ref.search(Wf, Xf, xmag, spec.bits, spec.group, spec.grid, spec.mode)
    ref.quantize_pack(Wf, s_best, spec.bits, spec.group, spec.mode)
    dt = time.perf_counter() - t1
    rate = spec.n_alpha * spec.tokens * rows * spec.inn / dt
    return {"alpha_macs_per_s": rate, "rows": rows, "stats_seconds": t1 - t0, "search_pack_seconds": dt,
            "layer_seconds_at_rate": (t1 - t0) + spec.alpha_macs / rate}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the AWQ search of one layer is measured on a "
              "single MI355X; several GPUs would each search their own rows of the layer "
              "(the row blocks are independent), which this measurement does not run.",
              file=sys.stderr)
        sys.exit(2)

    if args.decode_only:
        import torch
        from post_weight_quantization_30_amd import awq
        torch.cuda.set_device(0)
        print(json.dumps(decode_only(awq, torch)), flush=True)
        return

    probe = None if args.no_mfma_peak else measured_mfma_peak()

    import torch
    from post_weight_quantization_30_amd import awq, synth

    spec = synth.BY_NAME[args.config]
    torch.cuda.set_device(0)
    core, t = measure_layer(awq, torch, synth, spec, args.steps, args.warmup, probe)
    lay, W, X, xmag, s_best, qweight, scales, zeros, m, b = (t[k] for k in (
        "lay", "W", "X", "xmag", "s_best", "qweight", "scales", "zeros", "mse", "best"))
    dev = W.device
    grid = spec.grid
    rec = {
        "metric": METRIC,
        "value": core["alpha_macs_per_s"],
        "unit": "alpha-candidate MAC/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": core["ms_per_layer"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if spec.dtype == "f16" else spec.dtype,
        "data": "synthetic",
        "config": {"workload": spec.name, "out": spec.out, "in": spec.inn, "tokens": spec.tokens,
                   "bits": spec.bits, "group": spec.group, "mode": spec.mode, "n_alpha": spec.n_alpha,
                   "input_dtype": spec.dtype, "parallelism": "single GPU"},
        "roofline": dict(core["roofline"], traffic=traffic_from_profile(spec.name)),
        "stages_ms": core["stages_ms"],
        "search_alpha_macs_per_s": core["search_alpha_macs_per_s"],
        "stats_gbs": core["stats_gbs"],
        "pack_gbs": core["pack_gbs"],
        "stats_gbs_cold": core["stats_gbs_cold"],
        "pack_gbs_cold": core["pack_gbs_cold"],
        "mfma_probe": probe,
        "wall_ms_per_step": core["wall_ms_per_layer"],
        "result": core["result"],
    }
    if not args.no_clip:
        rec["clip_search"] = clip_measure(awq, torch, spec, W, X, s_best, args)
    rec["fold"] = fold_measure(awq, torch, spec, W, s_best, args)
    if spec.dtype == "f16" and not args.no_launch_cost:
        rec["search_launch_cost"] = search_launch_cost(awq, torch)
    if spec.dtype in ("f16", "bf16") and spec.bits in (4, 8) and spec.group in (32, 64, 128):
        rec["qgemm"] = qgemm_measure(awq, torch, spec, X, qweight, scales, zeros, s_best, args)
    if not args.no_gptq:
        rec["gptq"] = gptq_measure(awq, torch, spec, W, X, (float(m[b]) if b >= 0 else None, float(m[0])),
                                   args, (qweight, scales, zeros, s_best)
                                   if spec.dtype in ("f16", "bf16") else None)
    if args.copy_calib:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        rec["copy_calib_bytes"] = src.numel()
    if not args.no_configs:
        # The other workloads: a few steps each (a config is a layer, its
        # time scales with its alpha-candidate MACs), and the oracle's rate
        # on a row sample of the same layer.
        rec["configs"] = {}
        for other in synth.CONFIGS:
            if other.name == spec.name:
                continue
            n = 3 if other.alpha_macs > 1e12 else 10
            c, tt = measure_layer(awq, torch, synth, other, n, 2, probe, cold_reps=3)
            c["steps"] = n
            if not args.no_cpu_baseline:
                c["oracle"] = oracle_rate(other, tt["lay"], min(other.out, 64))
            rec["configs"][other.name] = c
            del tt
            torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        rec["cpu_baseline"], o = cpu_baseline(spec, lay, args.cpu_seconds)
        rec["parity"] = parity_record(awq, torch, spec, W, X, xmag, (m, b), o)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
