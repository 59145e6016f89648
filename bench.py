"""Benchmark of the KroQuant online activation quantizer on one MI355X.

One step = the streaming-stress workload: 57 back-to-back kq_quantize calls on
a bf16 activation X[18432 x 12288] (FLUX.1-schnell width, 4 x 4608 tokens),
alternating two input and two output buffer sets so that nothing is served
from the 256 MB Infinity Cache.  Throughput counts the algorithmic bytes of
the path, 2 B in + 0.5 B codes + 1/32 B scales per element (parameters, 23 KB
per call, excluded).  Inputs are resident in HBM before timing starts.

Prints one JSON line (rank 0).  Also reported in the same line: the other
KroQuant variants and the three comparison kernels on the same inputs, the
stream probe (the same traffic with no arithmetic: the ceiling of this access
pattern) with every kernel's share of it, the roofline position of the
dominant kernel, the CPU oracle's rate on every matrix (one thread and all
cores), and per-shape tables (median, min and max over repetitions).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "transform+MXFP4 quantize GB/s and % of MI355X HBM peak; Gelem/s per shape"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD public specification
BYTES_PER_ELEM = 2.0 + 0.5 + 1.0 / 32.0
CALLS = 57
ROUNDS = 7  # timed rounds per per-shape entry: median, min and max are over these
# sources of the default kernel (the block-per-lane butterfly) and its device helpers
KERNEL_SOURCES = ["kq_device.hpp", "kq_flat.hip"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "w4a4_diffusion_transformer_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def sha256_of(a) -> str:
    """SHA-256 of a host buffer's bytes (inputs are reported by hash, so that a
    run can be matched to the buffers it measured)."""
    import numpy as np
    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8).tobytes()).hexdigest()


def load_profile(kernel: str, workload: str) -> dict:
    """HBM bytes per launch (rocprofv3 counters) and the kernel-trace average of
    the committed summaries, if they were taken on the current kernel sources."""
    out = {}
    for key, fname in (("traffic_bytes_per_launch", f"traffic_{kernel}_{workload}.json"),
                       ("trace_avg_kernel_us", f"trace_{kernel}_{workload}.json")):
        try:
            with open(os.path.join(ROOT, "profiles", fname)) as f:
                t = json.load(f)
        except (OSError, ValueError):
            continue
        if t.get("kernel_source_hash") == kernel_source_hash():
            out[key] = t.get(key)
    return out


def cpu_info() -> dict:
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model}


def time_calls(torch, fn, argv, reps, rounds=ROUNDS):
    """Per-call seconds over `rounds` timed rounds of `reps` back-to-back calls
    (argv cycled), after >= 100 ms of warm-up calls: MI355X clocks drop while
    the GPU idles during input generation and take a while to come back."""
    n = len(argv)
    t_warm = time.perf_counter() + 0.1
    while time.perf_counter() < t_warm:
        for i in range(reps):
            assert fn(*argv[i % n]) == 0
        torch.cuda.synchronize()
    out = []
    for _ in range(rounds):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(reps):
            fn(*argv[i % n])
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) * 1e-3 / reps)
    return sorted(out)


def rate_entry(nbytes, nelem, secs, probe_sec=None):
    med = secs[len(secs) // 2]
    e = {"GBps": round(nbytes / med / 1e9, 1), "Gelem_s": round(nelem / med / 1e9, 1),
         "pct_peak": round(100 * nbytes / med / 1e9 / HBM_PEAK_GBS, 1), "us": round(med * 1e6, 2),
         "us_min": round(secs[0] * 1e6, 2), "us_max": round(secs[-1] * 1e6, 2)}
    if probe_sec:
        e["pct_of_probe"] = round(100 * probe_sec / med, 1)
    return e


def shape_table(kq, torch, np, synth, dev):
    """Every kernel on every matrix of the PixArt, SANA and FLUX workloads.

    Each matrix is copied enough times that one pass over the copies (inputs
    and outputs) exceeds 512 MB, twice the Infinity Cache, and calls cycle
    through the copies back to back on one stream; per call: the median,
    minimum and maximum over ROUNDS timed rounds.  The stream probe's time on
    the same copies gives each kernel's share of the access pattern's
    ceiling."""
    out = {}
    # plus the shard one GPU of an 8-way tensor-parallel FLUX.1-schnell MLP fc2 input would hold
    # (X2's 12288 channels split in eight 32-aligned slices: 4608 x 1536), same distribution as X2
    shard = synth.MatrixSpec("flux_x2_tp8_shard", 4608, 1536, 3, 3, synth.BASE_NORMAL, 0.005, 100.0, 1.0)
    for spec in [s_ for c in (1, 2, 3) for s_ in synth.CONFIGS[c]] + [shard]:
        X = synth.matrix(spec)
        P = synth.params(spec)
        m = synth.smooth_mult(X)
        T, d = spec.T, spec.d
        nbytes = BYTES_PER_ELEM * T * d
        copies = max(2, int(np.ceil(512e6 / nbytes)))
        X0 = torch.from_numpy(X.view(np.int16)).to(dev)
        Xs = [X0] + [X0.clone() for _ in range(copies - 1)]
        outs = [kq.alloc_outputs(X0) for _ in range(copies)]
        Pd = torch.from_numpy(P).to(dev)
        md = torch.from_numpy(m).to(dev)
        pstride = 0 if spec.shared_k else 15
        Kbf = torch.empty((P.shape[0], 3, 32, 32), dtype=torch.int16, device=dev)
        kq.kq_build_blocks(Pd, P.shape[0], None, Kbf, 3)
        # Calls go straight to the C ABI with pointers marshalled once: these kernels run
        # 6-40 us, so per-call host overhead must stay well below that for back-to-back
        # launches on the stream.
        L = kq.lib()
        stream = torch.cuda.current_stream().cuda_stream
        xs = [x.data_ptr() for x in Xs]
        os_ = [(c_.data_ptr(), s_.data_ptr()) for c_, s_ in outs]
        pp, mp, kp = Pd.data_ptr(), md.data_ptr(), Kbf.data_ptr()
        calls = {
            "stream_probe": (L.kq_stream_probe, lambda i: (xs[i], T, d, *os_[i], stream)),
            "kroquant": (L.kq_quantize_ex, lambda i: (xs[i], T, d, pp, pstride, None, kq.KQ_AUTO, *os_[i], stream)),
            "kroquant_mfma_otf": (L.kq_quantize_ex,
                                  lambda i: (xs[i], T, d, pp, pstride, None, kq.KQ_MFMA_OTF, *os_[i], stream)),
            "kroquant_mfma_dense": (L.kq_quantize_ex,
                                    lambda i: (xs[i], T, d, None, pstride, kp, kq.KQ_MFMA_DENSE, *os_[i], stream)),
        }
        if not spec.shared_k:
            calls["smoothquant"] = (L.kq_smooth_quantize, lambda i: (xs[i], T, d, mp, *os_[i], stream))
            calls["plain"] = (L.kq_mx_quantize, lambda i: (xs[i], T, d, *os_[i], stream))
            calls["hadamard32"] = (L.kq_hadamard_quantize, lambda i: (xs[i], T, d, *os_[i], stream))
        row = {"T": T, "d": d, "auto_variant": kq.variant_name(kq.kq_auto_variant(T, d, True, False)),
               "X_sha256": sha256_of(X), "params_sha256": sha256_of(P)}
        if not spec.shared_k:
            # kq_tune's record for this shape (K_params and the dense split both supplied), then
            # timed through KQ_AUTO on the cold copies
            tuned = kq.kq_tune(Xs[0], Pd, Kbf, *outs[0], reps=30)
            row["tuned_variant"] = kq.variant_name(tuned)
            calls["kroquant_tuned"] = (L.kq_quantize_ex,
                                       lambda i: (xs[i], T, d, pp, 15, kp, kq.KQ_AUTO, *os_[i], stream))
        probe = None
        for name, (fn, mk) in calls.items():
            argv = [mk(i) for i in range(copies)]
            secs = time_calls(torch, fn, argv, max(60, 4 * copies))
            if name == "stream_probe":
                probe = secs[len(secs) // 2]
            row[name] = rate_entry(nbytes, T * d, secs, probe)
        if "smoothquant" in row:
            row["kroquant_time_over_smoothquant_time"] = round(row["kroquant"]["us"] / row["smoothquant"]["us"], 3)
        out[spec.name] = row
        kq.kq_tune_reset()
        del Xs, outs
        print(f"# {spec.name}: " + ", ".join(f"{k} {v['GBps']}" for k, v in row.items() if isinstance(v, dict)),
              file=sys.stderr, flush=True)
    return out


def cpu_baseline(oracle, synth, X_stress, P_stress):
    """The oracle as it stands (plain single-threaded C, fp64) on the GPU machine's
    host cores: one full call per matrix of the PixArt, SANA and FLUX workloads
    and one of the stress matrix, on one thread and with the rows split across
    all the threads this box's share allows (the same C routine per thread)."""
    info = cpu_info()
    threads = max(1, min(16, os.cpu_count() or 1))
    per = {}
    total = {1: [0.0, 0.0], threads: [0.0, 0.0]}  # bytes, seconds
    mats = [(s.name, synth.matrix(s), synth.params(s), 0 if s.shared_k else 15)
            for c in (1, 2, 3) for s in synth.CONFIGS[c]]
    mats.append(("stress", X_stress, P_stress, 15))
    for name, X, P, pstride in mats:
        nbytes = BYTES_PER_ELEM * X.size
        e = {}
        for th in sorted(total):
            t0 = time.perf_counter()
            oracle.quantize_rows(oracle.KRON, X, P, pstride, threads=th)
            dt = time.perf_counter() - t0
            e[f"GBps_{th}_threads"] = round(nbytes / dt / 1e9, 4)
            total[th][0] += nbytes
            total[th][1] += dt
        per[name] = e
        print(f"# cpu oracle {name}: {e}", file=sys.stderr, flush=True)
    v = total[threads][0] / total[threads][1] / 1e9
    return {"value": round(v, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": (f"one full kq_quantize-equivalent call on each of the 8 matrices (PixArt, SANA, FLUX and "
                       f"stress), rows split over {threads} threads; {total[threads][1]:.1f} s on {threads} threads, "
                       f"{total[1][1]:.1f} s on one"),
            "single_thread_GBps": round(total[1][0] / total[1][1] / 1e9, 4),
            "nproc": info["nproc"], "cpu_model": info["cpu_model"], "per_matrix": per}


def adaln_table(kq, torch, np, synth, dev):
    """The fused AdaLN producer step + quantizer against the unfused pipeline.

    Unfused: a LayerNorm + modulation written as torch ops (fp32 math, one bf16
    tensor written back to HBM) followed by kq_quantize on that tensor.  Fused:
    kq_quantize_adaln on the raw activation with the row statistics.  The row
    statistics kernel is timed on its own and followed by the fused step on the
    same X (as a pipeline runs them: the second read of X may come from the
    Infinity Cache), and the fused step also on the MFMA kernel (mfma_otf).
    Inputs: FLUX.1-schnell width
    (one sample of 4608 tokens x 3072) and PixArt-Sigma width (2 x 4096 tokens
    x 1152), N(0,1) activations with 1% outlier channels, AdaLN vectors with 1%
    amplified channels."""
    out = {}
    for name, T, d, tps in (("flux_x1", 4608, 3072, 4608), ("pixart_x1", 8192, 1152, 4096)):
        X = synth.random_matrix(T, d, seed=41, n_outliers=d // 100, mult=50.0, token_sigma=0.5)
        P = synth.random_params(d // 32, seed=42)
        ns = (T + tps - 1) // tps
        sc, sh = synth.adaln_vectors(ns, d, seed=43)
        nbytes = BYTES_PER_ELEM * T * d
        copies = max(2, int(np.ceil(512e6 / nbytes)))
        X0 = torch.from_numpy(X.view(np.int16)).to(dev)
        Xs = [X0] + [X0.clone() for _ in range(copies - 1)]
        outs = [kq.alloc_outputs(X0) for _ in range(copies)]
        Pd = torch.from_numpy(P).to(dev)
        scd = torch.from_numpy(sc).to(dev)
        shd = torch.from_numpy(sh).to(dev)
        sts = [torch.empty((T, 2), dtype=torch.float32, device=dev) for _ in range(copies)]
        for i in range(copies):
            kq.kq_row_stats(Xs[i], 1e-6, sts[i])
        L = kq.lib()
        stream = torch.cuda.current_stream().cuda_stream
        xs = [x.data_ptr() for x in Xs]
        ops = [(c_.data_ptr(), s_.data_ptr()) for c_, s_ in outs]
        stp = [s_.data_ptr() for s_ in sts]
        rep_sc = scd.repeat_interleave(tps, 0)[:T]
        rep_sh = shd.repeat_interleave(tps, 0)[:T]

        def fused(i):
            return L.kq_quantize_adaln(xs[i], T, d, stp[i], scd.data_ptr(), shd.data_ptr(), tps, Pd.data_ptr(), 15,
                                       None, kq.KQ_AUTO, *ops[i], stream)

        def fused_otf(i):
            return L.kq_quantize_adaln(xs[i], T, d, stp[i], scd.data_ptr(), shd.data_ptr(), tps, Pd.data_ptr(), 15,
                                       None, kq.KQ_MFMA_OTF, *ops[i], stream)

        def stats(i):
            return L.kq_row_stats(xs[i], T, d, 1e-6, stp[i], stream)

        def stats_then_fused(i):  # the producer step as a pipeline runs it: both kernels on one X
            rc = L.kq_row_stats(xs[i], T, d, 1e-6, stp[i], stream)
            return rc or fused(i)

        def unfused(i):
            st = sts[i]
            xm = ((Xs[i].view(torch.bfloat16).float() - st[:, :1]) * st[:, 1:] * (1.0 + rep_sc) + rep_sh).to(torch.bfloat16)
            return L.kq_quantize_ex(xm.data_ptr(), T, d, Pd.data_ptr(), 15, None, kq.KQ_AUTO, *ops[i], stream)

        row = {"T": T, "d": d, "tokens_per_sample": tps, "X_sha256": sha256_of(X), "params_sha256": sha256_of(P),
               "scale_sha256": sha256_of(sc), "shift_sha256": sha256_of(sh)}
        for label, fn in (("fused_quantize_adaln", fused), ("fused_quantize_adaln_mfma_otf", fused_otf), ("row_stats", stats),
                          ("row_stats_then_fused_quantize_adaln", stats_then_fused),
                          ("unfused_torch_eager_modulate_then_quantize", unfused)):
            secs = time_calls(torch, fn, [(i,) for i in range(copies)], max(60, 4 * copies))
            sec = secs[len(secs) // 2]
            row[label] = {"us": round(sec * 1e6, 2), "us_min": round(secs[0] * 1e6, 2), "us_max": round(secs[-1] * 1e6, 2)}
            if label.startswith("fused_quantize_adaln"):
                fb = nbytes + 8 * T
                row[label].update({"GBps": round(fb / sec / 1e9, 1), "pct_peak": round(100 * fb / sec / 1e9 / HBM_PEAK_GBS, 1)})
            if label == "row_stats":
                rb = 2 * T * d + 8 * T
                row[label].update({"GBps": round(rb / sec / 1e9, 1)})
        row["unfused_over_fused_time"] = round(row["unfused_torch_eager_modulate_then_quantize"]["us"] / row["fused_quantize_adaln"]["us"], 3)
        # HBM bytes: fused = X read once + codes/scales + stats; an unfused pipeline with one ideal
        # producer kernel moves X in, X_mod out, then the quantizer's X_mod in + codes/scales
        row["algorithmic_bytes_fused"] = int(nbytes + 8 * T)
        row["algorithmic_bytes_unfused_min"] = int(nbytes + 4 * T * d + 8 * T)
        out[name] = row
        del Xs, outs
        print(f"# adaln {name}: " + json.dumps(row), file=sys.stderr, flush=True)
    return out


def gemm_table(kq, torch, np, dev):
    """The W4A4 consumer GEMM (kq_gemm_mx, MXFP4 x MXFP4 -> bf16) at DiT linear-layer shapes:
    FLUX.1-schnell MLP fc1 / fc2 and attention qkv at 4608 tokens, PixArt-Sigma MLP fc1 at 2 x 4096
    tokens.  Operands are random codes with scales in [2^-9, 2^6]; the time does not depend on values.
    TFLOP/s counts 2 M N K; the roofline peak is MI355X's dense FP4 figure, 10.1 PFLOP/s.
    Beside it, the ROCm library's MXFP4 GEMM on the same operands (hipBLASLt through
    torch._scaled_mm, E8M0 block scales, bf16 out), timed the same way, when this torch build
    offers it; the bf16 outputs of the two are compared too (largest difference in bf16 steps).
    And the bf16 GEMM of the same shape, the layer W4A4 replaces."""
    out = {}
    L = kq.lib()
    stream = torch.cuda.current_stream().cuda_stream
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    for name, M, N, K in (("flux_mlp_fc1", 4608, 12288, 3072), ("flux_mlp_fc2", 4608, 3072, 12288),
                          ("flux_attn_qkv", 4608, 9216, 3072), ("pixart_mlp_fc1", 8192, 4608, 1152)):
        a = torch.randint(0, 256, (M, K // 2), dtype=torch.uint8, device=dev, generator=g)
        asc = torch.randint(118, 134, (M, K // 32), dtype=torch.uint8, device=dev, generator=g)
        b = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device=dev, generator=g)
        bsc = torch.randint(118, 134, (N, K // 32), dtype=torch.uint8, device=dev, generator=g)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        args = (a.data_ptr(), asc.data_ptr(), M, b.data_ptr(), bsc.data_ptr(), N, K, None, y.data_ptr(), stream)
        t_warm = time.perf_counter() + 0.1
        while time.perf_counter() < t_warm:
            for _ in range(5):
                assert L.kq_gemm_mx(*args) == 0
            torch.cuda.synchronize()
        reps = 20
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            L.kq_gemm_mx(*args)
        e1.record()
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) * 1e-3 / reps
        tf = 2.0 * M * N * K / sec / 1e12
        out[name] = {"M": M, "N": N, "K": K, "us": round(sec * 1e6, 1), "TFLOPs": round(tf, 1),
                     "frac_fp4_peak": round(tf / 10100.0, 4)}
        out[name]["hipblaslt_mxfp4"] = library_mxfp4(torch, a, asc, b, bsc, y, M, N, K, sec)
        out[name]["bf16_matmul"] = bf16_matmul(torch, dev, M, N, K, sec)
        print(f"# gemm {name}: {out[name]}", file=sys.stderr, flush=True)
    return out


def bf16_matmul(torch, dev, M, N, K, kq_sec):
    """The same layer in bf16 (what W4A4 replaces): torch.matmul of X [M][K] and the weight stored
    transposed and contiguous [K][N] (hipBLASLt), timed like the GEMM above."""
    x = torch.randn((M, K), dtype=torch.bfloat16, device=dev)
    wt = torch.randn((K, N), dtype=torch.bfloat16, device=dev).contiguous()
    yb = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    t_warm = time.perf_counter() + 0.1
    while time.perf_counter() < t_warm:
        torch.matmul(x, wt, out=yb)
        torch.cuda.synchronize()
    reps = 20
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.matmul(x, wt, out=yb)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / reps
    return {"us": round(sec * 1e6, 1), "TFLOPs": round(2.0 * M * N * K / sec / 1e12, 1),
            "kq_time_over_bf16_time": round(kq_sec / sec, 3)}


def library_mxfp4(torch, a, asc, b, bsc, y, M, N, K, kq_sec):
    """hipBLASLt's MXFP4 GEMM (torch._scaled_mm) on the same operands; None if this torch build lacks
    the FP4 types, {"us": None, "error": ...} if the library call fails or one call takes more than 20
    times this kernel's time (not retried, not timed)."""
    f4, e8 = getattr(torch, "float4_e2m1fn_x2", None), getattr(torch, "float8_e8m0fnu", None)
    if f4 is None or e8 is None:
        return None

    def call():
        return torch._scaled_mm(a.view(f4), b.view(f4).t(), scale_a=asc.view(e8), scale_b=bsc.view(e8),
                                out_dtype=torch.bfloat16)

    try:
        yl = call()
        torch.cuda.synchronize()
        # bf16 steps between the two outputs (order-preserving integer map of the bf16 bit patterns)
        def key(t):
            i = t.view(torch.int16).to(torch.int32)
            return torch.where(i < 0, -32768 - i, i)
        steps = int((key(yl) - key(y)).abs().max().item())
        # one call first: where the library takes far longer than this kernel (seconds per call
        # at some shapes on MI355X), the shape is not timed and no figure is reported for it
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        torch.cuda.synchronize()
        if e0.elapsed_time(e1) * 1e-3 > 20 * kq_sec:
            return {"us": None, "max_bf16_steps_apart": steps,
                    "error": "one call took more than 20 times this kernel's time; not timed"}
        t_warm = time.perf_counter() + 0.1
        while time.perf_counter() < t_warm:
            call()
            torch.cuda.synchronize()
        reps = 20
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            call()
        e1.record()
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) * 1e-3 / reps
        return {"us": round(sec * 1e6, 1), "TFLOPs": round(2.0 * M * N * K / sec / 1e12, 1),
                "kq_time_over_library_time": round(kq_sec / sec, 3), "max_bf16_steps_apart": steps,
                "reps": reps}
    except RuntimeError as e:
        # the library's failure is recorded as it is; this shape is not called again
        print(f"# hipBLASLt MXFP4 failed at {M}x{N}x{K}: {str(e)[:160]}", file=sys.stderr, flush=True)
        return {"us": None, "error": str(e)[:300]}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--variant", default="auto", choices=["auto", "mfma_dense", "mfma_otf", "butterfly"])
    ap.add_argument("--no-compare", action="store_true", help="skip the comparison kernels")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-shapes", action="store_true", help="skip the per-shape table of the other workloads")
    ap.add_argument("--no-adaln", action="store_true", help="skip the fused AdaLN producer-step table")
    ap.add_argument("--no-gemm", action="store_true", help="skip the W4A4 GEMM table")
    ap.add_argument("--profile-pass", action="store_true",
                    help="few launches of each kernel plus a plain copy of known size, for rocprofv3 counter runs")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the quantizer needs no communication and this build runs on a single "
              "MI355X; multi-GPU sharding is described in DESIGN.md, not run.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import w4a4_diffusion_transformer_amd as kq

    dev = torch.device("cuda:0")
    spec = synth.CONFIGS[4][0]
    T, d = spec.T, spec.d
    nb = d // 32
    n = T * d
    t0 = time.time()
    X = synth.matrix(spec)
    P = synth.params(spec)
    m = synth.smooth_mult(X)
    x_sha, p_sha = sha256_of(X), sha256_of(P)
    print(f"# generated {T}x{d} in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    Xs = [torch.from_numpy(X.view(np.int16)).to(dev)]
    Xs.append(Xs[0].clone())
    Pd = torch.from_numpy(P).to(dev)
    md = torch.from_numpy(m).to(dev)
    outs = [kq.alloc_outputs(Xs[0]) for _ in range(2)]
    Kbf = torch.empty((nb, 3, 32, 32), dtype=torch.int16, device=dev)
    kq.kq_build_blocks(Pd, nb, None, Kbf, 3)
    torch.cuda.synchronize()

    def kron(v):
        if v == kq.KQ_MFMA_DENSE:
            return lambda i: kq.kq_quantize_ex(Xs[i & 1], None, 15, Kbf, v, *outs[i & 1])
        if v == kq.KQ_AUTO:
            return lambda i: kq.kq_quantize(Xs[i & 1], Pd, *outs[i & 1])
        return lambda i: kq.kq_quantize_ex(Xs[i & 1], Pd, 15, None, v, *outs[i & 1])

    def step(call):
        for i in range(CALLS):
            call(i)

    def timed(call, steps, warmup):
        """(total ms over `steps` steps, sorted per-step ms): events around every step on the launch stream."""
        for _ in range(warmup):
            step(call)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record()
        for k in range(steps):
            step(call)
            ev[k + 1].record()
        torch.cuda.synchronize()
        per = sorted(ev[k].elapsed_time(ev[k + 1]) for k in range(steps))
        return ev[0].elapsed_time(ev[-1]), per

    main_v = kq.VARIANTS[args.variant]
    if args.profile_pass:
        for _ in range(3):
            kron(main_v)(0)
        for v in (kq.KQ_MFMA_DENSE, kq.KQ_MFMA_OTF, kq.KQ_BUTTERFLY):
            kron(v)(1)
        kq.kq_stream_probe(Xs[0], *outs[0])
        kq.kq_smooth_quantize(Xs[0], md, *outs[0])
        kq.kq_mx_quantize(Xs[0], *outs[0])
        kq.kq_hadamard_quantize(Xs[0], *outs[0])
        # the FLUX matrices once each with the default kernel and the SmoothQuant kernel
        for fs in synth.CONFIGS[3]:
            fx = torch.from_numpy(synth.matrix(fs).view(np.int16)).to(dev)
            fp = torch.from_numpy(synth.params(fs)).to(dev)
            fo = kq.alloc_outputs(fx)
            fm = torch.ones(fs.d, dtype=torch.float32, device=dev)
            kq.kq_quantize(fx, fp, *fo)
            kq.kq_smooth_quantize(fx, fm, *fo)
            kq.kq_quantize_ex(fx, fp, 15, None, kq.KQ_MFMA_OTF, *fo)
            del fx, fo
        # the AdaLN producer step at FLUX X1 (one sample) and PixArt X1 (two samples), the inputs of
        # the adaln table: row statistics, then the fused quantizer (default kernel)
        for at, ad, atps in ((4608, 3072, 4608), (8192, 1152, 4096)):
            ax = torch.from_numpy(synth.random_matrix(at, ad, seed=41, n_outliers=ad // 100, mult=50.0,
                                                      token_sigma=0.5).view(np.int16)).to(dev)
            ap = torch.from_numpy(synth.random_params(ad // 32, seed=42)).to(dev)
            asc, ash = synth.adaln_vectors((at + atps - 1) // atps, ad, seed=43)
            ast = torch.empty((at, 2), dtype=torch.float32, device=dev)
            ao = kq.alloc_outputs(ax)
            kq.kq_row_stats(ax, 1e-6, ast)
            kq.kq_quantize_adaln(ax, ast, torch.from_numpy(asc).to(dev), torch.from_numpy(ash).to(dev), atps, ap, *ao)
            del ax, ao
        # the W4A4 GEMM once at the FLUX MLP fc1 shape
        gm, gn, gk = 4608, 12288, 3072
        ga = torch.randint(0, 256, (gm, gk // 2), dtype=torch.uint8, device=dev)
        gas = torch.full((gm, gk // 32), 127, dtype=torch.uint8, device=dev)
        gb = torch.randint(0, 256, (gn, gk // 2), dtype=torch.uint8, device=dev)
        gbs = torch.full((gn, gk // 32), 127, dtype=torch.uint8, device=dev)
        gy = torch.empty((gm, gn), dtype=torch.bfloat16, device=dev)
        kq.kq_gemm_mx(ga, gas, gb, gbs, None, gy)
        del ga, gb, gy
        # plain copy kernel of known size for counter calibration: 1 GiB read + 1 GiB written
        a = torch.empty(1 << 29, dtype=torch.int16, device=dev).fill_(1)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"profile_pass": True, "copy_bytes": a.numel() * 2}))
        return

    ms, per_step = timed(kron(main_v), args.steps, args.warmup)
    ms_step = ms / args.steps
    bytes_call = BYTES_PER_ELEM * n
    gbs = bytes_call * CALLS * args.steps / (ms * 1e-3) / 1e9
    launch_us = ms * 1e3 / (args.steps * CALLS)
    print(f"# stress: {gbs:.1f} GB/s, {launch_us:.2f} us per launch", file=sys.stderr, flush=True)

    def leg(call, steps):
        t, per = timed(call, steps, 2)
        return {"GBps": round(bytes_call * CALLS * steps / (t * 1e-3) / 1e9, 1),
                "us": round(t * 1e3 / (steps * CALLS), 2),
                "us_min": round(per[0] * 1e3 / CALLS, 2), "us_max": round(per[-1] * 1e3 / CALLS, 2)}

    comparison = {}
    if not args.no_compare:
        k = max(5, args.steps // 2)
        comparison["stream_probe"] = leg(lambda i: kq.kq_stream_probe(Xs[i & 1], *outs[i & 1]), k)
        for name, v in (("mfma_dense", kq.KQ_MFMA_DENSE), ("mfma_otf", kq.KQ_MFMA_OTF),
                        ("butterfly", kq.KQ_BUTTERFLY)):
            comparison[f"kroquant_{name}"] = leg(kron(v), k)
        comparison["smoothquant_mxfp4"] = leg(lambda i: kq.kq_smooth_quantize(Xs[i & 1], md, *outs[i & 1]), k)
        comparison["plain_mxfp4"] = leg(lambda i: kq.kq_mx_quantize(Xs[i & 1], *outs[i & 1]), k)
        comparison["hadamard32_mxfp4"] = leg(lambda i: kq.kq_hadamard_quantize(Xs[i & 1], *outs[i & 1]), k)
        for hb in (64, 128, 256, 512):
            comparison[f"hadamard{hb}_mxfp4"] = leg(
                lambda i, hb=hb: kq.kq_hadamard_quantize_ex(Xs[i & 1], hb, *outs[i & 1]), k)
        probe_us = comparison["stream_probe"]["us"]
        for v in comparison.values():
            v["pct_of_probe"] = round(100 * probe_us / v["us"], 1)
        comparison["kroquant_time_over_smoothquant_time"] = round(launch_us / comparison["smoothquant_mxfp4"]["us"], 4)
        comparison["kroquant_pct_of_probe"] = round(100 * probe_us / launch_us, 1)
        comparison["pages_context"] = ("KroQuant quantizer up to 14% faster than the SmoothQuant kernel on an MI350 "
                                       "(Triton); another machine, context only")

    per_shape = None
    if not args.no_shapes:
        per_shape = shape_table(kq, torch, np, synth, dev)
    adaln = None
    if not args.no_adaln:
        adaln = adaln_table(kq, torch, np, synth, dev)
    gemm = None
    if not args.no_gemm:
        gemm = gemm_table(kq, torch, np, dev)
    cpu = None
    if not args.no_cpu:
        import oracle

        cpu = cpu_baseline(oracle, synth, X, P)

    variant_name = args.variant
    kernel = kq.variant_name(kq.kq_auto_variant(T, d, True, False)) if variant_name == "auto" else variant_name
    prof = load_profile(kernel, "stress")
    achieved = bytes_call / (launch_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": prof.get("traffic_bytes_per_launch"),
                "kernel": f"kq {kernel}", "avg_launch_us": round(launch_us, 2),
                "step_ms_median": round(per_step[len(per_step) // 2], 4), "step_ms_min": round(per_step[0], 4),
                "step_ms_max": round(per_step[-1], 4),
                "algorithmic_bytes_per_launch": int(bytes_call)}
    if prof.get("trace_avg_kernel_us"):
        roofline["trace_avg_kernel_us"] = prof["trace_avg_kernel_us"]
        roofline["frac_from_trace"] = round(bytes_call / (prof["trace_avg_kernel_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)

    out = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"stress: X[{T} x {d}] bf16 Student-t(3), 1% outlier channels x200, 1% zero blocks; "
                               f"{CALLS} back-to-back kq_quantize calls per step",
                   "tokens": T, "d": d, "calls_per_step": CALLS, "variant": variant_name,
                   "gelem_per_s": round(n * CALLS * args.steps / (ms * 1e-3) / 1e9, 1),
                   "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                   "X_sha256": x_sha, "params_sha256": p_sha},
        "device": {"name": torch.cuda.get_device_name(0),
                   "arch": getattr(torch.cuda.get_device_properties(0), "gcnArchName", ""),
                   "compute_units": torch.cuda.get_device_properties(0).multi_processor_count},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "comparison": comparison,
        "per_shape": per_shape,
        "adaln_fused": adaln,
        "w4a4_gemm": gemm,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
