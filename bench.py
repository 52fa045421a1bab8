#!/usr/bin/env python3
"""Benchmark of the H-BitLinear forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload wdown_7b] [--abits 4]

A step is one pass of the whole per-token path over one batch: RMSNorm + online FWHT +
per-token absmax INT4/INT8 quantisation (one kernel) and the ternary GEMM with its
dequant epilogue (one kernel), i.e. one hbl_forward call on the 7B-like Wdown shape
(M=8192 tokens, K=16384, N=4096).  Weights are ternarised once before timing (setup, as
in inference).  Inputs are synthetic (seeded) and resident in HBM before timing starts.

Timing: W untimed steps, then exactly K hbl_forward steps bracketed by device
synchronisation (wall clock) -> value.  A second pass issues the same two kernels through
their own C-ABI calls with HIP events between them on the launch stream, giving each
kernel's average duration for the roofline figures.  The oracle (CPU, all host threads)
is timed on a bounded sample of rows of the same workload.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "H-BitLinear a4 tokens/s + effective TOPS (% int8 MFMA peak), 7B-like Wdown"
PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
PEAK_FP4_TFLOPS = 10100.0    # MI355X dense FP6 / FP4 MFMA, 10.1 PFLOP/s
# fp32 vector adds: 157.3 TFLOP/s counts an FMA as two flops, so 78.6 T adds/s (packed, two per
# lane per clock: 256 CUs x 64 lanes x 2 x 2.4 GHz).  Code built without packed fp32, as
# this library is, issues at most half of that: 39.3 T adds/s.
PEAK_FP32_ADD_TOPS = 78.6
NONPACKED_FP32_ADD_TOPS = 39.3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--workload", default="wdown_7b")
    p.add_argument("--abits", type=int, default=4)
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle time of the CPU baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-alt", action="store_true", help="skip the FP6 x FP4 path measured beside the headline")
    p.add_argument("--copy-mb", type=int, default=0,
                   help="only run a plain device-to-device copy of this many MiB (3 times) and exit; used to "
                        "calibrate the FETCH_SIZE / WRITE_SIZE counters")
    return p.parse_args()


def copy_calibration(mb: int) -> None:
    import torch

    n = mb * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"[bench] copied {mb} MiB three times")


def code_digest(files) -> str:
    """SHA-256 of kernel sources (names under the package's csrc/) with comments, trailing
    blanks and empty lines removed, so that only a change of code invalidates a measurement."""
    import hashlib
    import re

    h = hashlib.sha256()
    for f in files:
        text = open(os.path.join(ROOT, "bit_quantized_gemm_bitlinear_amd", "csrc", f)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = (re.sub(r"//.*$", "", line).rstrip() for line in text.splitlines())
        h.update("\n".join(line for line in lines if line).encode())
    return h.hexdigest()


def measured_traffic(kernel: str):
    """HBM-side bytes per launch of `kernel` from profiles/traffic.json (rocprofv3 FETCH_SIZE and
    WRITE_SIZE per dispatch, each scaled by what the counter reads for a copy of known size),
    or None if the kernel's code has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    for e in json.load(open(path))["kernels"]:
        if e["kernel"] == kernel:
            return e["traffic_bytes"] if code_digest(e["sources"]) == e.get("code_sha256") else None
    return None


def mfma_ceiling(kind: str = "int8"):
    """The matrix-core rate this GPU sustains with no memory traffic and no other
    instructions (libhbl_probe.so), in TOP/s.  int8: v_mfma_i32_32x32x32_i8 with operands
    shaped like the GEMM's widened ones, bytes 16 q (q uniform in [-7, 7]) and 64 t (t in
    {-1, 0, 1}, 31 % zeros).  fp6fp4: v_mfma_scale_f32_32x32x64_f8f6f4 (FP6 x FP4) with
    random encodings."""
    import ctypes

    import numpy as np
    import torch

    path = os.path.join(ROOT, "bit_quantized_gemm_bitlinear_amd", "libhbl_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    f = lib.hbl_probe_mfma_ceiling if kind == "int8" else lib.hbl_probe_mfma_f6f4_ceiling
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    rng = np.random.default_rng(7)
    if kind == "int8":
        a = (rng.integers(-7, 8, 64 * 16) * 16).astype(np.int8)
        t = rng.choice([-1, 0, 1], size=64 * 16, p=[0.345, 0.31, 0.345])
        b = (t * 64).astype(np.int8)
        ops = torch.from_numpy(np.concatenate([a, b]).view(np.uint8)).cuda()
        per_mfma = 32 * 32 * 32 * 2
    else:
        ops = torch.from_numpy(rng.integers(0, 256, 128 * 32).astype(np.uint8)).cuda()
        per_mfma = 32 * 32 * 64 * 2
    blocks, iters = 768, 20000 if kind == "int8" else 10000  # one round of 4-wave blocks, 3 waves/SIMD
    out = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    sh = torch.cuda.current_stream().cuda_stream
    for _ in range(2):
        if f(ops.data_ptr(), blocks, iters, out.data_ptr(), sh) != 0:
            raise RuntimeError("hbl_probe_mfma_ceiling failed")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        f(ops.data_ptr(), blocks, iters, out.data_ptr(), sh)
    e1.record()
    torch.cuda.synchronize()
    t_one = e0.elapsed_time(e1) * 1e-3 / 3
    return blocks * 4 * iters * 4 * per_mfma / t_one / 1e12


def act_bytes_per_token(K: int, abits: int, x_bytes: int) -> int:
    """Algorithmic HBM bytes of the activation kernel per token: read x, write codes + deq."""
    return K * x_bytes + K * abits // 8 + 4


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the library has no multi-GPU path; "
              "the layer shards over tokens with no exchange, so N GPUs would run this same kernel on M/N rows.",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_mb:
        copy_calibration(args.copy_mb)
        return

    import numpy as np
    import torch

    from bit_quantized_gemm_bitlinear_amd import binding as B
    from bit_quantized_gemm_bitlinear_amd import inputs

    wl = inputs.WORKLOADS[args.workload]
    if wl.name == "ffn_7b":
        return bench_ffn(args, wl)
    if wl.name == "decode_7b":
        return bench_decode(args, wl)
    if wl.name == "kv_7b":
        return bench_kv(args, wl)
    abits = args.abits
    M, K, N = wl.M, wl.K, wl.N
    dev = torch.device("cuda:0")
    log(f"[bench] workload {wl.name} a{abits}: M={M} K={K} N={N} hadamard={wl.use_hadamard} norm={wl.norm}")

    t0 = time.time()
    x_np = wl.activations()
    W_np = wl.weights()
    log(f"[bench] inputs generated in {time.time() - t0:.1f}s")
    if x_np.dtype == np.uint16:
        x = torch.from_numpy(x_np.view(np.int16)).to(dev).view(torch.bfloat16)
        x_bytes = 2
    else:
        x = torch.from_numpy(x_np).to(dev)
        x_bytes = 4
    W = torch.from_numpy(W_np).to(dev)
    Wq, scale = B.quantize_weights(W)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    ws = B.forward_workspace(M, K, abits, dev)
    L = B.lib()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    norm = B.HBL_NORM_RMS if wl.norm else B.HBL_NORM_NONE
    xt = B._xdtype(x)
    ab = M * K * abits // 8
    codes_view = ws[:ab]
    deq_off = (ab + 255) // 256 * 256
    deq_view = ws[deq_off:deq_off + 4 * M].view(torch.float32)

    def step():
        st = L.hbl_forward(x.data_ptr(), xt, Wq.data_ptr(), scale.data_ptr(), M, K, N, abits, int(wl.use_hadamard),
                           norm, None, 1e-5, y.data_ptr(), ws.data_ptr(), ws.numel(), sh)
        if st != 0:
            raise RuntimeError(L.hbl_last_error().decode())

    def act():
        st = L.hbl_quantize_activations(x.data_ptr(), xt, M, K, norm, None, 1e-5, abits, int(wl.use_hadamard),
                                        codes_view.data_ptr(), deq_view.data_ptr(), sh)
        if st != 0:
            raise RuntimeError(L.hbl_last_error().decode())

    def gemm():
        st = L.hbl_gemm_dequant(codes_view.data_ptr(), deq_view.data_ptr(), Wq.data_ptr(), scale.data_ptr(), M, K,
                                N, abits, y.data_ptr(), sh)
        if st != 0:
            raise RuntimeError(L.hbl_last_error().decode())

    # ---- headline: K whole steps ----
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = M * args.steps / elapsed
    log(f"[bench] {args.steps} steps in {elapsed * 1e3:.2f} ms -> {ms_per_step:.4f} ms/step, {tokens_per_s:.4e} tok/s")

    # ---- per-kernel durations with HIP events on the launch stream ----
    n_ev = max(args.steps, 10)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_ev)]
    for _ in range(2):
        act()
        gemm()
    torch.cuda.synchronize()
    for i in range(n_ev):
        ev[i][0].record(stream)
        act()
        ev[i][1].record(stream)
        gemm()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    t_act = sum(e[0].elapsed_time(e[1]) for e in ev) / n_ev * 1e-3
    t_gemm = sum(e[1].elapsed_time(e[2]) for e in ev) / n_ev * 1e-3
    ops = 2.0 * M * N * K
    gemm_tops = ops / t_gemm / 1e12
    act_bytes = act_bytes_per_token(K, abits, x_bytes) * M
    act_gbs = act_bytes / t_act / 1e9
    eff_tops = ops / (ms_per_step * 1e-3) / 1e12
    log(f"[bench] act-quant {t_act * 1e6:.1f} us ({act_gbs:.0f} GB/s), gemm {t_gemm * 1e6:.1f} us "
        f"({gemm_tops:.0f} TOPS), effective {eff_tops:.0f} TOPS")

    # ---- the activation kernel from a cold Infinity Cache: a 512 MB read (twice the 256 MB
    # MALL) on the same stream before each launch, so x starts in HBM.  A read leaves clean
    # lines behind; a fill would leave 256 MB of dirty lines to be written back during the
    # timed launch. ----
    flush = torch.zeros(128 << 20, dtype=torch.float32, device=dev)
    evc = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(21)]
    for c0, c1 in evc:
        flush.sum()
        c0.record(stream)
        act()
        c1.record(stream)
    torch.cuda.synchronize()
    t_cold = sorted(c0.elapsed_time(c1) for c0, c1 in evc[1:])[10] * 1e-3
    del flush
    log(f"[bench] act-quant after a cache flush {t_cold * 1e6:.1f} us ({act_bytes / t_cold / 1e9:.0f} GB/s)")

    # ---- the same a4 forward on the FP6 x FP4 path (bit-identical outputs), reported beside ----
    alt = None
    if abits == 4 and not args.no_alt:
        Wq4 = B.weights_to_fp4(Wq, K)
        ws6 = torch.empty(max(L.hbl_forward_fp6fp4_workspace_bytes(M, K), 256), dtype=torch.uint8, device=dev)
        y6 = torch.empty_like(y)
        c6 = ws6[:M * K // 4 * 3]
        d6 = ws6[(M * K // 4 * 3 + 255) // 256 * 256:][:4 * M].view(torch.float32)

        def ok(st):
            if st != 0:
                raise RuntimeError(L.hbl_last_error().decode())

        def step6():
            ok(L.hbl_forward_fp6fp4(x.data_ptr(), xt, Wq4.data_ptr(), scale.data_ptr(), M, K, N, int(wl.use_hadamard),
                                    norm, None, 1e-5, y6.data_ptr(), ws6.data_ptr(), ws6.numel(), sh))

        for _ in range(args.warmup):
            step6()
        torch.cuda.synchronize()
        t6 = time.perf_counter()
        for _ in range(args.steps):
            step6()
        torch.cuda.synchronize()
        el6 = time.perf_counter() - t6
        ev6 = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_ev)]
        for i in range(n_ev):
            ev6[i][0].record(stream)
            ok(L.hbl_quantize_activations_fp6(x.data_ptr(), xt, M, K, norm, None, 1e-5, int(wl.use_hadamard),
                                              c6.data_ptr(), d6.data_ptr(), sh))
            ev6[i][1].record(stream)
            ok(L.hbl_gemm_fp6fp4_dequant(c6.data_ptr(), d6.data_ptr(), Wq4.data_ptr(), scale.data_ptr(), M, K, N,
                                         y6.data_ptr(), sh))
            ev6[i][2].record(stream)
        torch.cuda.synchronize()
        ta6 = sum(e[0].elapsed_time(e[1]) for e in ev6) / n_ev * 1e-3
        tg6 = sum(e[1].elapsed_time(e[2]) for e in ev6) / n_ev * 1e-3
        same = bool(torch.equal(y6.view(torch.int32), y.view(torch.int32)))
        g6 = ops / tg6 / 1e12
        ceil6 = mfma_ceiling("fp6fp4")
        alt = {"path": "FP6 (E2M3) INT4 codes x FP4 (E2M1) ternary weights, v_mfma_scale_f32_32x32x64_f8f6f4",
               "dtype": "fp6xfp4", "value": M * args.steps / el6, "unit": "tokens/s",
               "ms_per_step": el6 * 1e3 / args.steps, "outputs_bit_identical_to_int8_path": same,
               "kernels_us": {"actquant_fwht_fp6": ta6 * 1e6, "gemm_fp6fp4_dequant": tg6 * 1e6},
               "roofline": {"bound": "mfma", "achieved": g6, "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s",
                            "frac": g6 / PEAK_FP4_TFLOPS,
                            "traffic": measured_traffic("k_gemm_f6f4<256, 256, 4, 2, 1, true, false>"),
                            "kernel": "k_gemm_f6f4<256, 256, 4, 2, 1, true, false>",
                            "algorithmic": "2*M*N*K ops per launch"},
               "mfma_ceiling": None if not ceil6 else {
                   "tflops": ceil6, "frac_of_peak": ceil6 / PEAK_FP4_TFLOPS, "gemm_frac_of_ceiling": g6 / ceil6,
                   "method": "v_mfma_scale_f32_32x32x64_f8f6f4 (FP6 x FP4) only, 4 independent chains per wave"}}
        log(f"[bench] fp6xfp4 path: {el6 * 1e3 / args.steps:.4f} ms/step, act {ta6 * 1e6:.1f} us, gemm "
            f"{tg6 * 1e6:.1f} us ({g6:.0f} TFLOP/s), outputs identical: {same}"
            + (f"; FP6 x FP4 MFMA-only ceiling {ceil6:.0f} TFLOP/s, GEMM at {g6 / ceil6:.1%} of it" if ceil6 else ""))
        del Wq4, ws6, y6

    # ---- the INT4 absmean statistic (the activation-statistic switch), reported beside ----
    alt_mean = None
    if abits == 4 and not args.no_alt:
        def okm(st):
            if st != 0:
                raise RuntimeError(L.hbl_last_error().decode())

        def stepm():
            okm(L.hbl_forward_stat(x.data_ptr(), xt, Wq.data_ptr(), scale.data_ptr(), M, K, N, 4,
                                   int(wl.use_hadamard), norm, None, 1e-5, B.HBL_STAT_ABSMEAN, y.data_ptr(),
                                   ws.data_ptr(), ws.numel(), sh))

        for _ in range(args.warmup):
            stepm()
        torch.cuda.synchronize()
        tm = time.perf_counter()
        for _ in range(args.steps):
            stepm()
        torch.cuda.synchronize()
        elm = time.perf_counter() - tm
        evm = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_ev)]
        for i in range(n_ev):
            evm[i][0].record(stream)
            okm(L.hbl_quantize_activations_stat(x.data_ptr(), xt, M, K, norm, None, 1e-5, 4, int(wl.use_hadamard),
                                                B.HBL_STAT_ABSMEAN, codes_view.data_ptr(), deq_view.data_ptr(), sh))
            evm[i][1].record(stream)
        torch.cuda.synchronize()
        tam = sum(e[0].elapsed_time(e[1]) for e in evm) / n_ev * 1e-3
        alt_mean = {"statistic": "absmean (HBL_STAT_ABSMEAN)", "value": M * args.steps / elm, "unit": "tokens/s",
                    "ms_per_step": elm * 1e3 / args.steps, "actquant_us": tam * 1e6,
                    "actquant_gbs": act_bytes / tam / 1e9}
        log(f"[bench] absmean statistic: {elm * 1e3 / args.steps:.4f} ms/step, act {tam * 1e6:.1f} us")

    # The activation kernel with the transform is bound by its fp32 butterflies (K log2 K adds
    # per token), not by HBM; without the transform it streams.
    act_hbm = {"achieved": act_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": act_gbs / PEAK_HBM_GBS,
               "algorithmic": f"{act_bytes_per_token(K, abits, x_bytes)} B per token (read x, write packed codes + deq)"}
    if wl.use_hadamard:
        fwht_tops = M * K * (K.bit_length() - 1) / t_act / 1e12
        act_roofline = {"bound": "alu", "achieved": fwht_tops, "peak": PEAK_FP32_ADD_TOPS, "unit": "Tops/s",
                        "frac": fwht_tops / PEAK_FP32_ADD_TOPS,
                        "algorithmic": f"K*log2(K) = {K * (K.bit_length() - 1)} fp32 butterfly add/sub per token",
                        "peak_nonpacked": NONPACKED_FP32_ADD_TOPS, "hbm": act_hbm}
    else:
        act_roofline = {"bound": "hbm", **act_hbm}
    act_roofline["traffic_unit"] = "HBM-side bytes per launch (FETCH_SIZE x2.0 + WRITE_SIZE x1.0)"
    act_roofline["cold_cache"] = {"us": t_cold * 1e6, "achieved_gbs": act_bytes / t_cold / 1e9,
                                  "frac_hbm": act_bytes / t_cold / 1e9 / PEAK_HBM_GBS,
                                  "method": "512 MB read on the launch stream before each launch, median of 20"}
    gemm_kernel = f"k_gemm<{abits}, 256, 256, 2, 4, {256 if abits == 4 else 128}, 1, {'true' if K % (256 if abits == 4 else 128) == 0 else 'false'}, false>"
    act_kernel = f"k_actquant_h<{K.bit_length() - 1}, {abits}, 1, 1>"
    act_roofline["traffic"] = measured_traffic(act_kernel) if wl.name == "wdown_7b" else None

    ceiling = mfma_ceiling()
    if ceiling:
        log(f"[bench] MFMA-only int8 ceiling on this GPU: {ceiling:.0f} TOP/s; GEMM at {gemm_tops / ceiling:.1%} of it")

    # ---- CPU oracle baseline on a bounded sample of rows ----
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        oracle.build()
        threads = oracle.num_threads()
        T, alpha = oracle.quantize_weights(W_np)
        # Consecutive chunks of rows, each sized from the rate so far, until the target time
        # is spent (or the rows run out); only the oracle calls are timed.
        rows, dt, chunk = 0, 0.0, max(16, 2 * threads)
        while rows < M and dt < args.cpu_seconds:
            n = min(M - rows, chunk)
            tc = time.perf_counter()
            oracle.forward(np.ascontiguousarray(x_np[rows:rows + n]), T, alpha, abits, wl.use_hadamard, norm=wl.norm)
            dt += time.perf_counter() - tc
            rows += n
            chunk = max(16, int(rows / dt * (args.cpu_seconds - dt)) + 1)
        cpu = {"value": rows / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"first {rows} of {M} token rows of the same workload (weights ternarised beforehand, "
                         f"{dt:.1f} s of scalar C with OpenMP over rows)"}
        log(f"[bench] oracle: {rows} rows in {dt:.1f}s on {threads} threads -> {rows / dt:.1f} tok/s")

    out = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": f"{wl.name} a{abits}: {wl.description}", "M": M, "K": K, "N": N, "abits": abits,
                   "hadamard": bool(wl.use_hadamard), "norm": "rms" if wl.norm else "none",
                   "x_dtype": "bf16" if x_bytes == 2 else "fp32"},
        "effective_tops": eff_tops,
        "effective_pct_int8_peak": 100.0 * eff_tops / PEAK_INT8_TOPS,
        "kernels_us": {"actquant_fwht": t_act * 1e6, "gemm_dequant": t_gemm * 1e6},
        "roofline": {"bound": "mfma", "achieved": gemm_tops, "peak": PEAK_INT8_TOPS, "unit": "TFLOP/s",
                     "frac": gemm_tops / PEAK_INT8_TOPS,
                     "traffic": measured_traffic(gemm_kernel) if wl.name == "wdown_7b" else None,
                     "traffic_unit": "HBM-side bytes per launch (FETCH_SIZE x2.0 + WRITE_SIZE x1.0)",
                     "kernel": "k_gemm (ternary x INT%d, v_mfma_i32_32x32x32_i8)" % abits,
                     "algorithmic": "2*M*N*K int8 ops per launch"},
        "roofline_actquant": act_roofline,
        "mfma_ceiling": None if not ceiling else {
            "tops": ceiling, "frac_of_peak": ceiling / PEAK_INT8_TOPS, "gemm_frac_of_ceiling": gemm_tops / ceiling,
            "method": "v_mfma_i32_32x32x32_i8 only (no memory, no VALU), 4 independent chains per wave, 3 waves per "
                      "SIMD, operands shaped like the GEMM's widened codes and weights"},
        "cpu_baseline": cpu,
        "alt_fp6fp4": alt,
        "alt_absmean": alt_mean,
    }
    print(json.dumps(out), flush=True)


def bench_ffn(args, wl):
    """The 7B-like a4 FFN block: RMSNorm -> BitLinear gate and up (one shared activation
    quantisation, one fused GEMM whose epilogue writes h = silu(g) * u in bf16) -> H-BitLinear
    down.  A step is one hbl_ffn_forward call.  Reported separately from the headline."""
    import numpy as np
    import torch

    from bit_quantized_gemm_bitlinear_amd import binding as B
    from bit_quantized_gemm_bitlinear_amd import inputs

    M, hid, ffn = wl.M, wl.extra["hidden"], wl.extra["ffn"]
    abits = 4
    dev = torch.device("cuda:0")
    log(f"[bench] workload {wl.name}: M={M} hidden={hid} ffn={ffn}")
    x_np = wl.activations()
    x = torch.from_numpy(x_np.view(np.int16)).to(dev).view(torch.bfloat16)
    Wq = {}
    for name, (n, k, seed) in {"gate": (ffn, hid, wl.extra["seed_gate"]), "up": (ffn, hid, wl.extra["seed_up"]),
                               "down": (hid, ffn, wl.extra["seed_down"])}.items():
        Wq[name] = B.quantize_weights(torch.from_numpy(inputs.make_weights(n, k, seed=seed)).to(dev))
    Wgu = B.interleave_gate_up(Wq["gate"][0], Wq["up"][0], hid)
    sg, su = Wq["gate"][1], Wq["up"][1]
    qd, sd = Wq["down"]
    torch.cuda.synchronize()
    L = B.lib()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    ht = B.HBL_BF16
    ws = B.ffn_workspace(M, hid, ffn, abits, torch.bfloat16, dev)
    y = torch.empty((M, hid), dtype=torch.float32, device=dev)
    codes = torch.empty((M, hid * abits // 8), dtype=torch.uint8, device=dev)
    deq = torch.empty(M, dtype=torch.float32, device=dev)
    h = torch.empty((M, ffn), dtype=torch.bfloat16, device=dev)
    ws_down = B.forward_workspace(M, ffn, abits, dev)

    def ok(st):
        if st != 0:
            raise RuntimeError(L.hbl_last_error().decode())

    def step():
        ok(L.hbl_ffn_forward(x.data_ptr(), B.HBL_BF16, Wgu.data_ptr(), sg.data_ptr(), su.data_ptr(), qd.data_ptr(),
                             sd.data_ptr(), M, hid, ffn, abits, None, None, 1e-5, ht, y.data_ptr(), ws.data_ptr(),
                             ws.numel(), sh))

    def q():
        ok(L.hbl_quantize_activations(x.data_ptr(), B.HBL_BF16, M, hid, B.HBL_NORM_RMS, None, 1e-5, abits, 0,
                                      codes.data_ptr(), deq.data_ptr(), sh))

    def gate_up():
        ok(L.hbl_gate_up_swiglu(codes.data_ptr(), deq.data_ptr(), Wgu.data_ptr(), sg.data_ptr(), su.data_ptr(), M,
                                hid, ffn, abits, ht, h.data_ptr(), sh))

    def down_act():
        ok(L.hbl_quantize_activations(h.data_ptr(), B.HBL_BF16, M, ffn, B.HBL_NORM_RMS, None, 1e-5, abits, 1,
                                      ws_down.data_ptr(), ws_down[(M * ffn * abits // 8 + 255) // 256 * 256:]
                                      .data_ptr(), sh))

    def down_gemm():
        off = (M * ffn * abits // 8 + 255) // 256 * 256
        ok(L.hbl_gemm_dequant(ws_down.data_ptr(), ws_down[off:].data_ptr(), qd.data_ptr(), sd.data_ptr(), M, ffn,
                              hid, abits, y.data_ptr(), sh))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    parts = [("actquant_gate_up", q), ("gemm_gate_up_swiglu", gate_up), ("actquant_down_fwht", down_act),
             ("gemm_down", down_gemm)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)]
    sums = [0.0] * len(parts)
    n_ev = max(args.steps, 10)
    for _ in range(n_ev):
        ev[0].record(stream)
        for i, (_, f) in enumerate(parts):
            f()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        for i in range(len(parts)):
            sums[i] += ev[i].elapsed_time(ev[i + 1]) * 1e3 / n_ev
    ops = 3 * 2.0 * M * hid * ffn
    t_gu = sums[1] * 1e-6
    gu_tops = 2 * 2.0 * M * hid * ffn / t_gu / 1e12
    out = {"metric": "7B-like a4 FFN block tokens/s (RMSNorm, BitLinear gate/up + SwiGLU fused, H-BitLinear down)",
           "value": M * args.steps / el, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": el * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "i8", "data": "synthetic",
           "config": {"workload": f"{wl.name}: {wl.description}", "M": M, "hidden": hid, "ffn": ffn, "abits": abits,
                      "h_dtype": "bf16"},
           "effective_tops": ops / (el / args.steps) / 1e12,
           "parts_us": {name: v for (name, _), v in zip(parts, sums)},
           "roofline": {"bound": "mfma", "achieved": gu_tops, "peak": PEAK_INT8_TOPS, "unit": "TFLOP/s",
                        "frac": gu_tops / PEAK_INT8_TOPS,
                        "traffic": measured_traffic("k_gemm<4, 128, 256, 1, 4, 256, 3, true, false>"),
                        "traffic_unit": "HBM-side bytes per launch (FETCH_SIZE x2.0 + WRITE_SIZE x1.0)",
                        "kernel": "k_gemm fused gate/up + SwiGLU epilogue (v_mfma_i32_32x32x32_i8)",
                        "algorithmic": "2*M*(2*ffn)*hidden int8 ops per launch"}}
    log(f"[bench] ffn block {out['ms_per_step']:.3f} ms/step, parts " +
        ", ".join(f"{k} {v:.0f} us" for k, v in out["parts_us"].items()))
    print(json.dumps(out), flush=True)


def bench_decode(args, wl):
    """H-BitLinear a4 forward in the decode regime (M = 1..64 token rows per step) at the
    7B-like Wdown shape.  Each step uses the next of several copies of the packed weights, so
    the 16.8 MB weight read comes from HBM rather than the 256 MB Infinity Cache, as it would
    for a model whose layers do not fit there.  The headline line is M = 16; the other batch
    sizes are listed under "per_batch"."""
    import numpy as np
    import torch

    from bit_quantized_gemm_bitlinear_amd import binding as B

    K, N = wl.K, wl.N
    dev = torch.device("cuda:0")
    batches = wl.extra["batches"]
    copies = wl.extra["weight_copies"]
    x_np = wl.activations(max(batches))
    x_all = torch.from_numpy(x_np.view(np.int16)).to(dev).view(torch.bfloat16)
    Wq0, scale = B.quantize_weights(torch.from_numpy(wl.weights()).to(dev))
    Wqs = [Wq0.clone() for _ in range(copies)]
    L = B.lib()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    ws = B.forward_workspace(max(batches), K, 4, dev)
    y = torch.empty((max(batches), N), dtype=torch.float32, device=dev)
    steps = max(args.steps, 100)
    per = {}
    for M in batches:
        x = x_all[:M]
        codes = ws[:M * K // 2]
        deq = ws[(M * K // 2 + 255) // 256 * 256:][:4 * M].view(torch.float32)

        def ok(st):
            if st != 0:
                raise RuntimeError(L.hbl_last_error().decode())

        def step(i, stream_handle=sh):
            ok(L.hbl_forward(x.data_ptr(), B.HBL_BF16, Wqs[i % copies].data_ptr(), scale.data_ptr(), M, K, N, 4, 1,
                             B.HBL_NORM_RMS, None, 1e-5, y.data_ptr(), ws.data_ptr(), ws.numel(), stream_handle))

        for i in range(max(args.warmup, copies)):
            step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        el = (time.perf_counter() - t0) / steps
        # per-kernel durations: HIP events on the launch stream around `steps` back-to-back
        # launches of each kernel (an event pair per launch would add its own few microseconds
        # to kernels this short)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record(stream)
        for i in range(steps):
            ok(L.hbl_quantize_activations(x.data_ptr(), B.HBL_BF16, M, K, B.HBL_NORM_RMS, None, 1e-5, 4, 1,
                                          codes.data_ptr(), deq.data_ptr(), sh))
        ev[1].record(stream)
        for i in range(steps):
            ok(L.hbl_gemm_dequant(codes.data_ptr(), deq.data_ptr(), Wqs[i % copies].data_ptr(), scale.data_ptr(), M,
                                  K, N, 4, y.data_ptr(), sh))
        ev[2].record(stream)
        torch.cuda.synchronize()
        t_act = ev[0].elapsed_time(ev[1]) / steps * 1e-3
        t_gemv = ev[1].elapsed_time(ev[2]) / steps * 1e-3
        gemv_bytes = N * K // 4 + M * K // 2 + 4 * M + 4 + 4 * M * N
        fused = bool(L.hbl_forward_fused(M, K, 4, 1))
        # The same steps replayed from a HIP graph (one step per weight copy, captured once),
        # as a serving loop would run them: no host launch cost between steps.
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cs = torch.cuda.current_stream().cuda_stream
            for i in range(copies):
                step(i, cs)
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        reps = max(1, steps // copies)
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(reps):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        t_graph = g0.elapsed_time(g1) * 1e-3 / (reps * copies)
        del graph
        per[M] = {"us_per_step": el * 1e6, "tokens_per_s": M / el,
                  "graph_us_per_step": t_graph * 1e6, "graph_tokens_per_s": M / t_graph,
                  "path": "one fused kernel" if fused else "activation kernel + decode GEMM",
                  "separate_calls_us": {"actquant": t_act * 1e6, "gemv": t_gemv * 1e6},
                  "gemv_bytes": gemv_bytes, "gemv_gbs": gemv_bytes / t_gemv / 1e9}
        log(f"[bench] decode M={M}: {el * 1e6:.2f} us/step, {t_graph * 1e6:.2f} from a graph ({per[M]['path']}); "
            f"separate calls: act "
            f"{t_act * 1e6:.2f} us, gemv {t_gemv * 1e6:.2f} us ({gemv_bytes / t_gemv / 1e9:.0f} GB/s)")
    head = per[wl.M]
    out = {"metric": "H-BitLinear a4 decode tokens/s, 7B-like Wdown (weights streamed from HBM)",
           "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
           "ms_per_step": head["us_per_step"] * 1e-3, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "i8", "data": "synthetic",
           "config": {"workload": f"{wl.name}: {wl.description}", "M": wl.M, "K": K, "N": N, "abits": 4},
           "per_batch": {str(k): v for k, v in per.items()},
           "roofline": {"bound": "hbm", "achieved": head["gemv_gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": head["gemv_gbs"] / PEAK_HBM_GBS, "traffic": None,
                        "kernel": "k_gemv (decode GEMM, v_mfma_i32_16x16x64_i8)",
                        "algorithmic": "N*K/4 weight bytes + M*K/2 code bytes + 4*M*N output bytes per launch"}}
    print(json.dumps(out), flush=True)


def bench_kv(args, wl):
    """Unsigned absmax quantisation of post-RoPE K (or V) states into a 3-bit KV cache:
    8192 tokens x 32 heads x 128, bf16 in.  HBM-bound; reported against 8 TB/s.  A step is
    one launch over all 262144 head rows."""
    import numpy as np
    import torch

    from bit_quantized_gemm_bitlinear_amd import binding as B
    from bit_quantized_gemm_bitlinear_amd import inputs

    T, H, d, bits = wl.M, wl.extra["heads"], wl.extra["head_dim"], wl.extra["bits"]
    rows = T * H
    rng = np.random.default_rng(inputs.SEED_X)
    x = rng.standard_normal((rows, d)) * np.exp(rng.uniform(-4, 4, (rows, 1)))
    x[:, :3] *= 20.0
    xd = torch.from_numpy(inputs.f32_to_bf16_bits(x.astype(np.float32)).view(np.int16)).cuda().view(torch.bfloat16)
    del x
    # five copies (335 MB) used in turn, so the input is read from HBM, not the 256 MB Infinity Cache
    xs = [xd] + [xd.clone() for _ in range(4)]
    L = B.lib()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    codes = torch.empty((rows, d * bits // 8), dtype=torch.uint8, device="cuda")
    gamma = torch.empty(rows, dtype=torch.float32, device="cuda")

    def step(i):
        if L.hbl_quantize_qkv(xs[i % len(xs)].data_ptr(), B.HBL_BF16, rows, d, bits, codes.data_ptr(),
                              gamma.data_ptr(), sh):
            raise RuntimeError(L.hbl_last_error().decode())

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    el = (time.perf_counter() - t0) / args.steps
    t_k = e0.elapsed_time(e1) * 1e-3 / args.steps
    nbytes = rows * d * 2 + rows * d * bits // 8 + 4 * rows
    gbs = nbytes / t_k / 1e9
    log(f"[bench] kv quant {t_k * 1e6:.2f} us per launch, {gbs:.0f} GB/s")
    out = {"metric": "3-bit KV-cache quantisation tokens/s (unsigned absmax per head, 7B-like K states)",
           "value": T / el, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": el * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f32", "data": "synthetic",
           "config": {"workload": f"{wl.name}: {wl.description}", "tokens": T, "heads": H, "head_dim": d,
                      "bits": bits},
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": gbs / PEAK_HBM_GBS, "traffic": None, "kernel": "k_qkv_quant<3, bf16, 4>",
                        "algorithmic": f"{d * 2 + d * bits // 8 + 4} B per head row (read bf16, write codes + gamma)"}}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
