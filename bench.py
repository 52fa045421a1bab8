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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="wdown_7b")
    p.add_argument("--abits", type=int, default=4)
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle time of the CPU baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
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


def act_bytes_per_token(K: int, abits: int, x_bytes: int) -> int:
    """Algorithmic HBM bytes of the activation kernel per token: read x, write codes + deq."""
    return K * x_bytes + K * abits // 8 + 4


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): this build has no multi-GPU path; "
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

    # ---- CPU oracle baseline on a bounded sample of rows ----
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        oracle.build()
        threads = oracle.num_threads()
        T, alpha = oracle.quantize_weights(W_np)
        probe = 16
        tp = time.perf_counter()
        oracle.forward(x_np[:probe], T, alpha, abits, wl.use_hadamard, norm=wl.norm)
        per_row = (time.perf_counter() - tp) / probe
        rows = int(min(M, max(probe, args.cpu_seconds / max(per_row, 1e-9))))
        tc = time.perf_counter()
        oracle.forward(np.ascontiguousarray(x_np[:rows]), T, alpha, abits, wl.use_hadamard, norm=wl.norm)
        dt = time.perf_counter() - tc
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
                     "frac": gemm_tops / PEAK_INT8_TOPS, "traffic": None,
                     "kernel": "k_gemm (ternary x INT%d, v_mfma_i32_16x16x64_i8)" % abits,
                     "algorithmic": "2*M*N*K int8 ops per launch"},
        "roofline_actquant": {"bound": "hbm", "achieved": act_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                              "frac": act_gbs / PEAK_HBM_GBS, "traffic": None,
                              "algorithmic": f"{act_bytes_per_token(K, abits, x_bytes)} B per token "
                                             "(read x, write packed codes + deq)"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_ffn(args, wl):
    """The 7B-like a4 FFN block: RMSNorm -> INT4 BitLinear gate and up (one shared activation
    quantisation) -> SwiGLU -> H-BitLinear down.  Reported separately from the headline."""
    import numpy as np
    import torch

    from bit_quantized_gemm_bitlinear_amd import binding as B
    from bit_quantized_gemm_bitlinear_amd import inputs

    M, hid, ffn = wl.M, wl.extra["hidden"], wl.extra["ffn"]
    dev = torch.device("cuda:0")
    log(f"[bench] workload {wl.name}: M={M} hidden={hid} ffn={ffn}")
    x_np = wl.activations()
    x = torch.from_numpy(x_np.view(np.int16)).to(dev).view(torch.bfloat16)
    Wq = {}
    for name, (n, k, seed) in {"gate": (ffn, hid, wl.extra["seed_gate"]), "up": (ffn, hid, wl.extra["seed_up"]),
                               "down": (hid, ffn, wl.extra["seed_down"])}.items():
        Wq[name] = B.quantize_weights(torch.from_numpy(inputs.make_weights(n, k, seed=seed)).to(dev))
    torch.cuda.synchronize()
    L = B.lib()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    codes = torch.empty((M, hid // 2), dtype=torch.uint8, device=dev)
    deq = torch.empty(M, dtype=torch.float32, device=dev)
    g = torch.empty((M, ffn), dtype=torch.float32, device=dev)
    u = torch.empty_like(g)
    h = torch.empty_like(g)
    y = torch.empty((M, hid), dtype=torch.float32, device=dev)
    ws = B.forward_workspace(M, ffn, 4, dev)

    def ok(st):
        if st != 0:
            raise RuntimeError(L.hbl_last_error().decode())

    def q():
        ok(L.hbl_quantize_activations(x.data_ptr(), B.HBL_BF16, M, hid, B.HBL_NORM_RMS, None, 1e-5, 4, 0,
                                      codes.data_ptr(), deq.data_ptr(), sh))

    def gate():
        ok(L.hbl_gemm_dequant(codes.data_ptr(), deq.data_ptr(), Wq["gate"][0].data_ptr(), Wq["gate"][1].data_ptr(),
                              M, hid, ffn, 4, g.data_ptr(), sh))

    def up():
        ok(L.hbl_gemm_dequant(codes.data_ptr(), deq.data_ptr(), Wq["up"][0].data_ptr(), Wq["up"][1].data_ptr(),
                              M, hid, ffn, 4, u.data_ptr(), sh))

    def glu():
        ok(L.hbl_swiglu(g.data_ptr(), u.data_ptr(), g.numel(), h.data_ptr(), sh))

    def down():
        ok(L.hbl_forward(h.data_ptr(), B.HBL_F32, Wq["down"][0].data_ptr(), Wq["down"][1].data_ptr(), M, ffn, hid, 4,
                         1, B.HBL_NORM_RMS, None, 1e-5, y.data_ptr(), ws.data_ptr(), ws.numel(), sh))

    parts = [("actquant_gate_up", q), ("gemm_gate", gate), ("gemm_up", up), ("swiglu", glu), ("down_forward", down)]
    for _ in range(args.warmup):
        for _, f in parts:
            f()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for _, f in parts:
            f()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)]
    sums = [0.0] * len(parts)
    for _ in range(args.steps):
        ev[0].record(stream)
        for i, (_, f) in enumerate(parts):
            f()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        for i in range(len(parts)):
            sums[i] += ev[i].elapsed_time(ev[i + 1]) * 1e3 / args.steps
    ops = 3 * 2.0 * M * hid * ffn
    out = {"metric": "7B-like a4 FFN block tokens/s (RMSNorm, BitLinear gate/up, SwiGLU, H-BitLinear down)",
           "value": M * args.steps / el, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": el * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "i8", "data": "synthetic",
           "config": {"workload": f"{wl.name}: {wl.description}", "M": M, "hidden": hid, "ffn": ffn, "abits": 4},
           "effective_tops": ops / (el / args.steps) / 1e12,
           "parts_us": {name: v for (name, _), v in zip(parts, sums)}}
    log(f"[bench] ffn block {out['ms_per_step']:.3f} ms/step, parts " +
        ", ".join(f"{k} {v:.0f} us" for k, v in out["parts_us"].items()))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
