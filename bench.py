#!/usr/bin/env python3
"""Benchmark of the H-BitLinear forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload wdown_7b] [--abits 4]

A step is one pass of the whole per-token path over one batch: RMSNorm + online FWHT +
per-token absmax INT4/INT8 quantisation (one kernel) and the ternary GEMM with its
dequant epilogue (one kernel), i.e. one hbl_forward call on the 7B-like Wdown shape
(M=8192 tokens, K=16384, N=4096).  Weights are ternarised once before timing (setup, as
in inference).  Inputs are synthetic (seeded) and resident in HBM before timing starts.

Timing: first untimed steps for --settle-ms (300 ms), since the clocks rise over the first
~100 ms of sustained load.  Then the two kernels are launched through their own C-ABI calls,
max(K, 20) times each, with HIP events around every launch on the launch stream: their mean
durations feed the roofline figures (the medians are reported beside).  Then W untimed steps
and exactly K hbl_forward steps bracketed by device synchronisation (wall clock) -> value.  After the timed steps the line gains: the shader clock
under matrix-core load and a plain device-copy bandwidth, both measured on the same GPU; the
activation kernel from a cold Infinity Cache; the same forward on the FP6 x FP4 path and with
the absmean statistic; every other configuration of the benchmark set (tiny exact-class layer,
1.3B Wo a8 and a4, 3B Wdown a4, 7B Wdown a8, the 7B FFN block) with its step time and kernel
rooflines; and the oracle (CPU) on a bounded sample of rows, on all host threads and on one
core for the small configurations.

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
    p.add_argument("--settle-ms", type=float, default=300.0,
                   help="untimed steps for this long before any timing (the clocks ramp up under load)")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the other configurations (tiny, 1.3B Wo a8/a4, 3B Wdown, 7B a8, FFN block)")
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


def event_times(stream, fns, n: int):
    """Runs the launch functions `fns` in order, n times, with a HIP event recorded on `stream`
    (the stream the library launches on) around each launch; returns one list of durations in
    seconds per function."""
    import torch

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(n)]
    for i in range(n):
        ev[i][0].record(stream)
        for j, f in enumerate(fns):
            f()
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    return [[ev[i][j].elapsed_time(ev[i][j + 1]) * 1e-3 for i in range(n)] for j in range(len(fns))]


def mean(v):
    return sum(v) / len(v)


def median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def shader_clock():
    """Average shader clock (MHz) under int8 matrix-core load on this GPU, from the probe kernel
    that reads the shader-clock and constant-rate counters at the start and end of each block
    (one round of 768 resident blocks, median over blocks), with the constant counter's rate."""
    import ctypes

    import numpy as np
    import torch

    path = os.path.join(ROOT, "bit_quantized_gemm_bitlinear_amd", "libhbl_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.hbl_probe_clock.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p]
    lib.hbl_probe_wallclock_khz.restype = ctypes.c_int
    khz = lib.hbl_probe_wallclock_khz()
    if khz <= 0:
        return None
    # operands shaped like the GEMM's widened ones (bytes 16 q and 64 t), as in mfma_ceiling:
    # the matrix cores' power, hence the clock, depends on the operand bits
    rng = np.random.default_rng(7)
    a = (rng.integers(-7, 8, 64 * 16) * 16).astype(np.int8)
    t8 = (rng.choice([-1, 0, 1], size=64 * 16, p=[0.345, 0.31, 0.345]) * 64).astype(np.int8)
    ops = torch.from_numpy(np.concatenate([a, t8]).view(np.uint8)).cuda()
    blocks, iters = 768, 20000
    out = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    ts = torch.zeros(2 * blocks, dtype=torch.int64, device="cuda")
    sh = torch.cuda.current_stream().cuda_stream
    if lib.hbl_probe_clock(ops.data_ptr(), blocks, iters, out.data_ptr(), ts.data_ptr(), sh) != 0:
        raise RuntimeError("hbl_probe_clock failed")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    lib.hbl_probe_clock(ops.data_ptr(), blocks, iters, out.data_ptr(), ts.data_ptr(), sh)
    e1.record()
    torch.cuda.synchronize()
    t_launch = e0.elapsed_time(e1) * 1e-3
    t = ts.view(blocks, 2).cpu().numpy().astype(np.float64)
    mhz = t[:, 0] / np.maximum(t[:, 1], 1) * khz / 1e3
    # int8 rate of the same launch, and the clock it implies at 32 cycles per
    # v_mfma_i32_32x32x32_i8 per SIMD (5.0 POP/s at 2.4 GHz on 256 CUs)
    tops = blocks * 4 * iters * 4 * 65536 / t_launch / 1e12
    return {"memtime_mhz": float(np.median(mhz)), "memtime_min_mhz": float(mhz.min()),
            "memtime_max_mhz": float(mhz.max()), "launch_tops": tops,
            "mhz_implied_by_mfma_rate": tops * 1e12 / (256 * 4 * 2048) / 1e6,
            "method": "probe kernel of int8 MFMA chains only, operands shaped like the GEMM's (768 blocks, all "
                      f"resident): s_memtime ticks over s_memrealtime ticks ({khz} kHz) per block, median over "
                      "blocks; and the launch's int8 rate divided by 256 CUs x 4 SIMDs x 2048 ops per clock"}


def copy_ceiling(mb: int = 1024):
    """HBM bandwidth a plain device copy reaches on this GPU (read + write bytes per second):
    torch copies of a buffer four times the 256 MB Infinity Cache, median of 7."""
    import torch

    n = mb * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    ts = event_times(torch.cuda.current_stream(), [lambda: b.copy_(a)], 7)[0]
    t = median(ts)
    del a, b
    return {"gbs": 2 * n * 4 / t / 1e9, "method": f"device-to-device copy of {mb} MiB (read + write), median of 7"}


def stream_ceiling(x):
    """HBM rate (GB/s) of a plain streaming kernel with the activation kernel's traffic mix on
    the same input: x read in 16-byte chunks, 4 bytes written per chunk (as bf16 rows in, INT4
    codes out), best of 2048 and 4096 blocks, median of 7 launches each."""
    import ctypes

    import torch

    path = os.path.join(ROOT, "bit_quantized_gemm_bitlinear_amd", "libhbl_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.hbl_probe_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    n16 = x.numel() * x.element_size() // 16
    out = torch.empty(n16, dtype=torch.int32, device=x.device)
    sh = torch.cuda.current_stream().cuda_stream
    best = None
    for blocks in (2048, 4096):
        run = lambda: lib.hbl_probe_stream(x.data_ptr(), n16, out.data_ptr(), blocks, sh)
        if run() != 0:
            raise RuntimeError("hbl_probe_stream failed")
        t = median(event_times(torch.cuda.current_stream(), [run], 7)[0])
        gbs = n16 * 20 / t / 1e9
        if best is None or gbs > best["gbs"]:
            best = {"gbs": gbs, "us": t * 1e6, "blocks": blocks}
    best["method"] = ("streaming kernel over the activation input: 16 bytes read and 4 written per chunk, four loads "
                      "in flight per thread, median of 7 launches")
    return best


class LayerRun:
    """One H-BitLinear (or BitLinear) workload set up on the GPU: inputs resident in HBM,
    weights ternarised, workspace carved; the step and its two kernels as C-ABI calls on
    torch's current stream."""

    def __init__(self, wl, abits: int, x_np=None, W_np=None):
        import numpy as np
        import torch

        from bit_quantized_gemm_bitlinear_amd import binding as B

        self.wl, self.abits = wl, abits
        self.M, self.K, self.N = wl.M, wl.K, wl.N
        dev = torch.device("cuda:0")
        x_np = wl.activations() if x_np is None else x_np
        W_np = wl.weights() if W_np is None else W_np
        if x_np.dtype == np.uint16:
            self.x = torch.from_numpy(x_np.view(np.int16)).to(dev).view(torch.bfloat16)
            self.x_bytes = 2
        else:
            self.x = torch.from_numpy(x_np).to(dev)
            self.x_bytes = 4
        self.Wq, self.scale = B.quantize_weights(torch.from_numpy(W_np).to(dev))
        self.y = torch.empty((self.M, self.N), dtype=torch.float32, device=dev)
        self.ws = B.forward_workspace(self.M, self.K, abits, dev)
        self.L = B.lib()
        self.stream = torch.cuda.current_stream()
        self.sh = self.stream.cuda_stream
        self.norm = B.HBL_NORM_RMS if wl.norm else B.HBL_NORM_NONE
        self.xt = B._xdtype(self.x)
        ab = self.M * self.K * abits // 8
        self.codes = self.ws[:ab]
        off = (ab + 255) // 256 * 256
        self.deq = self.ws[off:off + 4 * self.M].view(torch.float32)
        torch.cuda.synchronize()

    def _ok(self, st):
        if st != 0:
            raise RuntimeError(self.L.hbl_last_error().decode())

    def step(self):
        self._ok(self.L.hbl_forward(self.x.data_ptr(), self.xt, self.Wq.data_ptr(), self.scale.data_ptr(), self.M,
                                    self.K, self.N, self.abits, int(self.wl.use_hadamard), self.norm, None, 1e-5,
                                    self.y.data_ptr(), self.ws.data_ptr(), self.ws.numel(), self.sh))

    def act(self):
        self._ok(self.L.hbl_quantize_activations(self.x.data_ptr(), self.xt, self.M, self.K, self.norm, None, 1e-5,
                                                 self.abits, int(self.wl.use_hadamard), self.codes.data_ptr(),
                                                 self.deq.data_ptr(), self.sh))

    def gemm(self):
        self._ok(self.L.hbl_gemm_dequant(self.codes.data_ptr(), self.deq.data_ptr(), self.Wq.data_ptr(),
                                         self.scale.data_ptr(), self.M, self.K, self.N, self.abits, self.y.data_ptr(),
                                         self.sh))

    def timed_steps(self, steps: int, warmup: int):
        """W untimed steps, then exactly `steps` steps between two device synchronisations."""
        import torch

        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    def kernel_times(self, n: int):
        """Per-launch durations (s) of the activation kernel and the GEMM, n launches each."""
        self.act()
        self.gemm()
        return event_times(self.stream, [self.act, self.gemm], n)

    def back_to_back(self, f, n: int) -> float:
        """Mean duration (s) of n back-to-back launches of f between one pair of events: for
        kernels of a few microseconds an event pair around every launch adds its own time."""
        import torch

        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f()
        e0.record(self.stream)
        for _ in range(n):
            f()
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / n

    def summary(self, steps: int, warmup: int, n_ev: int):
        """ms/step, tokens/s and the two kernels' times and rooflines, for the extra configs."""
        t_act_l, t_gemm_l = self.kernel_times(n_ev)
        el = self.timed_steps(steps, warmup)
        t_act, t_gemm = self.back_to_back(self.act, n_ev), self.back_to_back(self.gemm, n_ev)
        ops = 2.0 * self.M * self.N * self.K
        act_bytes = act_bytes_per_token(self.K, self.abits, self.x_bytes) * self.M
        return {"workload": f"{self.wl.name} a{self.abits}: {self.wl.description}",
                "M": self.M, "K": self.K, "N": self.N, "abits": self.abits, "steps": steps, "warmup": warmup,
                "ms_per_step": el * 1e3 / steps, "tokens_per_s": self.M * steps / el,
                "effective_tops": ops / (el / steps) / 1e12,
                "kernels_us": {"actquant": t_act * 1e6, "gemm_dequant": t_gemm * 1e6},
                "kernels_median_us": {"actquant": median(t_act_l) * 1e6, "gemm_dequant": median(t_gemm_l) * 1e6},
                "launches_per_kernel": n_ev,
                "timing": "kernels_us: mean of back-to-back launches between one event pair; kernels_median_us: "
                          "median of launches with an event pair each",
                "gemm_roofline": {"bound": "mfma", "achieved": ops / t_gemm / 1e12, "peak": PEAK_INT8_TOPS,
                                  "unit": "TFLOP/s", "frac": ops / t_gemm / 1e12 / PEAK_INT8_TOPS},
                "actquant_roofline": {"bound": "hbm", "achieved": act_bytes / t_act / 1e9, "peak": PEAK_HBM_GBS,
                                      "unit": "GB/s", "frac": act_bytes / t_act / 1e9 / PEAK_HBM_GBS}}


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
    lay = LayerRun(wl, abits, x_np, W_np)
    L, stream, sh = lay.L, lay.stream, lay.sh
    x, xt, norm, Wq, scale, y, ws = lay.x, lay.xt, lay.norm, lay.Wq, lay.scale, lay.y, lay.ws
    codes_view, deq_view, x_bytes = lay.codes, lay.deq, lay.x_bytes
    ops = 2.0 * M * N * K
    act_bytes = act_bytes_per_token(K, abits, x_bytes) * M

    # ---- the GPU's clocks rise over the first ~100 ms of sustained load: untimed steps until
    # `settle_ms` have passed, so that every figure below is taken in the steady state ----
    settle_steps, t_settle = 0, time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(10):
            lay.step()
        torch.cuda.synchronize()
        settle_steps += 10
    t_settle = time.perf_counter() - t_settle
    log(f"[bench] settled with {settle_steps} untimed steps in {t_settle * 1e3:.0f} ms")

    # ---- per-kernel durations: HIP events around each launch on the launch stream, at least 20
    # launches of each kernel (mean for the rooflines, median beside it) ----
    n_ev = max(args.steps, 20)
    t_act_l, t_gemm_l = lay.kernel_times(n_ev)
    t_act, t_gemm = mean(t_act_l), mean(t_gemm_l)
    gemm_tops = ops / t_gemm / 1e12
    act_gbs = act_bytes / t_act / 1e9

    # ---- headline: W untimed steps, then exactly K whole steps ----
    elapsed = lay.timed_steps(args.steps, args.warmup)
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = M * args.steps / elapsed
    eff_tops = ops / (ms_per_step * 1e-3) / 1e12
    log(f"[bench] {args.steps} steps in {elapsed * 1e3:.2f} ms -> {ms_per_step:.4f} ms/step, {tokens_per_s:.4e} tok/s")
    log(f"[bench] act-quant {t_act * 1e6:.1f} us (median {median(t_act_l) * 1e6:.1f}, {act_gbs:.0f} GB/s), gemm "
        f"{t_gemm * 1e6:.1f} us (median {median(t_gemm_l) * 1e6:.1f}, {gemm_tops:.0f} TOPS), effective {eff_tops:.0f} TOPS")

    clock = shader_clock()
    copy = copy_ceiling()
    stream_c = stream_ceiling(x)
    if stream_c:
        log(f"[bench] streaming ceiling at the activation kernel's traffic mix {stream_c['gbs']:.0f} GB/s")
    if clock:
        log(f"[bench] clock probe: s_memtime rate {clock['memtime_mhz']:.0f} MHz, int8 rate {clock['launch_tops']:.0f} "
            f"TOP/s = {clock['mhz_implied_by_mfma_rate']:.0f} MHz at 2048 ops/clock/SIMD")
    log(f"[bench] device copy ceiling {copy['gbs']:.0f} GB/s")

    # ---- the activation kernel from a cold Infinity Cache: a 512 MB read (twice the 256 MB
    # MALL) on the same stream before each launch, so x starts in HBM.  A read leaves clean
    # lines behind; a fill would leave 256 MB of dirty lines to be written back during the
    # timed launch. ----
    flush = torch.zeros(128 << 20, dtype=torch.float32, device=dev)
    evc = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(21)]
    for c0, c1 in evc:
        flush.sum()
        c0.record(stream)
        lay.act()
        c1.record(stream)
    torch.cuda.synchronize()
    t_cold = median([c0.elapsed_time(c1) for c0, c1 in evc[1:]]) * 1e-3
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

        def act6():
            ok(L.hbl_quantize_activations_fp6(x.data_ptr(), xt, M, K, norm, None, 1e-5, int(wl.use_hadamard),
                                              c6.data_ptr(), d6.data_ptr(), sh))

        def gemm6():
            ok(L.hbl_gemm_fp6fp4_dequant(c6.data_ptr(), d6.data_ptr(), Wq4.data_ptr(), scale.data_ptr(), M, K, N,
                                         y6.data_ptr(), sh))

        ta6_l, tg6_l = event_times(stream, [act6, gemm6], n_ev)
        for _ in range(args.warmup):
            step6()
        torch.cuda.synchronize()
        t6 = time.perf_counter()
        for _ in range(args.steps):
            step6()
        torch.cuda.synchronize()
        el6 = time.perf_counter() - t6
        ta6, tg6 = mean(ta6_l), mean(tg6_l)
        lay.step()
        torch.cuda.synchronize()
        same = bool(torch.equal(y6.view(torch.int32), y.view(torch.int32)))
        g6 = ops / tg6 / 1e12
        ceil6 = mfma_ceiling("fp6fp4")
        alt = {"path": "FP6 (E2M3) INT4 codes x FP4 (E2M1) ternary weights, v_mfma_scale_f32_32x32x64_f8f6f4",
               "dtype": "fp6xfp4", "value": M * args.steps / el6, "unit": "tokens/s",
               "ms_per_step": el6 * 1e3 / args.steps, "outputs_bit_identical_to_int8_path": same,
               "kernels_us": {"actquant_fwht_fp6": ta6 * 1e6, "gemm_fp6fp4_dequant": tg6 * 1e6},
               "kernels_median_us": {"actquant_fwht_fp6": median(ta6_l) * 1e6,
                                     "gemm_fp6fp4_dequant": median(tg6_l) * 1e6},
               "roofline": {"bound": "mfma", "achieved": g6, "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s",
                            "frac": g6 / PEAK_FP4_TFLOPS,
                            "traffic": measured_traffic("k_gemm_f6f4_dma<1>"),
                            "kernel": "k_gemm_f6f4_dma<1>",
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

        def actm():
            okm(L.hbl_quantize_activations_stat(x.data_ptr(), xt, M, K, norm, None, 1e-5, 4, int(wl.use_hadamard),
                                                B.HBL_STAT_ABSMEAN, codes_view.data_ptr(), deq_view.data_ptr(), sh))

        tam_l = event_times(stream, [actm], n_ev)[0]
        for _ in range(args.warmup):
            stepm()
        torch.cuda.synchronize()
        tm = time.perf_counter()
        for _ in range(args.steps):
            stepm()
        torch.cuda.synchronize()
        elm = time.perf_counter() - tm
        tam = mean(tam_l)
        alt_mean = {"statistic": "absmean (HBL_STAT_ABSMEAN)", "value": M * args.steps / elm, "unit": "tokens/s",
                    "ms_per_step": elm * 1e3 / args.steps, "actquant_us": tam * 1e6,
                    "actquant_median_us": median(tam_l) * 1e6, "actquant_gbs": act_bytes / tam / 1e9}
        log(f"[bench] absmean statistic: {elm * 1e3 / args.steps:.4f} ms/step, act {tam * 1e6:.1f} us")

    # The activation kernel is bound by HBM: it reads x once and writes the packed codes once.
    # Its fp32 butterflies (K log2 K adds per token) are reported beside, as context.
    act_roofline = {"bound": "hbm", "achieved": act_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": act_gbs / PEAK_HBM_GBS, "target_frac": 0.70,
                    "algorithmic": f"{act_bytes_per_token(K, abits, x_bytes)} B per token (read x, write packed "
                                   "codes + deq)",
                    "median_us": median(t_act_l) * 1e6, "mean_us": t_act * 1e6,
                    "copy_ceiling": {"gbs": copy["gbs"], "frac_of_copy": act_gbs / copy["gbs"],
                                     "method": copy["method"]},
                    "stream_ceiling": None if not stream_c else {
                        **stream_c, "frac_of_stream": act_gbs / stream_c["gbs"]}}
    if wl.use_hadamard:
        fwht = M * K * (K.bit_length() - 1) / t_act / 1e12
        act_roofline["alu_context"] = {
            "achieved": fwht, "unit": "T adds/s", "peak_nonpacked": NONPACKED_FP32_ADD_TOPS,
            "frac_nonpacked": fwht / NONPACKED_FP32_ADD_TOPS,
            "algorithmic": f"K*log2(K) = {K * (K.bit_length() - 1)} butterfly add/sub per token (5 of the "
                           f"{K.bit_length() - 1} stages on the bf16 matrix cores for bf16 rows)"}
    act_roofline["traffic_unit"] = "HBM-side bytes per launch (FETCH_SIZE x2.0 + WRITE_SIZE x1.0)"
    act_roofline["cold_cache"] = {"us": t_cold * 1e6, "achieved_gbs": act_bytes / t_cold / 1e9,
                                  "frac_hbm": act_bytes / t_cold / 1e9 / PEAK_HBM_GBS,
                                  "method": "512 MB read on the launch stream before each launch, median of 20"}
    bk = 256 if abits == 4 else 128   # stage depth of the large-tile GEMMs
    # K a multiple of the stage depth: the kernel that loads its tiles straight into LDS
    gemm_kernel = (f"k_gemm_dma<{abits}, 256, 256, 2, 4, 1, 3>" if K % bk == 0 else
                   f"k_gemm<{abits}, 256, 256, 2, 4, {bk}, 1, false, false>")
    act_kernel = f"k_actquant_hm<{K.bit_length() - 1}, {abits}, 1>"
    act_roofline["kernel"] = act_kernel
    act_roofline["traffic"] = measured_traffic(act_kernel) if wl.name == "wdown_7b" else None

    ceiling = mfma_ceiling()
    if ceiling:
        log(f"[bench] MFMA-only int8 ceiling on this GPU: {ceiling:.0f} TOP/s; GEMM at {gemm_tops / ceiling:.1%} of it")

    # ---- every other configuration of the benchmark set, measured the same way ----
    configs = None
    if not args.no_configs and wl.name == "wdown_7b" and abits == 4:
        del lay
        torch.cuda.empty_cache()
        configs = {}
        steps_c = max(args.steps, 20)
        for name, ab in [("tiny_exact", 4), ("wo_1p3b", 8), ("wo_1p3b", 4), ("wdown_3b", 4), ("wdown_7b", 8)]:
            run = LayerRun(inputs.WORKLOADS[name], ab, x_np=x_np if name == "wdown_7b" else None,
                           W_np=W_np if name == "wdown_7b" else None)
            configs[f"{name}_a{ab}"] = run.summary(steps_c, args.warmup, n_ev)
            c = configs[f"{name}_a{ab}"]
            log(f"[bench] {name} a{ab}: {c['ms_per_step']:.4f} ms/step, {c['tokens_per_s']:.4e} tok/s, act "
                f"{c['kernels_us']['actquant']:.1f} us ({c['actquant_roofline']['frac']:.1%} HBM), gemm "
                f"{c['kernels_us']['gemm_dequant']:.1f} us ({c['gemm_roofline']['frac']:.1%} int8)")
            del run
            torch.cuda.empty_cache()
        configs["ffn_7b_a4"] = ffn_measure(inputs.WORKLOADS["ffn_7b"], steps_c, args.warmup, n_ev)
        c = configs["ffn_7b_a4"]
        log(f"[bench] ffn_7b a4 block: {c['ms_per_step']:.4f} ms/step, {c['tokens_per_s']:.4e} tok/s")
        torch.cuda.empty_cache()

    # ---- CPU oracle baseline on a bounded sample of rows (all host threads), and a single
    # core on the small configurations ----
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
        single = {}
        oracle.set_num_threads(1)
        try:
            for name, ab, n_rows in [("tiny_exact", 4, 16), ("wo_1p3b", 4, 128)]:
                w2 = inputs.WORKLOADS[name]
                xs = w2.activations(n_rows)
                T2, a2 = oracle.quantize_weights(w2.weights())
                tc = time.perf_counter()
                oracle.forward(xs, T2, a2, ab, w2.use_hadamard, norm=w2.norm)
                d = time.perf_counter() - tc
                single[f"{name}_a{ab}"] = {"tokens_per_s": n_rows / d, "rows": n_rows, "seconds": d}
                log(f"[bench] oracle, one core, {name} a{ab}: {n_rows} rows in {d:.3f}s")
        finally:
            oracle.set_num_threads(threads)
        cpu["single_core"] = single

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
        "kernels_median_us": {"actquant_fwht": median(t_act_l) * 1e6, "gemm_dequant": median(t_gemm_l) * 1e6},
        "launches_per_kernel": n_ev,
        "settle": {"steps": settle_steps, "ms": t_settle * 1e3,
                   "note": "untimed steps before the per-kernel timings and the W warm-up steps, until the clocks "
                           "reach their loaded state"},
        "roofline": {"bound": "mfma", "achieved": gemm_tops, "peak": PEAK_INT8_TOPS, "unit": "TFLOP/s",
                     "frac": gemm_tops / PEAK_INT8_TOPS,
                     "traffic": measured_traffic(gemm_kernel) if wl.name == "wdown_7b" else None,
                     "traffic_unit": "HBM-side bytes per launch (FETCH_SIZE x2.0 + WRITE_SIZE x1.0)",
                     "kernel": f"{gemm_kernel} (ternary x INT{abits}, v_mfma_i32_32x32x32_i8)",
                     "algorithmic": "2*M*N*K int8 ops per launch",
                     "median_us": median(t_gemm_l) * 1e6, "mean_us": t_gemm * 1e6},
        "roofline_actquant": act_roofline,
        "mfma_ceiling": None if not ceiling else {
            "tops": ceiling, "frac_of_peak": ceiling / PEAK_INT8_TOPS, "gemm_frac_of_ceiling": gemm_tops / ceiling,
            "method": "v_mfma_i32_32x32x32_i8 only (no memory, no VALU), 4 independent chains per wave, 3 waves per "
                      "SIMD, operands shaped like the GEMM's widened codes and weights"},
        "shader_clock": clock,
        "hbm_copy_ceiling": copy,
        "configs": configs,
        "cpu_baseline": cpu,
        "alt_fp6fp4": alt,
        "alt_absmean": alt_mean,
    }
    print(json.dumps(out), flush=True)


def ffn_measure(wl, steps: int, warmup: int, n_ev: int):
    """The 7B-like a4 FFN block: RMSNorm -> BitLinear gate and up (one shared activation
    quantisation, one fused GEMM whose epilogue writes h = silu(g) * u in bf16) -> H-BitLinear
    down.  A step is one hbl_ffn_forward call."""
    import numpy as np
    import torch

    from bit_quantized_gemm_bitlinear_amd import binding as B
    from bit_quantized_gemm_bitlinear_amd import inputs

    M, hid, ffn = wl.M, wl.extra["hidden"], wl.extra["ffn"]
    abits = 4
    dev = torch.device("cuda:0")
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
    off = (M * ffn * abits // 8 + 255) // 256 * 256

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
                                      ws_down.data_ptr(), ws_down[off:].data_ptr(), sh))

    def down_gemm():
        ok(L.hbl_gemm_dequant(ws_down.data_ptr(), ws_down[off:].data_ptr(), qd.data_ptr(), sd.data_ptr(), M, ffn,
                              hid, abits, y.data_ptr(), sh))

    parts = [("actquant_gate_up", q), ("gemm_gate_up_swiglu", gate_up), ("actquant_down_fwht", down_act),
             ("gemm_down", down_gemm)]
    times = event_times(stream, [f for _, f in parts], n_ev)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ops = 3 * 2.0 * M * hid * ffn
    t_gu = mean(times[1])
    gu_tops = 2 * 2.0 * M * hid * ffn / t_gu / 1e12
    return {"workload": f"{wl.name}: {wl.description}", "M": M, "hidden": hid, "ffn": ffn, "abits": abits,
            "h_dtype": "bf16", "steps": steps, "warmup": warmup, "ms_per_step": el * 1e3 / steps,
            "tokens_per_s": M * steps / el, "effective_tops": ops / (el / steps) / 1e12,
            "parts_us": {name: mean(t) * 1e6 for (name, _), t in zip(parts, times)},
            "parts_median_us": {name: median(t) * 1e6 for (name, _), t in zip(parts, times)},
            "launches_per_kernel": n_ev,
            "roofline": {"bound": "mfma", "achieved": gu_tops, "peak": PEAK_INT8_TOPS, "unit": "TFLOP/s",
                         "frac": gu_tops / PEAK_INT8_TOPS,
                         "traffic": measured_traffic("k_gemm_dma<4, 128, 256, 1, 4, 3, 2>"),
                         "traffic_unit": "HBM-side bytes per launch (FETCH_SIZE x2.0 + WRITE_SIZE x1.0)",
                         "kernel": "k_gemm_dma<4, 128, 256, 1, 4, 3, 2> (fused gate/up + SwiGLU epilogue, "
                                   "v_mfma_i32_32x32x32_i8)",
                         "algorithmic": "2*M*(2*ffn)*hidden int8 ops per launch"}}


def bench_ffn(args, wl):
    """The FFN block as its own JSON line (--workload ffn_7b)."""
    r = ffn_measure(wl, args.steps, args.warmup, max(args.steps, 20))
    out = {"metric": "7B-like a4 FFN block tokens/s (RMSNorm, BitLinear gate/up + SwiGLU fused, H-BitLinear down)",
           "value": r["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": r["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "i8", "data": "synthetic",
           "config": {"workload": r["workload"], "M": r["M"], "hidden": r["hidden"], "ffn": r["ffn"],
                      "abits": r["abits"], "h_dtype": "bf16"},
           "effective_tops": r["effective_tops"], "parts_us": r["parts_us"], "parts_median_us": r["parts_median_us"],
           "roofline": r["roofline"]}
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
    # Same-run references for launches this small, on the same stream: a device copy of one
    # packed weight copy (16.8 MB read and written, the source rotated over the copies as the
    # steps do) and a one-element fill (launch and completion latency alone).
    dst = torch.empty_like(Wq0)
    one = torch.empty(1, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    for i in range(copies):
        dst.copy_(Wqs[i])
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(steps):
        dst.copy_(Wqs[i % copies])
    ev[1].record(stream)
    for i in range(steps):
        one.fill_(1.0)
    ev[2].record(stream)
    torch.cuda.synchronize()
    t_copy = ev[0].elapsed_time(ev[1]) / steps * 1e-3
    t_fill = ev[1].elapsed_time(ev[2]) / steps * 1e-3
    reference = {"copy_us": t_copy * 1e6, "copy_gbs": 2 * Wq0.numel() / t_copy / 1e9, "fill_us": t_fill * 1e6,
                 "method": f"{steps} back-to-back device copies of one {Wq0.numel() / 1e6:.1f} MB weight copy "
                           f"(source rotated over {copies}) and {steps} one-element fills, events on the launch stream"}
    log(f"[bench] same-run references: weight-sized copy {t_copy * 1e6:.2f} us ({reference['copy_gbs']:.0f} GB/s), "
        f"one-element fill {t_fill * 1e6:.2f} us")
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
                        "algorithmic": "N*K/4 weight bytes + M*K/2 code bytes + 4*M*N output bytes per launch",
                        "same_run_reference": reference}}
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
