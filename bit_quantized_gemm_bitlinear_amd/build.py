"""Builds libhbl.so in-tree with hipcc for gfx950.

    python -m bit_quantized_gemm_bitlinear_amd.build

Every translation unit under csrc/ is compiled to an object (in parallel), then linked into
bit_quantized_gemm_bitlinear_amd/libhbl.so.  Flags: -O3, no FMA contraction
(-ffp-contract=off: the kernels round every fp32 product as written), IEEE fp32 division
and sqrt (HIP's default), packed-fp32 instructions disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libhbl.so")
PROBE_SRC = os.path.join(PKG, "probe", "mfma_ceiling.hip")
PROBE_LIB = os.path.join(PKG, "libhbl_probe.so")   # measurement aid for bench.py, not the layer
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libhbl)")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def common_flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


# Per-file extra flags.  The activation kernels read the results of their bf16 matrix
# products with VALU instructions: the VGPR form of the MFMAs writes them straight to VGPRs
# instead of AGPRs (saves one v_accvgpr_read per value).
EXTRA_FLAGS = {
    "k_actquant_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "k_actquant.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str, obj: str) -> tuple[str, int, str]:
    cmd = [hipcc(), "-x", "hip", "-c", src, "-o", obj] + common_flags() + EXTRA_FLAGS.get(os.path.basename(src), [])
    p = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the packed-fp32 target feature; that warning is harmless.
    err = "\n".join(l for l in (p.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    return src, p.returncode, err


def build(verbose: bool = False, jobs: int | None = None) -> str:
    srcs = sources()
    tmpdir = tempfile.mkdtemp(prefix="hbl_build_")
    try:
        objs = [os.path.join(tmpdir, os.path.basename(s) + ".o") for s in srcs]
        jobs = jobs or min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
        with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
            results = list(ex.map(lambda so: _compile(*so), zip(srcs, objs)))
        failed = [r for r in results if r[1] != 0]
        for src, rc, err in results:
            if err.strip() and (verbose or rc != 0):
                print(f"--- {os.path.basename(src)} ---\n{err}", file=sys.stderr)
        if failed:
            raise RuntimeError("hipcc failed for: " + ", ".join(os.path.basename(f[0]) for f in failed))
        tmp_lib = LIB + f".tmp{os.getpid()}"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib] + objs
        p = subprocess.run(cmd, capture_output=True, text=True)
        if p.returncode != 0:
            raise RuntimeError("link failed:\n" + p.stderr)
        os.replace(tmp_lib, LIB)
        tmp_probe = PROBE_LIB + f".tmp{os.getpid()}"
        p = subprocess.run([hipcc(), "-x", "hip", "-shared", PROBE_SRC, "-o", tmp_probe] + common_flags(),
                           capture_output=True, text=True)
        if p.returncode != 0:
            raise RuntimeError("probe build failed:\n" + p.stderr)
        os.replace(tmp_probe, PROBE_LIB)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
