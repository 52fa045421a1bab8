"""AddressSanitizer and UndefinedBehaviorSanitizer runs of the host code, on the CPU:

- the oracle (oracle/hbl_oracle.c) built with gcc -fsanitize=address,undefined, and the
  oracle's pin tests run against that build;
- the C ABI layer (csrc/api.cpp with the host-only plan.cpp) built with g++ and the same
  sanitizers, linked with stand-ins for the kernel launchers, and the ABI tests
  (tests/test_abi.py, argument validation, exported symbols) run against it.

Each run is a subprocess with gcc's ASan runtime preloaded into the Python interpreter;
any sanitizer report makes it fail (UBSan does not recover)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_quantized_gemm_bitlinear_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _asan_runtime():
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not available")
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(p) or not os.path.exists(p):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return p


def _run_under_asan(args, env_extra, timeout):
    env = dict(os.environ)
    env.update(env_extra)
    env["LD_PRELOAD"] = _asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu"] + args,
                       capture_output=True, text=True, timeout=timeout, cwd=ROOT, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    return out


def test_oracle_pins_under_sanitizers(tmp_path):
    lib = tmp_path / "liboracle_san.so"
    src = os.path.join(ROOT, "oracle", "hbl_oracle.c")
    cmd = ["gcc", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math"] + SAN + \
          ["-o", str(lib), src, "-lm"]
    subprocess.run(cmd, check=True, timeout=300)
    pins = sorted(f"tests/{f}" for f in os.listdir(os.path.join(ROOT, "tests"))
                  if f.startswith("test_oracle_") and f != "test_oracle_mutations.py")
    out = _run_under_asan(pins, {"HBL_ORACLE_LIB": str(lib), "OMP_NUM_THREADS": "4"}, timeout=900)
    assert " passed" in out


def test_abi_validation_under_sanitizers(tmp_path):
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    if not os.path.exists(os.path.join(rocm, "include", "hip", "hip_runtime.h")):
        pytest.skip("HIP headers are not installed")
    lib = tmp_path / "libhbl_hostcheck.so"
    # a host-only build: no device compiler, so the scratch array of hbl_forward_noalloc is an
    # ordinary host array here (never reached: every call in the ABI tests stops at validation)
    defs = ["-D__HIP_PLATFORM_AMD__", "-D__align__(n)=__attribute__((aligned(n)))",
            "-DHIP_SYMBOL(x)=((const void*)&(x))"]
    srcs = [os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "plan.cpp"),
            os.path.join(ROOT, "tests", "sanitize", "stub_launchers.cpp")]
    cmd = ["g++", "-std=c++17", "-fPIC", "-shared"] + SAN + defs + \
          [f"-I{rocm}/include", f"-I{ROOT}/include", f"-I{CSRC}", "-o", str(lib)] + srcs + \
          [f"-L{rocm}/lib", "-lamdhip64", f"-Wl,-rpath,{rocm}/lib"]
    subprocess.run(cmd, check=True, timeout=300)
    out = _run_under_asan(["tests/test_abi.py", "-k", "not probe_library"], {"HBL_LIBRARY": str(lib)}, timeout=600)
    assert " passed" in out


def test_harness_reports_a_planted_overflow(tmp_path):
    """Control: the same build flags and runtime catch a heap overflow in a library loaded by
    the interpreter, so a clean run above means something."""
    src = tmp_path / "bad.c"
    src.write_text("#include <stdlib.h>\nint bad(void) { int* p = malloc(4 * sizeof(int)); p[4] = 1; "
                   "int r = p[0]; free(p); return r; }\n")
    lib = tmp_path / "libbad.so"
    subprocess.run(["gcc", "-fPIC", "-shared"] + SAN + ["-o", str(lib), str(src)], check=True, timeout=120)
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), ASAN_OPTIONS="detect_leaks=0")
    r = subprocess.run([sys.executable, "-c", f"import ctypes; ctypes.CDLL({str(lib)!r}).bad()"], capture_output=True,
                       text=True, timeout=120, env=env)
    assert r.returncode != 0 and ("heap-buffer-overflow" in r.stderr or "runtime error" in r.stderr)
