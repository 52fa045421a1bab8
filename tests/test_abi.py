"""C ABI checks that need no GPU: the library loads, exports every function the header
declares, and rejects every invalid argument synchronously with the documented status
(validation runs before any HIP call, so fake device pointers are safe here)."""
import ctypes
import math
import os
import re

import pytest

from bit_quantized_gemm_bitlinear_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hbl.h")

FAKE = 0x10000          # 64 KiB-aligned fake device address; never dereferenced
FAKE_MIS = FAKE + 4     # 4-byte aligned only
S = None                # null stream


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libhbl.so not built")
    return B.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hbl_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_expected_entry_points():
    names = declared_functions()
    for required in ["hbl_quantize_weights", "hbl_quantize_activations", "hbl_gemm_s32", "hbl_gemm_dequant",
                     "hbl_forward", "hbl_swiglu", "hbl_status_string", "hbl_last_error"]:
        assert required in names


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings(L):
    for code, name in enumerate(["HBL_OK", "HBL_ERR_INVALID_ARG", "HBL_ERR_UNSUPPORTED", "HBL_ERR_WORKSPACE",
                                 "HBL_ERR_HIP"]):
        assert L.hbl_status_string(code).decode() == name
    assert L.hbl_version() >= 100


def test_size_helpers(L):
    assert L.hbl_packed_weight_bytes(4096, 16384) == 4096 * 16384 // 4
    assert L.hbl_packed_act_bytes(8192, 16384, 4) == 8192 * 16384 // 2
    assert L.hbl_packed_act_bytes(8192, 16384, 8) == 8192 * 16384
    assert L.hbl_packed_act_bytes(3, 100, 4) == 0          # K not a multiple of 64
    assert L.hbl_packed_act_bytes(3, 128, 5) == 0          # bad abits
    assert L.hbl_wquant_workspace_bytes(4096, 16384) == 4096 * 8
    ws = L.hbl_forward_workspace_bytes(8192, 16384, 4)
    assert ws >= 8192 * 16384 // 2 + 8192 * 4 and ws % 256 == 0
    assert L.hbl_forward_workspace_bytes(0, 256, 4) == 0


def _fwd(L, x=FAKE, xt=B.HBL_BF16, Wq=FAKE, sc=FAKE, M=16, K=256, N=256, abits=4, h=1, norm=B.HBL_NORM_RMS,
         gamma=None, eps=1e-5, y=FAKE, ws=FAKE, wsb=1 << 30):
    return L.hbl_forward(x, xt, Wq, sc, M, K, N, abits, h, norm, gamma, eps, y, ws, wsb, S)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), B.HBL_ERR_INVALID_ARG),
    (dict(N=0), B.HBL_ERR_INVALID_ARG),
    (dict(K=100), B.HBL_ERR_INVALID_ARG),
    (dict(K=0), B.HBL_ERR_INVALID_ARG),
    (dict(K=262144, h=0), B.HBL_ERR_UNSUPPORTED),
    (dict(K=65536), B.HBL_ERR_UNSUPPORTED),          # Hadamard above 32768
    (dict(K=192), B.HBL_ERR_UNSUPPORTED),            # Hadamard needs a power of two
    (dict(abits=5), B.HBL_ERR_INVALID_ARG),
    (dict(abits=2), B.HBL_ERR_INVALID_ARG),
    (dict(xt=7), B.HBL_ERR_INVALID_ARG),
    (dict(norm=3), B.HBL_ERR_INVALID_ARG),
    (dict(h=2), B.HBL_ERR_INVALID_ARG),
    (dict(eps=-1.0), B.HBL_ERR_INVALID_ARG),
    (dict(eps=math.inf), B.HBL_ERR_INVALID_ARG),
    (dict(x=None), B.HBL_ERR_INVALID_ARG),
    (dict(x=FAKE_MIS), B.HBL_ERR_INVALID_ARG),
    (dict(Wq=None), B.HBL_ERR_INVALID_ARG),
    (dict(sc=None), B.HBL_ERR_INVALID_ARG),
    (dict(y=None), B.HBL_ERR_INVALID_ARG),
    (dict(y=FAKE_MIS), B.HBL_ERR_INVALID_ARG),
    (dict(gamma=FAKE_MIS), B.HBL_ERR_INVALID_ARG),
    (dict(ws=None), B.HBL_ERR_WORKSPACE),
    (dict(wsb=100), B.HBL_ERR_WORKSPACE),
    (dict(ws=FAKE + 16), B.HBL_ERR_INVALID_ARG),     # workspace must be 256-byte aligned
])
def test_forward_rejects(L, kw, status):
    assert _fwd(L, **kw) == status
    assert L.hbl_last_error().decode().startswith("hbl_forward")


def test_forward_m0_is_a_noop(L):
    assert _fwd(L, M=0, x=None, y=None, ws=None) == B.HBL_OK


def test_quantize_weights_rejects(L):
    q = L.hbl_quantize_weights
    assert q(FAKE, 0, 256, FAKE, FAKE, FAKE, 1 << 20, S) == B.HBL_ERR_INVALID_ARG
    assert q(FAKE, 4, 100, FAKE, FAKE, FAKE, 1 << 20, S) == B.HBL_ERR_INVALID_ARG
    assert q(None, 4, 256, FAKE, FAKE, FAKE, 1 << 20, S) == B.HBL_ERR_INVALID_ARG
    assert q(FAKE, 4, 256, FAKE_MIS, FAKE, FAKE, 1 << 20, S) == B.HBL_ERR_INVALID_ARG
    assert q(FAKE, 4, 256, FAKE, None, FAKE, 1 << 20, S) == B.HBL_ERR_INVALID_ARG
    assert q(FAKE, 4, 256, FAKE, FAKE, None, 1 << 20, S) == B.HBL_ERR_WORKSPACE
    assert q(FAKE, 4, 256, FAKE, FAKE, FAKE, 31, S) == B.HBL_ERR_WORKSPACE


def test_quantize_activations_rejects(L):
    q = L.hbl_quantize_activations
    args = dict(x=FAKE, xt=B.HBL_BF16, M=4, K=256, norm=0, gamma=None, eps=1e-5, abits=4, h=1, codes=FAKE, deq=FAKE)

    def call(**kw):
        a = dict(args, **kw)
        return q(a["x"], a["xt"], a["M"], a["K"], a["norm"], a["gamma"], a["eps"], a["abits"], a["h"], a["codes"],
                 a["deq"], S)

    assert call(M=-3) == B.HBL_ERR_INVALID_ARG
    assert call(K=192, h=1) == B.HBL_ERR_UNSUPPORTED
    assert call(K=96, h=1) == B.HBL_ERR_INVALID_ARG
    assert call(abits=3) == B.HBL_ERR_INVALID_ARG
    assert call(codes=None) == B.HBL_ERR_INVALID_ARG
    assert call(codes=FAKE + 8) == B.HBL_ERR_INVALID_ARG
    assert call(deq=None) == B.HBL_ERR_INVALID_ARG
    assert call(deq=FAKE + 2) == B.HBL_ERR_INVALID_ARG
    assert call(M=0, x=None, codes=None, deq=None) == B.HBL_OK


def test_gemm_rejects(L):
    assert L.hbl_gemm_s32(FAKE, FAKE, 4, 256, 0, 4, FAKE, S) == B.HBL_ERR_INVALID_ARG
    assert L.hbl_gemm_s32(FAKE, FAKE, 4, 200, 8, 4, FAKE, S) == B.HBL_ERR_INVALID_ARG
    assert L.hbl_gemm_s32(FAKE, None, 4, 256, 8, 4, FAKE, S) == B.HBL_ERR_INVALID_ARG
    assert L.hbl_gemm_s32(FAKE, FAKE, 4, 256, 8, 6, FAKE, S) == B.HBL_ERR_INVALID_ARG
    assert L.hbl_gemm_s32(FAKE, FAKE, 4, 256, 8, 4, None, S) == B.HBL_ERR_INVALID_ARG
    assert L.hbl_gemm_s32(None, FAKE, 0, 256, 8, 4, None, S) == B.HBL_OK
    assert L.hbl_gemm_dequant(FAKE, FAKE, FAKE, None, 4, 256, 8, 4, FAKE, S) == B.HBL_ERR_INVALID_ARG
    assert L.hbl_gemm_dequant(FAKE, None, FAKE, FAKE, 4, 256, 8, 4, FAKE, S) == B.HBL_ERR_INVALID_ARG
    assert L.hbl_gemm_dequant(FAKE, FAKE, FAKE, FAKE, 4, 256, (1 << 31), 4, FAKE, S) == B.HBL_ERR_INVALID_ARG


def test_swiglu_rejects(L):
    assert L.hbl_swiglu(FAKE, FAKE, -1, FAKE, S) == B.HBL_ERR_INVALID_ARG
    assert L.hbl_swiglu(None, FAKE, 16, FAKE + 4096, S) == B.HBL_ERR_INVALID_ARG
    assert L.hbl_swiglu(FAKE, FAKE + 4096, 16, FAKE + 32, S) == B.HBL_ERR_INVALID_ARG   # h overlaps g
    assert L.hbl_swiglu(None, None, 0, None, S) == B.HBL_OK


def test_last_error_is_thread_local(L):
    import threading

    assert _fwd(L, abits=5) == B.HBL_ERR_INVALID_ARG
    seen = []

    def other():
        L.hbl_quantize_activations(FAKE, 1, 4, 256, 0, None, 1e-5, 4, 1, None, FAKE, S)
        seen.append(L.hbl_last_error().decode())

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen[0].startswith("hbl_quantize_activations")
    assert "abits" in L.hbl_last_error().decode()


def test_fp6fp4_rejects(L):
    assert L.hbl_packed_weight_fp4_bytes(8, 256) == 8 * 128
    assert L.hbl_packed_act_fp6_bytes(8, 256) == 8 * 192
    assert L.hbl_packed_act_fp6_bytes(8, 100) == 0
    assert L.hbl_weights_to_fp4(FAKE, 0, 256, FAKE, S) == B.HBL_ERR_INVALID_ARG
    assert L.hbl_weights_to_fp4(FAKE, 8, 256, FAKE_MIS, S) == B.HBL_ERR_INVALID_ARG
    q6 = L.hbl_quantize_activations_fp6
    assert q6(FAKE, 1, 4, 192, 0, None, 1e-5, 1, FAKE, FAKE, S) == B.HBL_ERR_UNSUPPORTED
    assert q6(FAKE, 1, 4, 256, 0, None, 1e-5, 1, None, FAKE, S) == B.HBL_ERR_INVALID_ARG
    assert q6(None, 1, 0, 256, 0, None, 1e-5, 1, None, None, S) == B.HBL_OK
    assert L.hbl_gemm_fp6fp4_s32(FAKE, FAKE, 4, 200, 8, FAKE, S) == B.HBL_ERR_INVALID_ARG
    assert L.hbl_gemm_fp6fp4_dequant(FAKE, FAKE, FAKE, None, 4, 256, 8, FAKE, S) == B.HBL_ERR_INVALID_ARG
    f = L.hbl_forward_fp6fp4
    assert f(FAKE, 1, FAKE, FAKE, 4, 256, 8, 1, 1, None, 1e-5, FAKE, FAKE, 100, S) == B.HBL_ERR_WORKSPACE
    assert f(FAKE, 1, FAKE, FAKE, 4, 256, 8, 2, 1, None, 1e-5, FAKE, FAKE, 1 << 20, S) == B.HBL_ERR_INVALID_ARG


def test_ffn_size_helpers(L):
    assert L.hbl_packed_gate_up_bytes(16384, 4096) == 2 * 16384 * 1024
    assert L.hbl_packed_gate_up_bytes(48, 256) == 0                     # F % 32 != 0
    ws = L.hbl_ffn_workspace_bytes(8192, 4096, 16384, 4, B.HBL_BF16)
    assert ws >= 8192 * 2048 + 8192 * 4 + 8192 * 16384 * 2 + 8192 * 8192 + 8192 * 4 and ws % 256 == 0
    assert L.hbl_ffn_workspace_bytes(8, 4096, 12288, 4, B.HBL_BF16) == 0  # F not a power of two


def test_gate_up_rejects(L):
    il = L.hbl_interleave_gate_up
    assert il(FAKE, FAKE + (1 << 24), 48, 256, FAKE + (1 << 25), S) == B.HBL_ERR_INVALID_ARG
    assert il(FAKE, FAKE + (1 << 24), 64, 256, FAKE + 1024, S) == B.HBL_ERR_INVALID_ARG    # Wgu overlaps gate
    assert il(FAKE, None, 64, 256, FAKE + (1 << 25), S) == B.HBL_ERR_INVALID_ARG
    g = L.hbl_gate_up_swiglu
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 256, 40, 4, 1, FAKE, S) == B.HBL_ERR_INVALID_ARG   # F % 32
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 256, 64, 4, 5, FAKE, S) == B.HBL_ERR_INVALID_ARG   # h dtype
    assert g(FAKE, FAKE, FAKE, None, FAKE, 4, 256, 64, 4, 1, FAKE, S) == B.HBL_ERR_INVALID_ARG
    assert g(FAKE, FAKE, FAKE, FAKE, None, 4, 256, 64, 4, 1, FAKE, S) == B.HBL_ERR_INVALID_ARG
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 256, 64, 4, 1, FAKE_MIS, S) == B.HBL_ERR_INVALID_ARG
    assert g(None, None, FAKE, FAKE, FAKE, 0, 256, 64, 4, 1, None, S) == B.HBL_OK


def _ffn(L, x=FAKE, xt=B.HBL_BF16, M=16, D=256, F=512, abits=4, ht=B.HBL_BF16, y=FAKE, ws=FAKE, wsb=1 << 30,
         gi=None, gd=None, eps=1e-5):
    return L.hbl_ffn_forward(x, xt, FAKE, FAKE, FAKE, FAKE, FAKE, M, D, F, abits, gi, gd, eps, ht, y, ws, wsb, S)


@pytest.mark.parametrize("kw,status", [
    (dict(F=768), B.HBL_ERR_UNSUPPORTED),             # the down projection's transform needs a power of two
    (dict(F=65536), B.HBL_ERR_UNSUPPORTED),
    (dict(D=200), B.HBL_ERR_INVALID_ARG),
    (dict(abits=6), B.HBL_ERR_INVALID_ARG),
    (dict(ht=9), B.HBL_ERR_INVALID_ARG),
    (dict(xt=9), B.HBL_ERR_INVALID_ARG),
    (dict(gd=FAKE_MIS), B.HBL_ERR_INVALID_ARG),
    (dict(y=None), B.HBL_ERR_INVALID_ARG),
    (dict(wsb=1000), B.HBL_ERR_WORKSPACE),
    (dict(ws=FAKE + 64), B.HBL_ERR_INVALID_ARG),
    (dict(M=0, x=None, y=None, ws=None), B.HBL_OK),
])
def test_ffn_forward_rejects(L, kw, status):
    assert _ffn(L, **kw) == status


def test_qkv_rejects(L):
    assert L.hbl_packed_qkv_bytes(10, 128, 3) == 10 * 48
    assert L.hbl_packed_qkv_bytes(10, 96, 3) == 0
    q = L.hbl_quantize_qkv
    assert q(FAKE, 1, 10, 96, 3, FAKE, FAKE, S) == B.HBL_ERR_UNSUPPORTED
    assert q(FAKE, 1, 10, 128, 9, FAKE, FAKE, S) == B.HBL_ERR_INVALID_ARG
    assert q(FAKE, 1, 10, 128, 1, FAKE, FAKE, S) == B.HBL_ERR_INVALID_ARG
    assert q(FAKE, 5, 10, 128, 3, FAKE, FAKE, S) == B.HBL_ERR_INVALID_ARG
    assert q(FAKE, 1, -1, 128, 3, FAKE, FAKE, S) == B.HBL_ERR_INVALID_ARG
    assert q(FAKE_MIS, 1, 10, 128, 3, FAKE, FAKE, S) == B.HBL_ERR_INVALID_ARG
    assert q(FAKE, 1, 10, 128, 3, None, FAKE, S) == B.HBL_ERR_INVALID_ARG
    assert q(None, 1, 0, 128, 3, None, None, S) == B.HBL_OK
    dq = L.hbl_dequantize_qkv
    assert dq(FAKE, FAKE, 10, 128, 3, FAKE_MIS, S) == B.HBL_ERR_INVALID_ARG
    assert dq(FAKE, None, 10, 128, 3, FAKE, S) == B.HBL_ERR_INVALID_ARG


def test_forward_fused_query(L):
    # one fused kernel only with the transform, K in 4096..16384 and M <= 256 / (K / 64)
    assert L.hbl_forward_fused(1, 16384, 4, 1) == 1
    assert L.hbl_forward_fused(2, 16384, 4, 1) == 0
    assert L.hbl_forward_fused(2, 8192, 8, 1) == 1
    assert L.hbl_forward_fused(4, 4096, 4, 1) == 1
    assert L.hbl_forward_fused(5, 4096, 4, 1) == 0
    assert L.hbl_forward_fused(1, 2048, 4, 1) == 0
    assert L.hbl_forward_fused(1, 16384, 4, 0) == 0
    assert L.hbl_forward_fused(0, 16384, 4, 1) == 0
    assert L.hbl_forward_fused(1, 12288, 4, 1) == 0


def test_stat_rejects(L):
    q = L.hbl_quantize_activations_stat
    assert q(FAKE, 1, 4, 256, 0, None, 1e-5, 4, 1, 2, FAKE, FAKE, S) == B.HBL_ERR_INVALID_ARG      # unknown stat
    assert q(FAKE, 1, 4, 256, 0, None, 1e-5, 8, 1, 1, FAKE, FAKE, S) == B.HBL_ERR_UNSUPPORTED      # absmean needs a4
    assert q(None, 1, 0, 256, 0, None, 1e-5, 4, 1, 1, None, None, S) == B.HBL_OK
    f = L.hbl_forward_stat
    assert f(FAKE, 1, FAKE, FAKE, 4, 256, 8, 4, 1, 1, None, 1e-5, 3, FAKE, FAKE, 1 << 20, S) == B.HBL_ERR_INVALID_ARG
    assert f(FAKE, 1, FAKE, FAKE, 4, 256, 8, 8, 1, 1, None, 1e-5, 1, FAKE, FAKE, 1 << 20, S) == B.HBL_ERR_UNSUPPORTED
    assert f(FAKE, 1, FAKE, FAKE, 4, 256, 8, 4, 1, 1, None, 1e-5, 1, FAKE, FAKE, 10, S) == B.HBL_ERR_WORKSPACE


def test_zero_rows_are_noops_everywhere(L):
    """M = 0 (rows = 0, n = 0) is valid for every per-row call and returns HBL_OK without
    touching the row buffers, which may then be null; the shape arguments are still checked."""
    K, N, F = 256, 64, 64
    assert L.hbl_gemm_dequant(None, None, FAKE, FAKE, 0, K, N, 4, None, S) == B.HBL_OK
    assert L.hbl_quantize_activations_stat(None, B.HBL_BF16, 0, K, 0, None, 1e-5, 4, 1, B.HBL_STAT_ABSMEAN, None,
                                           None, S) == B.HBL_OK
    assert L.hbl_forward_stat(None, B.HBL_BF16, FAKE, FAKE, 0, K, N, 4, 1, 0, None, 1e-5, B.HBL_STAT_ABSMEAN, None,
                              None, 0, S) == B.HBL_OK
    assert L.hbl_swiglu(None, None, 0, None, S) == B.HBL_OK
    assert L.hbl_gate_up_swiglu(None, None, FAKE, FAKE, FAKE, 0, K, F, 4, B.HBL_BF16, None, S) == B.HBL_OK
    assert L.hbl_quantize_activations_fp6(None, B.HBL_BF16, 0, K, 0, None, 1e-5, 1, None, None, S) == B.HBL_OK
    assert L.hbl_gemm_fp6fp4_s32(None, FAKE, 0, K, N, None, S) == B.HBL_OK
    assert L.hbl_gemm_fp6fp4_dequant(None, None, FAKE, FAKE, 0, K, N, None, S) == B.HBL_OK
    assert L.hbl_forward_fp6fp4(None, B.HBL_BF16, FAKE, FAKE, 0, K, N, 1, 0, None, 1e-5, None, None, 0, S) == B.HBL_OK
    assert L.hbl_quantize_qkv(None, B.HBL_BF16, 0, 128, 3, None, None, S) == B.HBL_OK
    assert L.hbl_dequantize_qkv(None, None, 0, 128, 3, None, S) == B.HBL_OK
    # the shape is still validated when there are no rows
    assert L.hbl_gemm_fp6fp4_s32(None, FAKE, 0, 100, N, None, S) == B.HBL_ERR_INVALID_ARG
    assert L.hbl_quantize_qkv(None, B.HBL_BF16, 0, 128, 9, None, None, S) == B.HBL_ERR_INVALID_ARG


def test_probe_library_exports_its_entry_point():
    """The measurement aid next to the library (the MFMA-only ceiling bench.py reports)."""
    path = os.path.join(os.path.dirname(B.LIB_PATH), "libhbl_probe.so")
    if not os.path.exists(path):
        pytest.skip("libhbl_probe.so not built")
    lib = ctypes.CDLL(path)
    f = lib.hbl_probe_mfma_ceiling
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert f(None, 1, 1, FAKE, S) == 1 and f(FAKE, 0, 1, FAKE, S) == 1   # rejected before any HIP call


def test_forward_noalloc_rejects(L):
    def call(M=16, K=256, N=256, abits=4, h=1, x=FAKE, y=FAKE, xt=B.HBL_BF16):
        return L.hbl_forward_noalloc(x, xt, FAKE, FAKE, M, K, N, abits, h, B.HBL_NORM_RMS, None, 1e-5, y, S)
    # the 7B Wdown batch in INT8 needs 128 MiB of codes: above the static scratch, refused
    assert call(M=8192, K=16384, N=4096, abits=8) == B.HBL_ERR_UNSUPPORTED
    assert "HBL_NOALLOC_SCRATCH_BYTES" in L.hbl_last_error().decode()
    assert L.hbl_forward_workspace_bytes(8192, 16384, 4) <= 80 << 20    # ... while INT4 fits
    assert call(M=-1) == B.HBL_ERR_INVALID_ARG
    assert call(K=192) == B.HBL_ERR_UNSUPPORTED
    assert call(abits=5) == B.HBL_ERR_INVALID_ARG
    assert call(x=None) == B.HBL_ERR_INVALID_ARG
    assert call(y=FAKE_MIS) == B.HBL_ERR_INVALID_ARG
    assert call(M=0, x=None, y=None) == B.HBL_OK
