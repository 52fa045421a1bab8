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
