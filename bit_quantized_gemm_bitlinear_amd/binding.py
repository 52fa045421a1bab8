"""Thin Python binding of libhbl (the C ABI in include/hbl.h).

Argument marshalling only: torch tensors provide device memory and the current HIP stream;
every step of the layer runs in libhbl's HIP kernels.  There is no fallback: if the
library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
# HBL_LIBRARY names another build of the C ABI to load instead (the sanitizer test points it
# at a host-only build of the validation layer).
LIB_PATH = os.environ.get("HBL_LIBRARY") or os.path.join(PKG, "libhbl.so")

HBL_OK, HBL_ERR_INVALID_ARG, HBL_ERR_UNSUPPORTED, HBL_ERR_WORKSPACE, HBL_ERR_HIP = range(5)
HBL_F32, HBL_BF16 = 0, 1
HBL_NORM_NONE, HBL_NORM_RMS = 0, 1
HBL_STAT_ABSMAX, HBL_STAT_ABSMEAN = 0, 1

_lock = threading.Lock()
_lib = None


class HBLError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def lib() -> ctypes.CDLL:
    """Loads libhbl.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m bit_quantized_gemm_bitlinear_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I, F, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        sig = {
            "hbl_packed_weight_bytes": (SZ, [I64, I64]),
            "hbl_packed_act_bytes": (SZ, [I64, I64, I]),
            "hbl_wquant_workspace_bytes": (SZ, [I64, I64]),
            "hbl_forward_workspace_bytes": (SZ, [I64, I64, I]),
            "hbl_quantize_weights": (I, [P, I64, I64, P, P, P, SZ, P]),
            "hbl_quantize_activations": (I, [P, I, I64, I64, I, P, F, I, I, P, P, P]),
            "hbl_gemm_s32": (I, [P, P, I64, I64, I64, I, P, P]),
            "hbl_gemm_dequant": (I, [P, P, P, P, I64, I64, I64, I, P, P]),
            "hbl_forward": (I, [P, I, P, P, I64, I64, I64, I, I, I, P, F, P, P, SZ, P]),
            "hbl_swiglu": (I, [P, P, I64, P, P]),
            "hbl_forward_fused": (I, [I64, I64, I, I]),
            "hbl_forward_noalloc": (I, [P, I, P, P, I64, I64, I64, I, I, I, P, F, P, P]),
            "hbl_quantize_activations_stat": (I, [P, I, I64, I64, I, P, F, I, I, I, P, P, P]),
            "hbl_forward_stat": (I, [P, I, P, P, I64, I64, I64, I, I, I, P, F, I, P, P, SZ, P]),
            "hbl_packed_weight_fp4_bytes": (SZ, [I64, I64]),
            "hbl_packed_act_fp6_bytes": (SZ, [I64, I64]),
            "hbl_forward_fp6fp4_workspace_bytes": (SZ, [I64, I64]),
            "hbl_weights_to_fp4": (I, [P, I64, I64, P, P]),
            "hbl_quantize_activations_fp6": (I, [P, I, I64, I64, I, P, F, I, P, P, P]),
            "hbl_gemm_fp6fp4_s32": (I, [P, P, I64, I64, I64, P, P]),
            "hbl_gemm_fp6fp4_dequant": (I, [P, P, P, P, I64, I64, I64, P, P]),
            "hbl_forward_fp6fp4": (I, [P, I, P, P, I64, I64, I64, I, I, P, F, P, P, SZ, P]),
            "hbl_packed_gate_up_bytes": (SZ, [I64, I64]),
            "hbl_interleave_gate_up": (I, [P, P, I64, I64, P, P]),
            "hbl_gate_up_swiglu": (I, [P, P, P, P, P, I64, I64, I64, I, I, P, P]),
            "hbl_ffn_workspace_bytes": (SZ, [I64, I64, I64, I, I]),
            "hbl_ffn_forward": (I, [P, I, P, P, P, P, P, I64, I64, I64, I, P, P, F, I, P, P, SZ, P]),
            "hbl_packed_qkv_bytes": (SZ, [I64, I64, I]),
            "hbl_quantize_qkv": (I, [P, I, I64, I64, I, P, P, P]),
            "hbl_dequantize_qkv": (I, [P, P, I64, I64, I, P, P]),
            "hbl_status_string": (ctypes.c_char_p, [I]),
            "hbl_last_error": (ctypes.c_char_p, []),
            "hbl_version": (I, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
        return L


def _check(status: int) -> None:
    if status != HBL_OK:
        L = lib()
        raise HBLError(status, f"{L.hbl_status_string(status).decode()}: {L.hbl_last_error().decode()}")


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream():
    import torch

    return torch.cuda.current_stream().cuda_stream


def _xdtype(x) -> int:
    import torch

    if x.dtype == torch.bfloat16:
        return HBL_BF16
    if x.dtype == torch.float32:
        return HBL_F32
    raise TypeError("activations must be torch.bfloat16 or torch.float32")


def _dev(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on the GPU")


class ShapeError(ValueError):
    """A tensor whose dtype or shape does not match what the call reads or writes (raised
    before anything is launched: the C ABI sees only pointers and cannot check extents)."""


def _want(t, name: str, dtype=None, shape=None, numel=None, optional: bool = False):
    """Checks dtype and extent of `t` (None passes when optional)."""
    import torch

    if t is None:
        if optional:
            return
        raise ShapeError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ShapeError(f"{name} must be a torch tensor")
    if dtype is not None and t.dtype != dtype:
        raise ShapeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ShapeError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() != numel:
        raise ShapeError(f"{name} must hold {numel} elements, got {t.numel()}")


def _rows(x, name: str):
    if x.dim() != 2:
        raise ShapeError(f"{name} must be 2-D, got {x.dim()}-D")
    return x.shape


def quantize_weights(W):
    """W [N, K] fp32 on the GPU -> (Wq uint8 [N, K/4], w_scale fp32 [1])."""
    import torch

    N, K = _rows(W, "W")
    _want(W, "W", torch.float32)
    _dev(W)
    L = lib()
    Wq = torch.empty((N, K // 4), dtype=torch.uint8, device=W.device)
    scale = torch.empty(1, dtype=torch.float32, device=W.device)
    wsb = L.hbl_wquant_workspace_bytes(N, K)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=W.device)
    _check(L.hbl_quantize_weights(_ptr(W), N, K, _ptr(Wq), _ptr(scale), _ptr(ws), ws.numel(), _stream()))
    return Wq, scale


def quantize_activations(x, abits: int, use_hadamard: bool, norm: bool = False, gamma=None, eps: float = 1e-5,
                         stat: int = HBL_STAT_ABSMAX):
    """x [M, K] bf16/fp32 -> (codes uint8 [M, K*abits/8], deq fp32 [M]); stat: absmax / absmean."""
    import torch

    M, K = _rows(x, "x")
    _xdtype(x)
    _want(gamma, "gamma", torch.float32, numel=K, optional=True)
    _dev(x, gamma)
    codes = torch.empty((M, K * abits // 8), dtype=torch.uint8, device=x.device)
    deq = torch.empty(M, dtype=torch.float32, device=x.device)
    _check(lib().hbl_quantize_activations_stat(_ptr(x), _xdtype(x), M, K, HBL_NORM_RMS if norm else HBL_NORM_NONE,
                                               _ptr(gamma), float(eps), int(abits), int(bool(use_hadamard)),
                                               int(stat), _ptr(codes), _ptr(deq), _stream()))
    return codes, deq


def gemm_s32(codes, Wq, K: int, abits: int):
    """codes [M, K*abits/8], Wq [N, K/4] -> acc int32 [M, N] (exact integer product)."""
    import torch

    M, N = _rows(codes, "codes")[0], _rows(Wq, "Wq")[0]
    _want(codes, "codes", torch.uint8, shape=(M, K * abits // 8))
    _want(Wq, "Wq", torch.uint8, shape=(N, K // 4))
    _dev(codes, Wq)
    acc = torch.empty((M, N), dtype=torch.int32, device=codes.device)
    _check(lib().hbl_gemm_s32(_ptr(codes), _ptr(Wq), M, K, N, int(abits), _ptr(acc), _stream()))
    return acc


def gemm_dequant(codes, deq, Wq, w_scale, K: int, abits: int, y=None):
    import torch

    M, N = _rows(codes, "codes")[0], _rows(Wq, "Wq")[0]
    _want(codes, "codes", torch.uint8, shape=(M, K * abits // 8))
    _want(Wq, "Wq", torch.uint8, shape=(N, K // 4))
    _want(deq, "deq", torch.float32, numel=M)
    _want(w_scale, "w_scale", torch.float32, numel=1)
    _want(y, "y", torch.float32, shape=(M, N), optional=True)
    _dev(codes, deq, Wq, w_scale, y)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=codes.device)
    _check(lib().hbl_gemm_dequant(_ptr(codes), _ptr(deq), _ptr(Wq), _ptr(w_scale), M, K, N, int(abits), _ptr(y),
                                  _stream()))
    return y


def forward_workspace(M: int, K: int, abits: int, device="cuda"):
    import torch

    n = lib().hbl_forward_workspace_bytes(M, K, abits)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def forward(x, Wq, w_scale, abits: int, use_hadamard: bool, norm: bool = False, gamma=None, eps: float = 1e-5,
            y=None, ws=None, stat: int = HBL_STAT_ABSMAX):
    """The whole (H-)BitLinear forward: x [M, K] -> y fp32 [M, N]."""
    import torch

    M, K = _rows(x, "x")
    _xdtype(x)
    N = _rows(Wq, "Wq")[0]
    _want(Wq, "Wq", torch.uint8, shape=(N, K // 4))
    _want(w_scale, "w_scale", torch.float32, numel=1)
    _want(gamma, "gamma", torch.float32, numel=K, optional=True)
    _want(y, "y", torch.float32, shape=(M, N), optional=True)
    _want(ws, "ws", torch.uint8, optional=True)
    _dev(x, Wq, w_scale, gamma, y, ws)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = forward_workspace(M, K, abits, x.device)
    _check(lib().hbl_forward_stat(_ptr(x), _xdtype(x), _ptr(Wq), _ptr(w_scale), M, K, N, int(abits),
                                  int(bool(use_hadamard)), HBL_NORM_RMS if norm else HBL_NORM_NONE, _ptr(gamma),
                                  float(eps), int(stat), _ptr(y), _ptr(ws), ws.numel(), _stream()))
    return y


def forward_noalloc(x, Wq, w_scale, abits: int, use_hadamard: bool, norm: bool = False, gamma=None,
                    eps: float = 1e-5, y=None):
    """hbl_forward_noalloc: the forward with its codes and deq in the library's static scratch
    (no workspace; the library allocates nothing).  y is allocated here unless given."""
    import torch

    M, K = _rows(x, "x")
    _xdtype(x)
    N = _rows(Wq, "Wq")[0]
    _want(Wq, "Wq", torch.uint8, shape=(N, K // 4))
    _want(w_scale, "w_scale", torch.float32, numel=1)
    _want(gamma, "gamma", torch.float32, numel=K, optional=True)
    _want(y, "y", torch.float32, shape=(M, N), optional=True)
    _dev(x, Wq, w_scale, gamma, y)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _check(lib().hbl_forward_noalloc(_ptr(x), _xdtype(x), _ptr(Wq), _ptr(w_scale), M, K, N, int(abits),
                                     int(bool(use_hadamard)), HBL_NORM_RMS if norm else HBL_NORM_NONE, _ptr(gamma),
                                     float(eps), _ptr(y), _stream()))
    return y


def swiglu(g, u, h=None):
    import torch

    _want(g, "g", torch.float32)
    _want(u, "u", torch.float32, numel=g.numel())
    _want(h, "h", torch.float32, numel=g.numel(), optional=True)
    _dev(g, u, h)
    if h is None:
        h = torch.empty_like(g)
    _check(lib().hbl_swiglu(_ptr(g), _ptr(u), g.numel(), _ptr(h), _stream()))
    return h


# ---- FFN block ----------------------------------------------------------------------------

def interleave_gate_up(Wq_gate, Wq_up, K: int):
    """Two packed weights [F, K/4] -> Wgu [2F, K/4], interleaved in blocks of 32 rows."""
    import torch

    F = _rows(Wq_gate, "Wq_gate")[0]
    _want(Wq_gate, "Wq_gate", torch.uint8, shape=(F, K // 4))
    _want(Wq_up, "Wq_up", torch.uint8, shape=(F, K // 4))
    _dev(Wq_gate, Wq_up)
    Wgu = torch.empty((2 * F, K // 4), dtype=torch.uint8, device=Wq_gate.device)
    _check(lib().hbl_interleave_gate_up(_ptr(Wq_gate), _ptr(Wq_up), F, K, _ptr(Wgu), _stream()))
    return Wgu


def _hdtype(h_dtype) -> int:
    import torch

    if h_dtype == torch.bfloat16:
        return HBL_BF16
    if h_dtype == torch.float32:
        return HBL_F32
    raise TypeError("h must be torch.bfloat16 or torch.float32")


def gate_up_swiglu(codes, deq, Wgu, scale_gate, scale_up, K: int, abits: int, h_dtype=None, h=None):
    """h [M, F] = silu(g) * u for the shared codes/deq and interleaved gate/up weights."""
    import torch

    M, F = _rows(codes, "codes")[0], _rows(Wgu, "Wgu")[0] // 2
    _want(codes, "codes", torch.uint8, shape=(M, K * abits // 8))
    _want(Wgu, "Wgu", torch.uint8, shape=(2 * F, K // 4))
    _want(deq, "deq", torch.float32, numel=M)
    _want(scale_gate, "scale_gate", torch.float32, numel=1)
    _want(scale_up, "scale_up", torch.float32, numel=1)
    _want(h, "h", shape=(M, F), optional=True)
    _dev(codes, deq, Wgu, scale_gate, scale_up, h)
    if h is None:
        h = torch.empty((M, F), dtype=h_dtype or torch.float32, device=codes.device)
    _check(lib().hbl_gate_up_swiglu(_ptr(codes), _ptr(deq), _ptr(Wgu), _ptr(scale_gate), _ptr(scale_up), M, K, F,
                                    int(abits), _hdtype(h.dtype), _ptr(h), _stream()))
    return h


def ffn_workspace(M: int, D: int, F: int, abits: int, h_dtype, device="cuda"):
    import torch

    n = lib().hbl_ffn_workspace_bytes(M, D, F, abits, _hdtype(h_dtype))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def ffn_forward(x, Wgu, scale_gate, scale_up, Wq_down, scale_down, abits: int = 4, h_dtype=None, gamma_in=None,
                gamma_down=None, eps: float = 1e-5, y=None, ws=None):
    """The FFN block x [M, D] -> y [M, D] fp32 (RMSNorm, gate/up, SwiGLU, H-BitLinear down)."""
    import torch

    M, D = _rows(x, "x")
    _xdtype(x)
    F = _rows(Wgu, "Wgu")[0] // 2
    _want(Wgu, "Wgu", torch.uint8, shape=(2 * F, D // 4))
    _want(Wq_down, "Wq_down", torch.uint8, shape=(D, F // 4))
    for name, t in (("scale_gate", scale_gate), ("scale_up", scale_up), ("scale_down", scale_down)):
        _want(t, name, torch.float32, numel=1)
    _want(gamma_in, "gamma_in", torch.float32, numel=D, optional=True)
    _want(gamma_down, "gamma_down", torch.float32, numel=F, optional=True)
    _want(y, "y", torch.float32, shape=(M, D), optional=True)
    _want(ws, "ws", torch.uint8, optional=True)
    _dev(x, Wgu, scale_gate, scale_up, Wq_down, scale_down, gamma_in, gamma_down, y, ws)
    h_dtype = h_dtype or torch.float32
    if y is None:
        y = torch.empty((M, D), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = ffn_workspace(M, D, F, abits, h_dtype, x.device)
    _check(lib().hbl_ffn_forward(_ptr(x), _xdtype(x), _ptr(Wgu), _ptr(scale_gate), _ptr(scale_up), _ptr(Wq_down),
                                 _ptr(scale_down), M, D, F, int(abits), _ptr(gamma_in), _ptr(gamma_down), float(eps),
                                 _hdtype(h_dtype), _ptr(y), _ptr(ws), ws.numel(), _stream()))
    return y


# ---- QKV states -----------------------------------------------------------------------------

def quantize_qkv(x, bits: int):
    """x [rows, d] (post-RoPE head vectors, bf16/fp32) -> (codes uint8 [rows, d*bits/8], gamma fp32 [rows])."""
    import torch

    rows, d = _rows(x, "x")
    _xdtype(x)
    _dev(x)
    codes = torch.empty((rows, d * bits // 8), dtype=torch.uint8, device=x.device)
    gamma = torch.empty(rows, dtype=torch.float32, device=x.device)
    _check(lib().hbl_quantize_qkv(_ptr(x), _xdtype(x), rows, d, int(bits), _ptr(codes), _ptr(gamma), _stream()))
    return codes, gamma


def dequantize_qkv(codes, gamma, d: int, bits: int):
    import torch

    rows = _rows(codes, "codes")[0]
    _want(codes, "codes", torch.uint8, shape=(rows, d * bits // 8))
    _want(gamma, "gamma", torch.float32, numel=rows)
    _dev(codes, gamma)
    out = torch.empty((rows, d), dtype=torch.float32, device=codes.device)
    _check(lib().hbl_dequantize_qkv(_ptr(codes), _ptr(gamma), rows, d, int(bits), _ptr(out), _stream()))
    return out


# ---- FP6 x FP4 a4 path -------------------------------------------------------------------

def weights_to_fp4(Wq, K: int):
    """2-bit Wq [N, K/4] -> FP4 Wq4 [N, K/2] (the weight scale is unchanged)."""
    import torch

    N = _rows(Wq, "Wq")[0]
    _want(Wq, "Wq", torch.uint8, shape=(N, K // 4))
    _dev(Wq)
    Wq4 = torch.empty((N, K // 2), dtype=torch.uint8, device=Wq.device)
    _check(lib().hbl_weights_to_fp4(_ptr(Wq), N, K, _ptr(Wq4), _stream()))
    return Wq4


def quantize_activations_fp6(x, use_hadamard: bool, norm: bool = False, gamma=None, eps: float = 1e-5):
    """x [M, K] -> (codes6 uint8 [M, 3K/4], deq fp32 [M]); the INT4 codes stored as FP6."""
    import torch

    M, K = _rows(x, "x")
    _xdtype(x)
    _want(gamma, "gamma", torch.float32, numel=K, optional=True)
    _dev(x, gamma)
    codes = torch.empty((M, K // 4 * 3), dtype=torch.uint8, device=x.device)
    deq = torch.empty(M, dtype=torch.float32, device=x.device)
    _check(lib().hbl_quantize_activations_fp6(_ptr(x), _xdtype(x), M, K, HBL_NORM_RMS if norm else HBL_NORM_NONE,
                                              _ptr(gamma), float(eps), int(bool(use_hadamard)), _ptr(codes),
                                              _ptr(deq), _stream()))
    return codes, deq


def gemm_fp6fp4_s32(codes6, Wq4, K: int):
    import torch

    M, N = _rows(codes6, "codes6")[0], _rows(Wq4, "Wq4")[0]
    _want(codes6, "codes6", torch.uint8, shape=(M, K // 4 * 3))
    _want(Wq4, "Wq4", torch.uint8, shape=(N, K // 2))
    _dev(codes6, Wq4)
    acc = torch.empty((M, N), dtype=torch.int32, device=codes6.device)
    _check(lib().hbl_gemm_fp6fp4_s32(_ptr(codes6), _ptr(Wq4), M, K, N, _ptr(acc), _stream()))
    return acc


def gemm_fp6fp4_dequant(codes6, deq, Wq4, w_scale, K: int, y=None):
    import torch

    M, N = _rows(codes6, "codes6")[0], _rows(Wq4, "Wq4")[0]
    _want(codes6, "codes6", torch.uint8, shape=(M, K // 4 * 3))
    _want(Wq4, "Wq4", torch.uint8, shape=(N, K // 2))
    _want(deq, "deq", torch.float32, numel=M)
    _want(w_scale, "w_scale", torch.float32, numel=1)
    _want(y, "y", torch.float32, shape=(M, N), optional=True)
    _dev(codes6, deq, Wq4, w_scale, y)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=codes6.device)
    _check(lib().hbl_gemm_fp6fp4_dequant(_ptr(codes6), _ptr(deq), _ptr(Wq4), _ptr(w_scale), M, K, N, _ptr(y),
                                         _stream()))
    return y


def forward_fp6fp4(x, Wq4, w_scale, use_hadamard: bool, norm: bool = False, gamma=None, eps: float = 1e-5,
                   y=None, ws=None):
    import torch

    M, K = _rows(x, "x")
    _xdtype(x)
    N = _rows(Wq4, "Wq4")[0]
    _want(Wq4, "Wq4", torch.uint8, shape=(N, K // 2))
    _want(w_scale, "w_scale", torch.float32, numel=1)
    _want(gamma, "gamma", torch.float32, numel=K, optional=True)
    _want(y, "y", torch.float32, shape=(M, N), optional=True)
    _want(ws, "ws", torch.uint8, optional=True)
    _dev(x, Wq4, w_scale, gamma, y, ws)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    if ws is None:
        n = lib().hbl_forward_fp6fp4_workspace_bytes(M, K)
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device=x.device)
    _check(lib().hbl_forward_fp6fp4(_ptr(x), _xdtype(x), _ptr(Wq4), _ptr(w_scale), M, K, N,
                                    int(bool(use_hadamard)), HBL_NORM_RMS if norm else HBL_NORM_NONE, _ptr(gamma),
                                    float(eps), _ptr(y), _ptr(ws), ws.numel(), _stream()))
    return y
