"""ctypes front end of the C oracle (hbl_oracle.c).  Test infrastructure only.

Every function takes and returns numpy arrays.  Activations are either float32 arrays or
bf16 bit patterns held in uint16 arrays (``dtype`` = BF16).  Nothing here does any of the
method's arithmetic except :func:`dense_reference`, the fp64 "unquantised" reference used
to bound quantisation error (it follows the same pages: RMSNorm, then the orthonormal
Hadamard transform, then the product with the dequantised ternary weights).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

F32 = 0
BF16 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hbl_oracle.c")
# HBL_ORACLE_LIB names another build of hbl_oracle.c to load instead (the mutation tests
# point it at copies with a planted mistake); build() then leaves it as it is.
_LIB = os.environ.get("HBL_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def lib_path() -> str:
    return _LIB


def compile_command(src: str, out: str) -> list:
    return ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-Wall",
            "-Wextra", "-o", out, src, "-lm"]


def build(force: bool = False) -> str:
    """Compile hbl_oracle.c with gcc (plain C11, OpenMP, no FMA contraction, no fast-math)."""
    if os.environ.get("HBL_ORACLE_LIB"):
        return _LIB
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        cmd = compile_command(_SRC, tmp)
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        Fl = ctypes.c_float
        lib.orc_num_threads.restype = I
        lib.orc_set_num_threads.argtypes = [I]
        lib.orc_fwht_f32.argtypes = [P, I64]
        lib.orc_fwht_f64.argtypes = [P, I64]
        lib.orc_quantize_weights.argtypes = [P, I64, I64, P, P]
        lib.orc_quantize_weights.restype = I
        lib.orc_quantize_activations_stat.argtypes = [P, I, I64, I64, I, P, Fl, I, I, I, P, P, P]
        lib.orc_quantize_activations_stat.restype = I
        lib.orc_gemm_s32.argtypes = [P, P, I64, I64, I64, P]
        lib.orc_gemm_s32.restype = I
        lib.orc_dequant.argtypes = [P, P, Fl, I64, I64, P]
        lib.orc_dequant.restype = I
        lib.orc_forward_stat.argtypes = [P, I, P, Fl, I64, I64, I64, I, I, I, P, Fl, I, P, P, P, P]
        lib.orc_forward_stat.restype = I
        lib.orc_swiglu.argtypes = [P, P, I64, P]
        lib.orc_round_bf16.argtypes = [P, I64, P]
        lib.orc_quantize_qkv.argtypes = [P, I, I64, I64, I, P, P]
        lib.orc_quantize_qkv.restype = I
        lib.orc_dequantize_qkv.argtypes = [P, P, I64, I64, I, P]
        lib.orc_dequantize_qkv.restype = I
        lib.orc_pack_bits.argtypes = [P, I64, I64, I, P]
        lib.orc_pack_bits.restype = I
        lib.orc_unpack_bits.argtypes = [P, I64, I64, I, P]
        lib.orc_unpack_bits.restype = I
        lib.orc_pack_weights.argtypes = [P, I64, I64, P]
        lib.orc_pack_weights.restype = I
        lib.orc_unpack_weights.argtypes = [P, I64, I64, P]
        lib.orc_unpack_weights.restype = I
        lib.orc_pack_codes.argtypes = [P, I64, I64, I, P]
        lib.orc_pack_codes.restype = I
        lib.orc_unpack_codes.argtypes = [P, I64, I64, I, P]
        lib.orc_unpack_codes.restype = I
        lib.orc_pack_codes_fp6.argtypes = [P, I64, I64, P]
        lib.orc_pack_codes_fp6.restype = I
        lib.orc_unpack_codes_fp6.argtypes = [P, I64, I64, P]
        lib.orc_unpack_codes_fp6.restype = I
        lib.orc_pack_weights_fp4.argtypes = [P, I64, I64, P]
        lib.orc_pack_weights_fp4.restype = I
        _lib = lib
        return lib


def _p(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(_load().orc_num_threads())


def set_num_threads(n: int) -> None:
    _load().orc_set_num_threads(int(n))


def _xdtype(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.uint16:
        return BF16
    raise TypeError("activations must be float32 or uint16 (bf16 bit patterns)")


def fwht_f32(v) -> np.ndarray:
    """Unnormalised Sylvester-order FWHT in fp32, ascending butterfly stages (copy)."""
    out = _c(v, np.float32).copy()
    n = out.shape[-1]
    rows = out.reshape(-1, n)
    for r in rows:
        _load().orc_fwht_f32(_p(r), n)
    return out


def fwht_f64(v) -> np.ndarray:
    out = _c(v, np.float64).copy()
    n = out.shape[-1]
    rows = out.reshape(-1, n)
    for r in rows:
        _load().orc_fwht_f64(_p(r), n)
    return out


def quantize_weights(W) -> tuple[np.ndarray, float]:
    """Per-tensor absmean ternarisation: returns (t int8 [N,K], alpha)."""
    W = _c(W, np.float32)
    N, K = W.shape
    T = np.empty((N, K), np.int8)
    a = np.zeros(1, np.float32)
    if _load().orc_quantize_weights(_p(W), N, K, _p(T), _p(a)) != 0:
        raise ValueError("orc_quantize_weights: bad arguments")
    return T, float(a[0])


def quantize_activations(x, abits: int, use_h: bool, norm: bool = False, gamma=None, eps: float = 1e-5,
                         stat: int = 0):
    """Returns (q int8 [M,K] unpacked, deq f32 [M], r f32 [M]).  stat: 0 absmax, 1 absmean."""
    x = np.ascontiguousarray(x)
    M, K = x.shape
    q = np.empty((M, K), np.int8)
    deq = np.empty(M, np.float32)
    r = np.empty(M, np.float32)
    g = None if gamma is None else _c(gamma, np.float32)
    rc = _load().orc_quantize_activations_stat(_p(x), _xdtype(x), M, K, int(bool(norm)), _p(g), float(eps),
                                               int(abits), int(bool(use_h)), int(stat), _p(q), _p(deq), _p(r))
    if rc != 0:
        raise ValueError("orc_quantize_activations: bad arguments")
    return q, deq, r


def gemm_s32(q, T) -> np.ndarray:
    q = _c(q, np.int8)
    T = _c(T, np.int8)
    M, K = q.shape
    N, K2 = T.shape
    assert K == K2
    acc = np.empty((M, N), np.int32)
    if _load().orc_gemm_s32(_p(q), _p(T), M, K, N, _p(acc)) != 0:
        raise ValueError("orc_gemm_s32: bad arguments")
    return acc


def dequant(acc, deq, alpha: float) -> np.ndarray:
    acc = _c(acc, np.int32)
    deq = _c(deq, np.float32)
    M, N = acc.shape
    y = np.empty((M, N), np.float32)
    _load().orc_dequant(_p(acc), _p(deq), float(alpha), M, N, _p(y))
    return y


def forward(x, T, alpha: float, abits: int, use_h: bool, norm: bool = False, gamma=None, eps: float = 1e-5,
            intermediates: bool = False, stat: int = 0):
    """Whole forward on the rows of x.  Returns y, or (y, q, acc, deq) with intermediates."""
    x = np.ascontiguousarray(x)
    T = _c(T, np.int8)
    M, K = x.shape
    N = T.shape[0]
    y = np.empty((M, N), np.float32)
    q = np.empty((M, K), np.int8) if intermediates else None
    acc = np.empty((M, N), np.int32) if intermediates else None
    deq = np.empty(M, np.float32) if intermediates else None
    g = None if gamma is None else _c(gamma, np.float32)
    rc = _load().orc_forward_stat(_p(x), _xdtype(x), _p(T), float(alpha), M, K, N, int(abits), int(bool(use_h)),
                                  int(bool(norm)), _p(g), float(eps), int(stat), _p(y), _p(q), _p(acc), _p(deq))
    if rc != 0:
        raise ValueError("orc_forward: bad arguments")
    return (y, q, acc, deq) if intermediates else y


def swiglu(g, u) -> np.ndarray:
    g = _c(g, np.float32)
    u = _c(u, np.float32)
    assert g.shape == u.shape
    h = np.empty_like(g)
    _load().orc_swiglu(_p(g), _p(u), g.size, _p(h))
    return h


def round_bf16(a) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    a = _c(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    _load().orc_round_bf16(_p(a), a.size, _p(out))
    return out


def ffn_forward(x, Tg, ag: float, Tu, au: float, Td, ad: float, abits: int = 4, h_bf16: bool = True,
                gamma_in=None, gamma_down=None, eps: float = 1e-5, intermediates: bool = False):
    """The BitNet v2 FFN block (write-up section "BitNet v2：原生4位激活": RMSNorm, SwishGLU,
    no biases; only the down projection is an H-BitLinear):

        g = BitLinear_gate(RMSNorm(x)), u = BitLinear_up(RMSNorm(x))   (no transform)
        h = silu(g) * u                                                  (fp32; bf16 if h_bf16)
        y = H-BitLinear_down(h)                                          (RMSNorm, FWHT over F)

    Returns y, or (y, h) with intermediates."""
    g = forward(x, Tg, ag, abits, False, norm=True, gamma=gamma_in, eps=eps)
    u = forward(x, Tu, au, abits, False, norm=True, gamma=gamma_in, eps=eps)
    h = swiglu(g, u)
    if h_bf16:
        h = round_bf16(h)
    y = forward(h, Td, ad, abits, True, norm=True, gamma=gamma_down, eps=eps)
    return (y, h) if intermediates else y


def quantize_qkv(x, bits: int):
    """Per-head unsigned absmax quantisation of post-RoPE Q/K/V head vectors.

    x: [rows, d] float32 or bf16 patterns (one row per token and head).
    Returns (u uint8 [rows, d] unpacked codes in 0 .. 2^bits - 1, gamma f32 [rows])."""
    x = np.ascontiguousarray(x)
    rows, d = x.shape
    u = np.empty((rows, d), np.uint8)
    g = np.empty(rows, np.float32)
    if _load().orc_quantize_qkv(_p(x), _xdtype(x), rows, d, int(bits), _p(u), _p(g)) != 0:
        raise ValueError("orc_quantize_qkv: bad arguments")
    return u, g


def dequantize_qkv(u, gamma, bits: int) -> np.ndarray:
    u = _c(u, np.uint8)
    gamma = _c(gamma, np.float32)
    rows, d = u.shape
    out = np.empty((rows, d), np.float32)
    if _load().orc_dequantize_qkv(_p(u), _p(gamma), rows, d, int(bits), _p(out)) != 0:
        raise ValueError("orc_dequantize_qkv: bad arguments")
    return out


def pack_bits(u, bits: int) -> np.ndarray:
    u = _c(u, np.uint8)
    rows, d = u.shape
    out = np.empty((rows, d * bits // 8), np.uint8)
    if _load().orc_pack_bits(_p(u), rows, d, int(bits), _p(out)) != 0:
        raise ValueError("orc_pack_bits: bad arguments or code out of range")
    return out


def unpack_bits(packed, d: int, bits: int) -> np.ndarray:
    packed = _c(packed, np.uint8)
    rows = packed.shape[0]
    u = np.empty((rows, d), np.uint8)
    if _load().orc_unpack_bits(_p(packed), rows, d, int(bits), _p(u)) != 0:
        raise ValueError("orc_unpack_bits: bad arguments")
    return u


def pack_weights(T) -> np.ndarray:
    T = _c(T, np.int8)
    N, K = T.shape
    Wq = np.empty((N, K // 4), np.uint8)
    if _load().orc_pack_weights(_p(T), N, K, _p(Wq)) != 0:
        raise ValueError("orc_pack_weights: bad arguments")
    return Wq


def unpack_weights(Wq, K: int) -> np.ndarray:
    Wq = _c(Wq, np.uint8)
    N = Wq.shape[0]
    T = np.empty((N, K), np.int8)
    if _load().orc_unpack_weights(_p(Wq), N, K, _p(T)) != 0:
        raise ValueError("orc_unpack_weights: bad arguments")
    return T


def pack_codes(q, abits: int) -> np.ndarray:
    q = _c(q, np.int8)
    M, K = q.shape
    out = np.empty((M, K * abits // 8), np.uint8)
    if _load().orc_pack_codes(_p(q), M, K, int(abits), _p(out)) != 0:
        raise ValueError("orc_pack_codes: bad arguments")
    return out


def unpack_codes(codes, K: int, abits: int) -> np.ndarray:
    codes = _c(codes, np.uint8)
    M = codes.shape[0]
    q = np.empty((M, K), np.int8)
    if _load().orc_unpack_codes(_p(codes), M, K, int(abits), _p(q)) != 0:
        raise ValueError("orc_unpack_codes: bad arguments")
    return q


def pack_codes_fp6(q) -> np.ndarray:
    """INT4 codes (|q| <= 7) -> FP6 E2M3, 6 bits per code, rows of 3K/4 bytes."""
    q = _c(q, np.int8)
    M, K = q.shape
    out = np.empty((M, K // 4 * 3), np.uint8)
    if _load().orc_pack_codes_fp6(_p(q), M, K, _p(out)) != 0:
        raise ValueError("orc_pack_codes_fp6: bad arguments or code out of range")
    return out


def unpack_codes_fp6(codes, K: int) -> np.ndarray:
    codes = _c(codes, np.uint8)
    M = codes.shape[0]
    q = np.empty((M, K), np.int8)
    if _load().orc_unpack_codes_fp6(_p(codes), M, K, _p(q)) != 0:
        raise ValueError("orc_unpack_codes_fp6: bad arguments")
    return q


def pack_weights_fp4(T) -> np.ndarray:
    """Ternary weights -> FP4 E2M1 nibbles, weight k in nibble k (low first)."""
    T = _c(T, np.int8)
    N, K = T.shape
    out = np.empty((N, K // 2), np.uint8)
    if _load().orc_pack_weights_fp4(_p(T), N, K, _p(out)) != 0:
        raise ValueError("orc_pack_weights_fp4: bad arguments")
    return out


def dense_reference(x, T, alpha: float, use_h: bool, norm: bool = False, gamma=None, eps: float = 1e-5):
    """fp64 layer output without activation quantisation: y* = (H_K/sqrt(K)) RMSNorm(x) . (alpha t)^T.

    It is what the quantised forward approximates; tests use it to bound the error of the
    INT4 / INT8 paths.
    """
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    else:
        xf = x.astype(np.float64)
    K = xf.shape[1]
    u = xf
    if norm:
        r = 1.0 / np.sqrt((xf * xf).sum(axis=1, keepdims=True) / K + eps)
        u = xf * (1.0 if gamma is None else np.asarray(gamma, np.float64)) * r
    if use_h:
        u = fwht_f64(u) / np.sqrt(K)
    return u @ (alpha * np.asarray(T, np.float64)).T
