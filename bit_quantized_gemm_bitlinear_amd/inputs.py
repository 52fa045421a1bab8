"""Seeded synthetic inputs for the H-BitLinear workloads.

This module only draws random numbers and shapes them into the activation statistics the
pages describe; it contains none of the layer's arithmetic (no normalisation, transform,
quantisation or product).  Both the HIP path and the CPU oracle consume exactly the bytes
produced here.

Statistics modelled (write-up of "BitNet v2", section "H-BitLinear模塊" and Fig. 1):
the inputs of the attention output projection Wo and of the FFN down projection Wdown have
a few outlier channels while most values sit near zero; the inputs of the other linears
are close to Gaussian.  Weights are N(0, 0.02) before ternarisation.

Recipe (all draws from numpy's PCG64 ``default_rng``):
  * activations are built in float64, scaled on the outlier channels, rounded to float32
    and then to bf16 with round-to-nearest-even (the tiny exact-arithmetic workload keeps
    float32 integers);
  * the outlier channels are ``round(frac * K)`` distinct channels drawn without replacement
    from their own seed;
  * "mixture": each entry is Laplace(0, 0.05) with probability 0.6, else N(0, 1);
  * "swiglu": silu(g) * u with g, u ~ N(0, 1) (the shape of a SwiGLU output feeding Wdown);
  * "normal": N(0, 1) hidden states;
  * "int_uniform": integers uniform in [-64, 64], kept as float32.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SEED_X = 0
SEED_W = 1
SEED_OUTLIERS = 2
SEED_W_UP = 3
SEED_W_DOWN = 4


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def outlier_channels(K: int, frac: float, seed: int = SEED_OUTLIERS) -> np.ndarray:
    count = int(round(frac * K))
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(K, size=count, replace=False))


def _mixture(rng, shape):
    pick = rng.random(shape) < 0.6
    lap = rng.laplace(0.0, 0.05, shape)
    nrm = rng.standard_normal(shape)
    return np.where(pick, lap, nrm)


def _swiglu_shaped(rng, shape):
    g = rng.standard_normal(shape)
    u = rng.standard_normal(shape)
    return g / (1.0 + np.exp(-g)) * u


def make_activations(kind: str, M: int, K: int, seed: int = SEED_X, outlier_frac: float = 0.0,
                     outlier_scale: float = 1.0, outlier_seed: int = SEED_OUTLIERS) -> np.ndarray:
    """Returns float32 [M, K] for kind 'int_uniform', else bf16 bit patterns uint16 [M, K]."""
    rng = np.random.default_rng(seed)
    if kind == "int_uniform":
        return rng.integers(-64, 65, size=(M, K)).astype(np.float32)
    if kind == "mixture":
        a = _mixture(rng, (M, K))
    elif kind == "swiglu":
        a = _swiglu_shaped(rng, (M, K))
    elif kind == "normal":
        a = rng.standard_normal((M, K))
    else:
        raise ValueError(f"unknown activation kind {kind!r}")
    if outlier_frac > 0.0:
        a[:, outlier_channels(K, outlier_frac, outlier_seed)] *= outlier_scale
    return f32_to_bf16_bits(a.astype(np.float32))


def make_weights(N: int, K: int, seed: int = SEED_W, std: float = 0.02) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((N, K)) * std).astype(np.float32)


@dataclass(frozen=True)
class Workload:
    """One synthetic layer workload: shapes, flags and the activation recipe."""
    name: str
    M: int
    K: int
    N: int
    abits: tuple
    use_hadamard: bool
    norm: bool
    act_kind: str
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    description: str = ""
    extra: dict = field(default_factory=dict)

    def activations(self, M: int | None = None, seed: int = SEED_X) -> np.ndarray:
        return make_activations(self.act_kind, self.M if M is None else M, self.K, seed=seed,
                                outlier_frac=self.outlier_frac, outlier_scale=self.outlier_scale)

    def weights(self, seed: int = SEED_W) -> np.ndarray:
        return make_weights(self.N, self.K, seed=seed)


WORKLOADS = {
    "tiny_exact": Workload(
        "tiny_exact", 16, 256, 256, (4,), True, False, "int_uniform",
        description="M=16, K=N=256, a4, fp32 integer activations in [-64,64], no norm, FWHT(256): "
                    "the exact-arithmetic class"),
    "wo_1p3b": Workload(
        "wo_1p3b", 2048, 2048, 2048, (8, 4), True, True, "mixture", 0.01, 50.0,
        description="1.3B-like attention Wo: M=K=N=2048, bf16 Laplace/normal mixture, 20 outlier "
                    "channels x50, RMSNorm, FWHT(2048)"),
    "wdown_3b": Workload(
        "wdown_3b", 4096, 8192, 3072, (4,), True, True, "swiglu", 0.005, 40.0,
        description="3B-like FFN Wdown: M=4096, K=8192, N=3072, bf16 SwiGLU-shaped, 41 outlier "
                    "channels x40, RMSNorm, FWHT(8192)"),
    "wdown_7b": Workload(
        "wdown_7b", 8192, 16384, 4096, (4, 8), True, True, "mixture", 0.01, 50.0,
        description="7B-like FFN Wdown: M=8192, K=16384, N=4096, bf16 mixture, 164 outlier channels "
                    "x50, RMSNorm, FWHT(16384)"),
    "ffn_7b": Workload(
        "ffn_7b", 8192, 4096, 16384, (4,), False, True, "normal", 0.01, 30.0,
        description="7B-like a4 FFN block: M=8192, hidden 4096, ffn 16384; bf16 N(0,1) hidden states "
                    "with 41 outlier channels x30; RMSNorm -> BitLinear gate/up -> SwiGLU -> "
                    "H-BitLinear down",
        extra={"hidden": 4096, "ffn": 16384, "seed_gate": SEED_W, "seed_up": SEED_W_UP,
               "seed_down": SEED_W_DOWN}),
    "decode_7b": Workload(
        "decode_7b", 16, 16384, 4096, (4,), True, True, "mixture", 0.01, 50.0,
        description="7B-like FFN Wdown in the decode regime: 16 token rows per step (also 1, 4 and 64), "
                    "K=16384, N=4096, the wdown_7b activation recipe, a fresh weight matrix per step "
                    "(48 copies rotated, 805 MB, so weights stream from HBM)",
        extra={"batches": (1, 4, 16, 64), "weight_copies": 48}),
    "kv_7b": Workload(
        "kv_7b", 8192, 128, 32, (3,), False, False, "normal", 0.0, 1.0,
        description="7B-like K (or V) states after RoPE: 8192 tokens x 32 heads x 128, bf16 N(0,1) with a "
                    "per-head scale exp(U(-4,4)) and 3 outlier dimensions x20; unsigned absmax, 3-bit KV cache",
        extra={"heads": 32, "head_dim": 128, "bits": 3}),
}
