"""Helpers shared by the GPU parity tests: numpy <-> torch device transfer and comparisons."""
import sys

import numpy as np


def torch_mod():
    import torch

    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible AMD GPU")
    return torch


def to_dev(a: np.ndarray):
    """numpy -> contiguous CUDA tensor; uint16 arrays are taken as bf16 bit patterns."""
    torch = torch_mod()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def to_host(t) -> np.ndarray:
    torch = torch_mod()
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def note(*args):
    """Print (and flush) what names a case before its GPU work starts."""
    print("[case]", *args, file=sys.stderr, flush=True)


def rel_fro(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a - b))


def assert_close_ulps(got, want, ulps: int = 4, what: str = ""):
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    tol = np.abs(want) * (ulps * 2.0 ** -23) + 1e-37
    bad = np.abs(got.astype(np.float64) - want.astype(np.float64)) > tol
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} values differ by more than {ulps} ulp"


def code_diffs(orc, got_packed, q_o, K: int, abits: int):
    """Unpacks GPU codes and returns |GPU - oracle| per code (int32 array)."""
    got = orc.unpack_codes(np.ascontiguousarray(got_packed), K, abits).astype(np.int32)
    return np.abs(got - np.asarray(q_o, np.int32))


def assert_code_bar(orc, got_packed, q_o, K: int, abits: int, what: str = "", frac: float = 1e-4):
    """The method's bar for codes decided in another summation order: at most `frac` of the
    codes differ from the oracle's, each by one step."""
    d = code_diffs(orc, got_packed, q_o, K, abits)
    n = int((d != 0).sum())
    note(f"{what}: {n} of {d.size} codes differ ({n / max(d.size, 1):.2e}), max |diff| {int(d.max()) if d.size else 0}")
    assert d.size == 0 or d.max() <= 1, f"{what}: codes differ by {d.max()}"
    assert n <= frac * d.size, f"{what}: {n} of {d.size} codes differ"
    return n / max(d.size, 1)
