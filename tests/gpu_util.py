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


# Rows that the library transforms with its first five stages on the matrix cores (bf16 input,
# unit gamma, K = 2^10 .. 2^14 under the transform) are summed in another order than the
# oracle's fp32 butterfly loop: their codes meet the code bar (assert_code_bar) instead of
# matching bit for bit.  deq = fl(fl(fl(g / Qb) r) hK) differs by the rounding of g = max|z|
# (a few ulp) and of r, whose sum of squares is taken in fp32 over 16 exact squares per lane
# before an fp64 reduction (relative error below 15 * 2^-24, about 4 ulp of r after the square
# root): DEQ_ULPS_MFMA bounds the sum with margin.  Outputs on rows whose codes all match
# differ by deq's error plus the epilogue's two roundings: Y_ULPS_MFMA.
DEQ_ULPS_MFMA = 16
Y_ULPS_MFMA = DEQ_ULPS_MFMA + 4


def mfma_transform(x, K: int, use_h: bool, gamma=None) -> bool:
    return (bool(use_h) and np.asarray(x).dtype == np.uint16 and gamma is None and 1024 <= K <= 16384
            and (K & (K - 1)) == 0)


def check_codes(orc, got_packed, q_o, K: int, abits: int, exact: bool, what: str = ""):
    """Bit-exact packed codes, or the code bar; returns a mask of rows whose codes all match."""
    got_packed = np.ascontiguousarray(got_packed)
    if exact:
        want = orc.pack_codes(q_o, abits)
        mism = int((got_packed != want).sum())
        assert mism == 0, f"{what}: {mism} packed code bytes differ"
        return np.ones(got_packed.shape[0], bool)
    assert_code_bar(orc, got_packed, q_o, K, abits, what)
    return (code_diffs(orc, got_packed, q_o, K, abits) == 0).all(axis=1)


def assert_rows_close(y, y_o, rows_ok, exact: bool, what: str = ""):
    """The method's output bar (relative Frobenius <= 1e-3) on all rows, and on rows whose codes
    match the oracle's 4 ulp (codes decided in the oracle's order) or Y_ULPS_MFMA."""
    ulps = 4 if exact else Y_ULPS_MFMA
    err = rel_fro(y, y_o)
    note(f"{what}: relative Frobenius error {err:.3e}, {int((~rows_ok).sum())} rows with a flipped code")
    assert err <= 1e-3, f"{what}: relative Frobenius error {err}"
    assert_close_ulps(np.asarray(y)[rows_ok], np.asarray(y_o)[rows_ok], ulps, what)
