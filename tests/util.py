"""Shared helpers of the tests: moving seeded workload tensors to the GPU and the float64
comparison metric.  No step of the block's arithmetic lives here."""
import math
import sys
import time

import numpy as np
import torch

import workloads as wl

TOL = {wl.F32: 1e-4, wl.BF16: 2e-2}
SIG_BITS = {torch.bfloat16: 8, torch.float16: 11, torch.float32: 24}


def log(*a):
    print(f"[{time.strftime('%H:%M:%S')}]", *a, flush=True)
    sys.stdout.flush()


def to_dev(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Stored workload tensor -> torch tensor on the GPU with the same bytes."""
    if dtype == wl.BF16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def to_host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = math.sqrt(float(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref))) / rms


def assert_close(name, got, ref, tol):
    e = rel_err(got, ref)
    log(f"  {name}: max|err|/rms = {e:.3e} (tol {tol:.0e})")
    assert np.all(np.isfinite(np.asarray(got))), f"{name}: non-finite values"
    assert e <= tol, f"{name}: max|err|/rms {e:.3e} > {tol:.0e}"
    return e


def half_ulp(ref: np.ndarray, dtype) -> np.ndarray:
    """Half the spacing of `dtype` around |ref| (round-to-nearest bound of storing ref)."""
    p = SIG_BITS[dtype]
    e = np.frexp(np.abs(ref))[1]
    h = np.ldexp(0.5, e - p)
    if dtype == torch.float16:
        h = np.maximum(h, 2.0 ** -25)
    return h


def assert_close_stored(name, got, ref, dtype, tol):
    """Parity of a result that is stored in `dtype`: the error beyond the unavoidable
    rounding to `dtype` (half an ulp at |ref|), relative to rms(ref), must be <= tol.  The
    plain max|err|/rms is logged beside it."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = math.sqrt(float(np.mean(ref * ref)))
    excess = np.maximum(np.abs(got - ref) - half_ulp(ref, dtype), 0.0)
    e = float(excess.max()) / rms
    log(f"  {name} [{str(dtype).replace('torch.', '')}]: error beyond storage rounding / rms = {e:.3e} "
        f"(tol {tol:.0e}); plain max|err|/rms = {rel_err(got, ref):.3e}")
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert e <= tol, f"{name}: {e:.3e} > {tol:.0e}"
    return e


def parity_rows(n: int, k: int, seed: int, bands=()) -> np.ndarray:
    """Sorted distinct query rows of a sampled full-size comparison: the first and last 32
    rows, every row of each (start, stop, step) band, then seeded random rows until there
    are k in all (every row when k >= n)."""
    if k >= n:
        return np.arange(n)
    must = [np.arange(min(32, n)), np.arange(max(0, n - 32), n)]
    for a, b, s in bands:
        must.append(np.arange(max(0, a), min(n, b), s))
    must = np.unique(np.concatenate(must))
    rest = np.setdiff1d(np.arange(n), must)
    extra = max(0, k - must.size)
    rng = np.random.default_rng(seed)
    pick = rng.choice(rest, size=min(extra, rest.size), replace=False)
    return np.unique(np.concatenate([must, pick]))
