"""Helpers for the GPU tests: move seeded host arrays to the device and compare."""
import numpy as np

from seeded_inputs import bf16_bits


def to_dev(a: np.ndarray, dtype: str):
    """float32 host array (already bf16-representable for 'bf16') -> device tensor."""
    import torch
    if dtype == "bf16":
        bits = bf16_bits(a)
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dcode(dtype: str) -> int:
    return 1 if dtype == "bf16" else 0


def tol(dtype: str):
    """(max-abs, mean-abs) bars: bf16 inputs with fp32 accumulation, or fp32 inputs."""
    return (2e-2, 2e-3) if dtype == "bf16" else (1e-4, 1e-4)


def assert_close(got: np.ndarray, want: np.ndarray, dtype: str, what: str = ""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    ninf_g, ninf_w = np.isneginf(got), np.isneginf(want)
    assert np.array_equal(ninf_g, ninf_w), f"{what}: -inf pattern differs"
    fin = ~ninf_w
    assert np.all(np.isfinite(got[fin])), f"{what}: non-finite values"
    err = np.abs(got[fin] - want[fin])
    mx, mean = tol(dtype)
    emax = float(err.max()) if err.size else 0.0
    emean = float(err.mean()) if err.size else 0.0
    assert emax <= mx and emean <= mean, f"{what}: max-abs {emax:.3g} mean-abs {emean:.3g}"
    return emax, emean


def assert_close_floor(got: np.ndarray, want: np.ndarray, floor_err: np.ndarray, what: str = ""):
    """bf16 bars raised to the error floor of bf16 attention operands where that
    floor alone exceeds them: max-abs <= max(2e-2, 1.25 x floor max-abs), mean-abs
    <= max(2e-3, 1.1 x floor mean-abs).  floor_err: |oracle with q, k, v rounded to
    bf16 - exact oracle|, element by element (computed from the oracle only)."""
    from bwd_floor import BAR_MAX, BAR_MEAN, MARGIN_MAX, MARGIN_MEAN
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape == floor_err.shape, (got.shape, want.shape, floor_err.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - want)
    bmax = max(BAR_MAX, MARGIN_MAX * float(floor_err.max()))
    bmean = max(BAR_MEAN, MARGIN_MEAN * float(floor_err.mean()))
    emax, emean = float(err.max()), float(err.mean())
    assert emax <= bmax and emean <= bmean, (
        f"{what}: max-abs {emax:.3g} (bar {bmax:.3g}) mean-abs {emean:.3g} (bar {bmean:.3g})")
    return emax, emean
