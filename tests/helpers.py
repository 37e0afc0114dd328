"""Shared test helpers: tolerances, case logging and device checks."""

import sys

import numpy as np
import pytest

# Tolerances on outputs compared with the float64 oracle fed identical inputs:
#   float32 path: max |gpu - ref| <= 1e-5;
#   bf16 path:    |gpu - ref| <= 2e-2 + 1e-2 * |ref| element by element.
F32_ATOL = 1e-5
BF16_ATOL = 2e-2
BF16_RTOL = 1e-2
# The bf16 kernels' row sum l adds the bf16-rounded weights, i.e. exactly the weights the P V
# product uses. Round-to-nearest-even to bf16 (8 significant bits) moves each positive weight
# by at most 2^-8 of itself, so the sum moves by at most 2^-8 of itself; the float32 scores,
# exp2 and accumulation add less than 1e-5 relative.
L_RTOL_BF16 = 2.0 ** -8 + 1e-5


def log_case(msg: str) -> None:
    """Name the case on the real stderr before a GPU step (not swallowed by capture)."""
    sys.__stderr__.write(f"[case] {msg}\n")
    sys.__stderr__.flush()


def cuda_device():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def to_np(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close(gpu, ref, dtype: str, what: str = "") -> dict:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), f"{what}: non-finite values in the GPU result"
    err = np.abs(gpu - ref)
    stats = {"max_abs": float(err.max()) if err.size else 0.0,
             "max_rel": float((err / np.maximum(np.abs(ref), 1e-30)).max()) if err.size else 0.0}
    if dtype == "f32":
        ok = err <= F32_ATOL
    else:
        ok = err <= BF16_ATOL + BF16_RTOL * np.abs(ref)
    if not ok.all():
        idx = np.unravel_index(np.argmax(err - (BF16_RTOL * np.abs(ref) if dtype != "f32" else 0)),
                               err.shape)
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} elements out of tolerance; "
                             f"max_abs {stats['max_abs']:.3e}; worst at {idx}: gpu {gpu[idx]!r} "
                             f"ref {ref[idx]!r}")
    return stats
