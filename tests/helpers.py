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


# e4m3 weights (fa_fwd_fp8 with e4m3 V). The kernel rounds every weight w_j (the exponential of
# a score against the row's current exponent reference r) to e4m3 before P V, and takes its
# row sum l from the same rounded weights, so the output is the convex combination
# O~ = sum_j w~_j v_j / sum_j w~_j. The reference only moves to 2^4 below a row maximum, so
# r <= 2^-4 w_max (w_max: the row's largest weight, in the same units); the weights stay at
# most 2^8 r, inside e4m3's range. Rounding to nearest moves a weight in e4m3's normal range
# (>= 2^-6 r) by at most 2^-4 of itself (3 stored mantissa bits), and a smaller one by at most
# half the subnormal step, 2^-10 r <= 2^-14 w_max, and never by more than itself (it rounds to
# 0 at worst). With b_j = min(w_j, max(2^-4 w_j, 2^-14 w_max)) + 1e-5 w_j (the last term for
# the float32 score and exp2 that feed the rounding), and the weights normalised to sum 1:
#   O~ - O = sum_j (w~_j - w_j)(v_j - O) / sum_j w~_j
#   |O~ - O| <= sum_j b_j |v_j - O| / (1 - sum_j b_j)          (element by element)
#   |l~ / l - 1| <= sum_j b_j.
# The float32 accumulation over the key tiles and the bf16 rounding of the output come on top.
E4M3_REL = 2.0 ** -4
E4M3_FLOOR = 2.0 ** -14
E4M3_EXP_SLACK = 1e-5


def e4m3_weight_bounds(w: np.ndarray, v: np.ndarray, o: np.ndarray, chunk: int = 32):
    """Bounds of the e4m3-weight rounding for rows of normalised weights w [R, Nk] over values
    v [Nk, d] with exact outputs o [R, d]: (element-wise bound on |O~ - O| [R, d], bound on
    |l~ / l - 1| [R])."""
    w = np.asarray(w, np.float64)
    v = np.asarray(v, np.float64)
    o = np.asarray(o, np.float64)
    wmax = w.max(axis=1, keepdims=True)
    b = np.minimum(w, np.maximum(E4M3_REL * w, E4M3_FLOOR * wmax)) + E4M3_EXP_SLACK * w
    sb = b.sum(axis=1)
    assert np.all(sb < 0.5), "the bound assumes the rounded weights keep most of the row sum"
    num = np.empty_like(o)
    for r0 in range(0, w.shape[0], chunk):
        r1 = min(r0 + chunk, w.shape[0])
        dev = np.abs(v[None, :, :] - o[r0:r1, None, :])
        num[r0:r1] = np.einsum("rk,rkd->rd", b[r0:r1], dev)
    return num / (1.0 - sb)[:, None], sb


def e4m3_output_tolerance(w, v, o, n_keys: int):
    """Element-wise tolerance of an e4m3-weight output: the rounding bound above, the float32
    accumulation (one add per 64-key tile plus the products inside a matrix instruction and the
    final division, each at most 2^-24 relative, of a sum bounded by max |v|) and the bf16
    rounding of the output (half an ulp: 2^-8 relative, bf16 keeping 8 significant bits).
    Returns (tolerance [R, d], l bound [R])."""
    bound, sb = e4m3_weight_bounds(w, v, o)
    vmax = float(np.abs(v).max()) if v.size else 0.0
    acc = 2.0 ** -24 * (n_keys / 64 + 72) * 2 * vmax
    tol = bound + acc + 2.0 ** -8 * (np.abs(o) + bound + acc) + 1e-7
    return tol, sb + 1e-5
