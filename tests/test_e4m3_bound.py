"""The tolerance of the e4m3-weight forward, checked on the CPU against a float64 model of that
rounding: scores taken in 64-key tiles, an exponent reference that moves only when a tile's
maximum passes it by more than 2^8 and then to 2^4 below that maximum, every weight rounded to
e4m3 against the reference in effect, and O = sum w~ v / sum w~. Whatever the score spread,
the error stays inside the bound the GPU tests apply, and no weight leaves e4m3's range."""

import numpy as np
import pytest

from exact_tiled_attention_24_amd import inputs as gen
from helpers import e4m3_weight_bounds


def rounded_weights_model(s, v, tile=64, lazy=8.0, head=4.0):
    """Float64 model of the e4m3-weight softmax of one row of base-2 scores s [Nk]."""
    ref = -np.inf
    acc = np.zeros(v.shape[1])
    l = 0.0
    wmax_seen = 0.0
    for t0 in range(0, s.shape[0], tile):
        st = s[t0:t0 + tile]
        mx = st.max()
        if mx > ref + lazy:
            new = mx - head
            f = np.exp2(ref - new) if np.isfinite(ref) else 0.0
            acc *= f
            l *= f
            ref = new
        w = np.exp2(st - ref)
        wmax_seen = max(wmax_seen, float(w.max()))
        wr = gen.round_to_e4m3(w).astype(np.float64)
        acc += wr @ v[t0:t0 + tile]
        l += wr.sum()
    return acc / l, l * np.exp2(ref - s.max()), wmax_seen


@pytest.mark.parametrize("spread", [0.3, 1.0, 3.0, 10.0, 40.0])
@pytest.mark.parametrize("n_keys", [64, 700, 4096])
def test_e4m3_weight_error_within_bound(spread, n_keys):
    rng = np.random.default_rng(int(spread * 10) + n_keys)
    d = 16
    v = gen.round_to_e4m3(rng.standard_normal((n_keys, d)).astype(np.float32)).astype(np.float64)
    for trial in range(6):
        s = rng.standard_normal(n_keys) * spread
        if trial == 1:
            s += np.linspace(0.0, 3 * spread, n_keys)   # maxima late in the row: the reference moves
        if trial == 2:
            s[: n_keys // 2] -= 5 * spread              # the first tiles far below the rest
        w = np.exp2(s - s.max())
        l_exact = w.sum()
        w /= l_exact
        o = w @ v
        o_r, l_r, wmax_seen = rounded_weights_model(s, v)
        assert wmax_seen <= 256.0                       # e4m3's largest finite value is 448
        bound, sb = e4m3_weight_bounds(w[None], v, o[None])
        err = np.abs(o_r - o)
        assert np.all(err <= bound[0] * (1 + 1e-9) + 1e-12), (spread, n_keys, trial, (err - bound[0]).max())
        assert abs(l_r / l_exact - 1) <= sb[0] * (1 + 1e-9)


def test_e4m3_bound_is_not_vacuous():
    """A row whose weight sits on one key: the bound is small next to the values, so an output
    that took the wrong value rows would fail it."""
    rng = np.random.default_rng(5)
    v = gen.round_to_e4m3(rng.standard_normal((512, 8)).astype(np.float32)).astype(np.float64)
    s = rng.standard_normal(512) * 30.0
    w = np.exp2(s - s.max())
    w /= w.sum()
    o = w @ v
    bound, _ = e4m3_weight_bounds(w[None], v, o[None])
    assert bound.max() < 0.1 * np.abs(v).mean()
