"""fa_fwd_fp8 on the GPU against the float64 oracle (parity tests, through the C ABI).

Q and K are rounded to OCP e4m3 on the host (the oracle is fed those exact values, V the
same bf16 values); the scores are exact products of e4m3 values accumulated in float32, so
the result carries the bf16 path's errors (P and O rounded to bf16) and is held to the bf16
tolerance.
"""

import numpy as np
import pytest

import oracle
import exact_tiled_attention_24_amd as fa
from exact_tiled_attention_24_amd import inputs as gen
from helpers import assert_close, cuda_device, log_case, to_np, L_RTOL_BF16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return cuda_device()


def run(x, dev, stats=True):
    import torch

    q = gen.to_torch(x.q, "e4m3", dev)
    k = gen.to_torch(x.k, "e4m3", dev)
    v = gen.to_torch(x.v, "bf16", dev)
    res = fa.fa_fwd_fp8(q, k, v, scale=x.scale, causal=x.causal, return_stats=stats)
    torch.cuda.synchronize()
    return res


CASES = [
    # B, Hq, Hkv, N, causal
    (1, 2, 2, 256, False),
    (2, 4, 4, 300, True),
    (1, 8, 2, 1000, True),
    (2, 4, 1, 777, False),
    (1, 16, 4, 2048, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}-Hq{c[1]}-Hkv{c[2]}-N{c[3]}-{'c' if c[4] else 'n'}")
def test_fp8_forward_matches_oracle(case, dev):
    B, Hq, Hkv, N, causal = case
    seed = 900 + CASES.index(case)
    log_case(f"fa_fwd_fp8 {case} seed={seed}")
    x = gen.fp8_fwd_inputs(B, Hq, Hkv, N, 128, seed, causal=causal)
    o, m, l = run(x, dev)
    o_ref, m_ref, l_ref = oracle.attention(x.q, x.k, x.v, x.scale, causal)
    assert_close(to_np(o), o_ref, "bf16", "fp8 forward O")
    np.testing.assert_allclose(to_np(m), m_ref, atol=1e-3, rtol=0)
    np.testing.assert_allclose(to_np(l), l_ref, rtol=L_RTOL_BF16)
    assert_close(to_np(run(x, dev, stats=False)), o_ref, "bf16", "fp8 forward O without statistics")


def test_fp8_forward_long_workload_sampled_rows(dev):
    """The long-prefill shape (B=2, H=32, N=8192, d=128, causal, K x2) with e4m3 Q and K, in
    the launch the bench times; sampled rows against the oracle."""
    log_case("fa_fwd_fp8 long workload")
    x = gen.fp8_fwd_inputs(2, 32, 32, 8192, 128, 3, causal=True, k_mult=2.0)
    o, m, l = run(x, dev)
    o, m, l = to_np(o), to_np(m), to_np(l)
    o2 = to_np(run(x, dev, stats=False))  # the launch the bench times
    rng = np.random.default_rng(950)
    for _ in range(8):
        b, h = int(rng.integers(2)), int(rng.integers(32))
        rows = np.unique(np.concatenate([[0, 8191], rng.integers(0, 8192, size=30)]))
        o_ref, m_ref, l_ref = oracle.attention_head(x.q[b, h], x.k[b, h], x.v[b, h], x.scale, True,
                                                    rows=rows)
        assert_close(o[b, h][rows], o_ref, "bf16", f"fp8 rows of (b={b}, h={h})")
        assert_close(o2[b, h][rows], o_ref, "bf16", f"fp8 rows of (b={b}, h={h}) without statistics")
        np.testing.assert_allclose(m[b, h][rows], m_ref, atol=2e-3)
        np.testing.assert_allclose(l[b, h][rows], l_ref, rtol=L_RTOL_BF16)
