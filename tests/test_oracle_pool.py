"""The oracle's head-parallel runner returns exactly what the oracle returns head by head."""

import numpy as np

import oracle
from oracle import pool
from exact_tiled_attention_24_amd import inputs as gen


def test_pool_forward_equals_direct_calls():
    x = gen.fwd_inputs(2, 4, 2, 70, 16, seed=5, causal=True)
    heads = [(b, h) for b in range(2) for h in range(4)]
    got = list(pool.attention_heads(((x.q[b, h], x.k[b, h // 2], x.v[b, h // 2]) for b, h in heads),
                                    x.scale, True, workers=2))
    ref_o, ref_m, ref_l = oracle.attention(x.q, x.k, x.v, x.scale, True)
    for (b, h), (o, m, l) in zip(heads, got):
        assert np.allclose(o, ref_o[b, h], rtol=1e-12, atol=1e-14)
        assert np.allclose(m, ref_m[b, h], rtol=1e-12, atol=1e-14)
        assert np.allclose(l, ref_l[b, h], rtol=1e-12, atol=1e-14)


def test_pool_backward_equals_direct_calls():
    x = gen.fwd_inputs(1, 3, 3, 40, 8, seed=6, causal=False)
    dout = gen.round_to_bf16(np.random.default_rng(7).standard_normal(x.q.shape, dtype=np.float32))
    got = list(pool.attention_backward_heads(
        ((x.q[0, h], x.k[0, h], x.v[0, h], dout[0, h]) for h in range(3)), x.scale, False, workers=2))
    dq, dk, dv = oracle.attention_backward(x.q, x.k, x.v, dout, x.scale, False)
    for h, (a, b, c) in enumerate(got):
        assert np.allclose(a, dq[0, h], rtol=1e-12, atol=1e-14)
        assert np.allclose(b, dk[0, h], rtol=1e-12, atol=1e-14)
        assert np.allclose(c, dv[0, h], rtol=1e-12, atol=1e-14)


def test_worker_count_is_bounded():
    assert 1 <= pool.worker_count() <= pool.MAX_WORKERS
    assert pool.worker_count(limit=1) == 1
