"""fa_fwd_block_sparse on the GPU against the float64 oracle (parity tests, through the C ABI)."""

import numpy as np
import pytest

import oracle
import exact_tiled_attention_24_amd as fa
from exact_tiled_attention_24_amd import inputs as gen
from helpers import assert_close, cuda_device, log_case, to_np, L_RTOL_BF16

pytestmark = pytest.mark.gpu

BQ, BK = gen.SPARSE_BQ, gen.SPARSE_BK


@pytest.fixture(scope="module")
def dev():
    return cuda_device()


def run(x, rows, dev, causal, stats=True):
    """Returns ((O, m, l) or O alone when not `stats`), offsets, indices. Without statistics the
    library runs its softmax without per-tile row maxima (another kernel instance)."""
    import torch

    offs, idx = gen.block_csr(rows)
    q, k, v = (gen.to_torch(t, "bf16", dev) for t in (x.q, x.k, x.v))
    ot = torch.from_numpy(offs).to(dev)
    it = torch.from_numpy(idx if idx.size else np.zeros(1, np.int32)).to(dev)
    if not idx.size:
        it = it[:0]
    res = fa.fa_fwd_block_sparse(q, k, v, ot, it, scale=x.scale, causal=causal, return_stats=stats)
    torch.cuda.synchronize()
    return res, offs, idx


def check(res, x, offs, idx, causal, what):
    o, m, l = (to_np(t) for t in res)
    o_ref, m_ref, l_ref = oracle.attention_block_sparse(x.q, x.k, x.v, x.scale, causal, offs, idx, BQ, BK)
    assert_close(o, o_ref, "bf16", what)
    empty = l_ref == 0
    assert np.all(m[empty] == -np.inf) and np.all(l[empty] == 0)
    np.testing.assert_allclose(m[~empty], m_ref[~empty], atol=1e-3)
    np.testing.assert_allclose(l[~empty], l_ref[~empty], rtol=L_RTOL_BF16)


CASES = [
    # B, Hq, Hkv, N, d, density, causal
    (1, 4, 2, 1000, 128, 0.5, False),
    (2, 4, 4, 777, 64, 0.3, True),
    (1, 8, 2, 2048, 128, 0.6, True),
    (2, 8, 8, 1536, 64, 0.8, False),
    (1, 16, 4, 3000, 128, 0.15, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}-Hq{c[1]}-Hkv{c[2]}-N{c[3]}-d{c[4]}-p{c[5]}-{'c' if c[6] else 'n'}")
def test_block_sparse_random_masks(case, dev):
    B, Hq, Hkv, N, d, density, causal = case
    seed = 700 + CASES.index(case)
    log_case(f"fa_fwd_block_sparse {case} seed={seed}")
    x = gen.fwd_inputs(B, Hq, Hkv, N, d, seed, causal=causal)
    rows = gen.random_blocks(B, Hq, N, density, seed + 50)
    nkb = -(-N // BK)
    rows[0] = []                                  # a query block with no key block
    rows[1] = rows[1] + [nkb + 3, -2]             # indices that name no key
    if len(rows) > 2:
        rows[2] = [nkb - 1, 0, 3 % nkb]           # out of order, with the ragged last block
    res, offs, idx = run(x, rows, dev, causal)
    check(res, x, offs, idx, causal, "block-sparse O")
    o2, _, _ = run(x, rows, dev, causal, stats=False)
    o_ref, _, _ = oracle.attention_block_sparse(x.q, x.k, x.v, x.scale, causal, offs, idx, BQ, BK)
    assert_close(to_np(o2), o_ref, "bf16", "block-sparse O without statistics")


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("d", [128, 64])
def test_block_sparse_full_lists_equal_dense_bitwise(causal, d, dev):
    """Listing every key tile the dense kernel visits, in its order, reproduces fa_fwd bit
    for bit."""
    import torch

    B, Hq, Hkv, N = 2, 8, 2, 1100
    log_case(f"fa_fwd_block_sparse full lists vs fa_fwd causal={causal} d={d}")
    x = gen.fwd_inputs(B, Hq, Hkv, N, d, 710 + d, causal=causal)
    nqb, nkb = -(-N // BQ), -(-N // BK)
    rows = [list(range(min(nkb, 4 * (qb + 1)) if causal else nkb)) for _ in range(B * Hq) for qb in range(nqb)]
    (o, m, l), _, _ = run(x, rows, dev, causal)
    q, k, v = (gen.to_torch(t, "bf16", dev) for t in (x.q, x.k, x.v))
    o_d, m_d, l_d = fa.fa_fwd(q, k, v, scale=x.scale, causal=causal, return_stats=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o_d) and torch.equal(m, m_d) and torch.equal(l, l_d)
    o2, _, _ = run(x, rows, dev, causal, stats=False)
    o2_d = fa.fa_fwd(q, k, v, scale=x.scale, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o2, o2_d)


def test_block_sparse_local_global_pattern(dev):
    B, Hq, Hkv, N, d = 1, 8, 2, 2500, 128
    log_case("fa_fwd_block_sparse local + global pattern")
    x = gen.fwd_inputs(B, Hq, Hkv, N, d, 720, causal=True)
    rows = gen.local_global_blocks(B, Hq, N, 512, 2, causal=True)
    res, offs, idx = run(x, rows, dev, True)
    check(res, x, offs, idx, True, "local+global O")


def test_block_sparse_only_blocks_above_diagonal(dev):
    """Query blocks that list only key blocks above their diagonal see no key at all."""
    B, Hq, Hkv, N, d = 1, 4, 4, 1024, 128
    log_case("fa_fwd_block_sparse blocks above the diagonal only")
    x = gen.fwd_inputs(B, Hq, Hkv, N, d, 721, causal=True)
    nqb, nkb = N // BQ, N // BK
    rows = [list(range(4 * (qb + 1), nkb)) for _ in range(B * Hq) for qb in range(nqb)]
    (o, m, l), offs, idx = run(x, rows, dev, True)
    o, m, l = to_np(o), to_np(m), to_np(l)
    assert np.all(o == 0) and np.all(m == -np.inf) and np.all(l == 0)


def test_block_sparse_workload_sampled_rows(dev):
    """The block-sparse workload at full size (2 x 32 query heads over 8 KV heads, N = 16384,
    d = 128, local window of 2048 keys + 256 global keys, causal) in the launch the bench
    times; sampled rows are compared with the oracle applied to the keys they admit."""
    import torch

    cfg = gen.BLOCK_SPARSE
    log_case(f"fa_fwd_block_sparse full workload: {cfg.name}")
    x = gen.fwd_inputs(cfg.B, cfg.Hq, cfg.Hkv, cfg.N, cfg.d, cfg.seed, causal=cfg.causal)
    rows = gen.local_global_blocks(cfg.B, cfg.Hq, cfg.N, cfg.window, cfg.n_global, cfg.causal)
    (o, m, l), offs, idx = run(x, rows, dev, cfg.causal)
    o, m, l = to_np(o), to_np(m), to_np(l)
    assert np.isfinite(o).all()
    o2 = to_np(run(x, rows, dev, cfg.causal, stats=False)[0])  # the launch the bench times
    rng = np.random.default_rng(730)
    nqb = cfg.N // BQ
    G = cfg.Hq // cfg.Hkv
    for _ in range(40):
        b, h = int(rng.integers(cfg.B)), int(rng.integers(cfg.Hq))
        i = int(rng.choice([0, 255, 256, cfg.N - 1, int(rng.integers(cfg.N))]))
        blocks = rows[(b * cfg.Hq + h) * nqb + i // BQ]
        keys = np.array([j for kb in blocks for j in range(kb * BK, (kb + 1) * BK) if j <= i])
        o_ref, m_ref, l_ref = oracle.attention_head(x.q[b, h, i:i + 1], x.k[b, h // G][keys],
                                                    x.v[b, h // G][keys], x.scale, False)
        assert_close(o[b, h, i], o_ref[0], "bf16", f"row (b={b}, h={h}, i={i})")
        assert_close(o2[b, h, i], o_ref[0], "bf16", f"row (b={b}, h={h}, i={i}) without statistics")
        assert abs(m[b, h, i] - m_ref[0]) <= 2e-3
        assert abs(l[b, h, i] - l_ref[0]) <= L_RTOL_BF16 * l_ref[0]
