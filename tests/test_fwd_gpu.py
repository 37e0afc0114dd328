"""fa_fwd on the GPU against the float64 oracle (parity tests, through the C ABI)."""

import math

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


def run_fwd(x: gen.FwdInputs, dev, stats=True):
    q = gen.to_torch(x.q, x.dtype, dev)
    k = gen.to_torch(x.k, x.dtype, dev)
    v = gen.to_torch(x.v, x.dtype, dev)
    res = fa.fa_fwd(q, k, v, scale=x.scale, causal=x.causal, return_stats=stats)
    import torch

    torch.cuda.synchronize()
    return res


SMALL = [
    # dtype, B, Hq, Hkv, N, d, causal
    ("bf16", 1, 2, 2, 1, 64, True),
    ("bf16", 1, 2, 2, 7, 128, False),
    ("bf16", 2, 4, 2, 129, 64, True),
    ("bf16", 1, 4, 1, 300, 128, True),
    ("bf16", 1, 1, 1, 128, 128, True),
    ("bf16", 1, 2, 2, 1000, 64, False),
    ("bf16", 2, 3, 3, 1000, 128, True),
    ("bf16", 1, 8, 2, 513, 128, False),
    ("bf16", 1, 2, 1, 2048, 128, True),
    # more work items than CUs: several items per persistent workgroup, ragged tiles
    ("bf16", 4, 32, 8, 1000, 128, True),
    ("bf16", 2, 64, 64, 777, 64, False),
    # wide query groups: 8 and 16 query heads per KV head
    ("bf16", 1, 16, 2, 600, 128, True),
    ("bf16", 2, 16, 1, 300, 64, False),
    ("f32", 1, 1, 1, 256, 64, False),
    ("f32", 2, 4, 2, 100, 128, True),
    ("f32", 1, 2, 1, 1, 64, True),
    ("f32", 1, 2, 2, 333, 64, True),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "-".join(map(str, c)))
def test_fwd_small_shapes(case, dev):
    dtype, B, Hq, Hkv, N, d, causal = case
    seed = 100 + SMALL.index(case)
    log_case(f"fa_fwd small {case} seed={seed}")
    x = gen.fwd_inputs(B, Hq, Hkv, N, d, seed=seed, dtype=dtype, causal=causal)
    o, m, l = run_fwd(x, dev)
    o_ref, m_ref, l_ref = oracle.attention(x.q, x.k, x.v, x.scale, causal)
    assert_close(to_np(o), o_ref, dtype, "O")
    np.testing.assert_allclose(to_np(m), m_ref, atol=1e-5 if dtype == "f32" else 1e-3, rtol=0)
    np.testing.assert_allclose(to_np(l), l_ref, rtol=1e-5 if dtype == "f32" else L_RTOL_BF16)
    # without statistics (bf16: the softmax without per-tile row maxima)
    assert_close(to_np(run_fwd(x, dev, stats=False)), o_ref, dtype, "O without statistics")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fwd_worked_example(dtype, dev):
    """The worked example of "FlashAttention, explained.": row [2, 1, 3, 0] against four keys.

    With scale 1, every query row [2, 1, 3, 0, 0, ...] and K = V = the zero-padded 4x4
    identity, every output row is the softmax weight vector in columns 0-3.
    """
    import torch

    log_case(f"fa_fwd worked example {dtype}")
    d, N = 64, 4
    q = np.zeros((1, 1, N, d), np.float32)
    q[0, 0, :, :4] = [2, 1, 3, 0]
    kv = np.zeros((1, 1, N, d), np.float32)
    kv[0, 0, :, :4] = np.eye(4)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    qt = torch.from_numpy(q).to(dev, tdt)
    kt = torch.from_numpy(kv).to(dev, tdt)
    o, m, l = fa.fa_fwd(qt, kt, kt.clone(), scale=1.0, causal=False, return_stats=True)
    w = np.exp(np.array([2, 1, 3, 0.0]) - 3)
    w /= w.sum()
    got = to_np(o)[0, 0]
    for row in got:
        np.testing.assert_allclose(row[:4], [0.2369, 0.0871, 0.6439, 0.0321], atol=5e-5 if dtype == "f32" else 5e-3)
        assert_close(row[:4], w, dtype, "weights")
        assert np.all(row[4:] == 0)
    np.testing.assert_allclose(to_np(m)[0, 0], 3.0, atol=1e-6)
    # bf16: l sums the bf16-rounded weights (within 2^-9 of each weight, relative)
    if dtype == "f32":
        np.testing.assert_allclose(to_np(l)[0, 0], 1.5530, atol=5e-5)
    else:
        np.testing.assert_allclose(to_np(l)[0, 0], 1.5530, rtol=L_RTOL_BF16)


def test_config1_full(dev):
    cfg = gen.CONFIGS[1]
    log_case(f"fa_fwd config: {cfg.name}")
    x = gen.config_fwd_inputs(cfg)
    o, m, l = run_fwd(x, dev)
    o_ref, m_ref, l_ref = oracle.attention(x.q, x.k, x.v, x.scale, cfg.causal)
    stats = assert_close(to_np(o), o_ref, "f32", "config 1 O")
    assert stats["max_abs"] <= 1e-5


def test_config2_full(dev):
    cfg = gen.CONFIGS[2]
    log_case(f"fa_fwd config: {cfg.name}")
    x = gen.config_fwd_inputs(cfg)
    o, m, l = run_fwd(x, dev)
    o_ref, m_ref, l_ref = oracle.attention(x.q, x.k, x.v, x.scale, cfg.causal)
    assert_close(to_np(o), o_ref, "bf16", "config 2 O")
    np.testing.assert_allclose(to_np(m), m_ref, atol=1e-3)
    np.testing.assert_allclose(to_np(l), l_ref, rtol=L_RTOL_BF16)


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("cfg_id", [3, 4])
def test_config_full_size_every_row(cfg_id, dev):
    """The full-size workload: every row of every head of O, m and l (the kernel instance with
    row statistics) and of O from the launch the bench times (no statistics: the softmax
    without per-tile row maxima) against the oracle, run head by head in worker processes;
    a second run of the latter must be bitwise identical."""
    import torch

    from oracle import pool

    cfg = gen.CONFIGS[cfg_id]
    log_case(f"fa_fwd config: {cfg.name} (every row)")
    x = gen.config_fwd_inputs(cfg)
    q = gen.to_torch(x.q, "bf16", dev)
    k = gen.to_torch(x.k, "bf16", dev)
    v = gen.to_torch(x.v, "bf16", dev)
    o, m, l = fa.fa_fwd(q, k, v, scale=x.scale, causal=True, return_stats=True)
    o2 = fa.fa_fwd(q, k, v, scale=x.scale, causal=True)
    o3 = fa.fa_fwd(q, k, v, scale=x.scale, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o2, o3), "two runs differ: the kernel is not deterministic"
    o_np, m_np, l_np = o.float().cpu().numpy(), m.cpu().numpy(), l.cpu().numpy()
    o2_np = o2.float().cpu().numpy()
    del q, k, v, o, o2, o3, m, l
    torch.cuda.empty_cache()
    G = cfg.Hq // cfg.Hkv
    heads = [(b, h) for b in range(cfg.B) for h in range(cfg.Hq)]
    refs = pool.attention_heads(((x.q[b, h], x.k[b, h // G], x.v[b, h // G]) for b, h in heads),
                                x.scale, True)
    worst = 0.0
    for n, ((b, h), (o_ref, m_ref, l_ref)) in enumerate(zip(heads, refs)):
        st = assert_close(o_np[b, h], o_ref, "bf16", f"config {cfg_id} O[b={b},h={h}]")
        st2 = assert_close(o2_np[b, h], o_ref, "bf16",
                           f"config {cfg_id} O[b={b},h={h}] without statistics")
        worst = max(worst, st["max_abs"], st2["max_abs"])
        np.testing.assert_allclose(m_np[b, h], m_ref, atol=2e-3, rtol=0)
        np.testing.assert_allclose(l_np[b, h], l_ref, rtol=L_RTOL_BF16)
        if n % 8 == 7:
            log_case(f"config {cfg_id}: {n + 1} of {len(heads)} heads match; max |err| {worst:.3e}")


def test_fwd_deterministic_and_gqa_equals_repeated_heads(dev):
    import torch

    log_case("fa_fwd GQA vs repeated heads")
    x = gen.fwd_inputs(1, 8, 2, 700, 128, seed=5, dtype="bf16", causal=True)
    o1 = run_fwd(x, dev, stats=False)
    xr = gen.FwdInputs(x.q, np.repeat(x.k, 4, axis=1), np.repeat(x.v, 4, axis=1), x.scale, True, "bf16")
    o2 = run_fwd(xr, dev, stats=False)
    assert torch.equal(o1, o2)
    o3 = run_fwd(x, dev, stats=False)
    assert torch.equal(o1, o3)


def test_fwd_empty_calls_are_noops(dev):
    import torch

    log_case("fa_fwd empty")
    q = torch.zeros(0, 2, 16, 64, dtype=torch.bfloat16, device=dev)
    assert fa.fa_fwd(q, q, q).shape == q.shape
    q = torch.zeros(1, 2, 0, 128, dtype=torch.bfloat16, device=dev)
    assert fa.fa_fwd(q, q, q, causal=True).shape == q.shape


def test_fwd_uniform_scores_give_prefix_mean(dev):
    """Q = 0 makes every admissible score equal, so O is the mean of V over the prefix."""
    import torch

    log_case("fa_fwd uniform scores")
    x = gen.fwd_inputs(1, 2, 2, 333, 64, seed=9, dtype="bf16", causal=True)
    x.q[:] = 0
    o = run_fwd(x, dev, stats=False)
    prefix = np.cumsum(x.v.astype(np.float64), axis=2) / np.arange(1, 334)[None, None, :, None]
    assert_close(to_np(o), prefix, "bf16", "prefix mean")
    torch.cuda.synchronize()


def test_fwd_causal_row0_is_v0(dev):
    log_case("fa_fwd causal row 0")
    x = gen.fwd_inputs(2, 2, 1, 200, 128, seed=10, dtype="f32", causal=True)
    o = run_fwd(x, dev, stats=False)
    got = to_np(o)[:, :, 0]
    ref = np.repeat(x.v[:, :, 0], 2, axis=1)
    np.testing.assert_allclose(got, ref, atol=1e-6)


def test_fwd_peaky_rows_large_scores(dev):
    """Scores of several hundred: without the max subtraction exp() would overflow."""
    log_case("fa_fwd peaky")
    x = gen.fwd_inputs(1, 2, 2, 256, 128, seed=11, dtype="bf16", causal=False, k_mult=8.0,
                       scale=1.0)
    o, m, l = run_fwd(x, dev)
    o_ref, m_ref, l_ref = oracle.attention(x.q, x.k, x.v, x.scale, False)
    assert_close(to_np(o), o_ref, "bf16", "peaky O")
    assert math.isfinite(float(to_np(m).max()))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [128, 64])
def test_fwd_without_stats_recovers_from_a_stale_reference(causal, d, dev):
    """Without statistics the exponent reference is the first half tile's row maximum. Keys
    past the first 32 whose scores lie hundreds of log2 units above it overflow the row sums;
    the work item is then computed again with per-tile maxima. The result must still match the
    oracle, with and without statistics, and across a first tile that some rows see only
    partly (causal)."""
    log_case(f"fa_fwd stale reference d={d} causal={causal}")
    x = gen.fwd_inputs(1, 4, 2, 700, d, seed=12, dtype="bf16", causal=causal, scale=1.0)
    x.k[:, :, :32] *= np.float32(0.01)   # the first half tile: scores near 0
    x.k[:, :, 32:] *= np.float32(4.0)    # the rest: scores of a few hundred
    x.k[:] = gen.round_to_bf16(x.k)
    o_ref, _, _ = oracle.attention(x.q, x.k, x.v, x.scale, causal)
    o = run_fwd(x, dev, stats=False)
    assert_close(to_np(o), o_ref, "bf16", "O without statistics")
    o2, m2, l2 = run_fwd(x, dev, stats=True)
    assert_close(to_np(o2), o_ref, "bf16", "O with statistics")


def test_fwd_at_the_offset_bound(dev):
    """One head at the largest size the forward accepts (N d 2 = 2^30 bytes per head: N = 2^22
    tokens at d = 128, causal): its last tiles sit just below 2^30 bytes into the K and V rows,
    where the 32-bit tile offsets and the pad offset must still stay apart. Sampled rows, among
    them the last, which sees every key, against the oracle; with and without statistics."""
    import torch

    N, d = 1 << 22, 128
    log_case(f"fa_fwd at the offset bound: N={N} d={d}")
    x = gen.fwd_inputs(1, 1, 1, N, d, 31, causal=True)
    q, k, v = (gen.to_torch(t, "bf16", dev) for t in (x.q, x.k, x.v))
    o, m, l = fa.fa_fwd(q, k, v, scale=x.scale, causal=True, return_stats=True)
    o2 = fa.fa_fwd(q, k, v, scale=x.scale, causal=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(32)
    rows = np.unique(np.concatenate([[0, 255, 256, N // 2, N - 257, N - 256, N - 1],
                                     rng.integers(N - (1 << 16), N, size=5)]))
    rows_t = torch.from_numpy(rows).to(dev)
    o_s, o2_s = to_np(o[0, 0][rows_t]), to_np(o2[0, 0][rows_t])
    m_s, l_s = to_np(m[0, 0][rows_t]), to_np(l[0, 0][rows_t])
    del o, o2, m, l, q, k, v
    o_ref, m_ref, l_ref = oracle.attention_head(x.q[0, 0], x.k[0, 0], x.v[0, 0], x.scale, True, rows=rows,
                                                row_block=4)
    assert_close(o_s, o_ref, "bf16", "rows at the offset bound")
    assert_close(o2_s, o_ref, "bf16", "rows at the offset bound, without statistics")
    np.testing.assert_allclose(m_s, m_ref, atol=1e-3, rtol=0)
    np.testing.assert_allclose(l_s, l_ref, rtol=L_RTOL_BF16)
