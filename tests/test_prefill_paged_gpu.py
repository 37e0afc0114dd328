"""fa_fwd_paged on the GPU against the float64 oracle (parity tests, through the C ABI).

The oracle sees each sequence's logical K/V; the kernel reads the scattered pages through the
block table, so paging is checked, not re-implemented. Unused cache slots and table entries
hold NaN and -1, so any read of them shows up in the result.
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


def upload(x, dev):
    import torch

    return dict(
        q=gen.to_torch(x.q, "bf16", dev),
        k_cache=gen.to_torch(x.k_cache, "bf16", dev),
        v_cache=gen.to_torch(x.v_cache, "bf16", dev),
        block_table=torch.from_numpy(x.block_table).to(dev),
        seq_lens=torch.from_numpy(x.lens.astype(np.int32)).to(dev),
    )


def run(t, scale, causal, stats=True):
    """(O, m, l), or O alone when not `stats` (the softmax without per-tile row maxima)."""
    import torch

    res = fa.fa_fwd_paged(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["seq_lens"],
                          scale=scale, causal=causal, return_stats=stats)
    torch.cuda.synchronize()
    return res


def check_stats(m, l, m_ref, l_ref):
    m, l = to_np(m), to_np(l)
    empty = l_ref == 0
    assert np.all(m[empty] == -np.inf) and np.all(l[empty] == 0)
    np.testing.assert_allclose(m[~empty], m_ref[~empty], atol=1e-3, rtol=0)
    np.testing.assert_allclose(l[~empty], l_ref[~empty], rtol=L_RTOL_BF16)


CASES = [
    # B, Hq, Hkv, Nq, lens, d, causal
    (2, 4, 4, 64, [64, 200], 128, True),          # Nq = L (plain causal) and a longer history
    (3, 8, 2, 300, [300, 517, 1000], 128, True),  # ragged query blocks, GQA 4:1
    (3, 8, 2, 300, [300, 517, 1000], 64, True),
    (2, 4, 1, 257, [1000, 2049], 128, False),     # unmasked, ragged key tail
    (2, 4, 2, 300, [100, 0], 128, True),          # L < Nq (first rows see nothing), L = 0
    (1, 8, 8, 1, [777], 128, True),               # one query: the decode case
    (4, 16, 4, 512, [513, 1024, 3000, 4096], 64, False),
    (2, 32, 8, 700, [5000, 8191], 128, True),     # 8 KV groups over the 8 XCDs
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}-Hq{c[1]}-Hkv{c[2]}-Nq{c[3]}-d{c[5]}-{'c' if c[6] else 'n'}")
def test_prefill_paged_small(case, dev):
    B, Hq, Hkv, Nq, lens, d, causal = case
    seed = 600 + CASES.index(case)
    log_case(f"fa_fwd_paged {case} seed={seed}")
    x = gen.prefill_paged_inputs(B, Hq, Hkv, Nq, d, 16, seed=seed, lens=lens,
                                 max_pages_per_seq=-(-max(lens) // 16) + 2, causal=causal)
    t = upload(x, dev)
    o, m, l = run(t, x.scale, causal)
    o_ref, m_ref, l_ref = oracle.prefill_paged(x.q, x.k_seqs, x.v_seqs, x.scale, causal)
    assert_close(to_np(o), o_ref, "bf16", "paged prefill O")
    check_stats(m, l, m_ref, l_ref)
    assert_close(to_np(run(t, x.scale, causal, stats=False)), o_ref, "bf16",
                 "paged prefill O without statistics")


def test_prefill_paged_matches_dense_forward_bitwise(dev):
    """With Nq = L the paged kernel runs the dense kernel's tiles in the same order on the
    same values: the results must be identical bit for bit."""
    import torch

    B, Hq, Hkv, N, d = 2, 8, 2, 700, 128
    log_case("fa_fwd_paged vs fa_fwd bitwise")
    x = gen.prefill_paged_inputs(B, Hq, Hkv, N, d, 16, seed=620, lens=[N, N])
    t = upload(x, dev)
    o_p, m_p, l_p = run(t, x.scale, True)
    k = gen.to_torch(np.stack(x.k_seqs), "bf16", dev)
    v = gen.to_torch(np.stack(x.v_seqs), "bf16", dev)
    o_d, m_d, l_d = fa.fa_fwd(t["q"], k, v, scale=x.scale, causal=True, return_stats=True)
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_d)
    assert torch.equal(m_p, m_d) and torch.equal(l_p, l_d)
    o2_p = run(t, x.scale, True, stats=False)
    o2_d = fa.fa_fwd(t["q"], k, v, scale=x.scale, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o2_p, o2_d)


def _shared_prefix_inputs(B, Hkv, d, P, suffix_lens, seed):
    """K/V of B sequences that share their first P tokens (P a multiple of 16): the prefix
    pages appear once in the pool and in every sequence's table row."""
    rng = np.random.default_rng(seed)
    pk = gen.round_to_bf16(rng.standard_normal((Hkv, P, d), dtype=np.float32))
    pv = gen.round_to_bf16(rng.standard_normal((Hkv, P, d), dtype=np.float32))
    sk = [gen.round_to_bf16(rng.standard_normal((Hkv, S, d), dtype=np.float32)) for S in suffix_lens]
    sv = [gen.round_to_bf16(rng.standard_normal((Hkv, S, d), dtype=np.float32)) for S in suffix_lens]
    n_pre = P // 16
    n_suf = [-(-S // 16) for S in suffix_lens]
    total = n_pre + sum(n_suf)
    perm = rng.permutation(total).astype(np.int32)
    kc = np.full((total, Hkv, 16, d), np.nan, np.float32)
    vc = np.full((total, Hkv, 16, d), np.nan, np.float32)

    def place(phys, seq_k, seq_v):
        n = len(phys)
        for cache, seq in ((kc, seq_k), (vc, seq_v)):
            padded = np.full((Hkv, n * 16, d), np.nan, np.float32)
            padded[:, :seq.shape[1]] = seq
            cache[phys] = padded.reshape(Hkv, n, 16, d).transpose(1, 0, 2, 3)

    pre_phys = perm[:n_pre]
    place(pre_phys, pk, pv)
    width = n_pre + max(n_suf)
    full_table = np.full((B, width), -1, np.int32)
    suf_table = np.full((B, max(n_suf)), -1, np.int32)
    off = n_pre
    for b in range(B):
        phys = perm[off:off + n_suf[b]]
        off += n_suf[b]
        place(phys, sk[b], sv[b])
        full_table[b, :n_pre] = pre_phys
        full_table[b, n_pre:n_pre + n_suf[b]] = phys
        suf_table[b, :n_suf[b]] = phys
    pre_table = np.tile(pre_phys, (B, 1)).astype(np.int32)
    k_seqs = [np.concatenate([pk, sk[b]], axis=1) for b in range(B)]
    v_seqs = [np.concatenate([pv, sv[b]], axis=1) for b in range(B)]
    return kc, vc, full_table, pre_table, suf_table, k_seqs, v_seqs


@pytest.mark.parametrize("d", [128, 64])
def test_shared_prefix_cascade_with_merge(d, dev):
    """A prefix shared by all sequences, attended without mask (every query lies after it),
    plus each sequence's own tokens with the causal mask, merged with fa_merge: equals
    attention over the whole history."""
    import torch

    B, Hq, Hkv, Nq, P = 3, 8, 2, 200, 512
    suffix = [200, 333, 1000]
    log_case(f"fa_fwd_paged shared prefix + fa_merge d={d}")
    kc, vc, full_t, pre_t, suf_t, k_seqs, v_seqs = _shared_prefix_inputs(B, Hkv, d, P, suffix, 630 + d)
    rng = np.random.default_rng(640 + d)
    q = gen.round_to_bf16(rng.standard_normal((B, Hq, Nq, d), dtype=np.float32))
    scale = 1.0 / np.sqrt(d)
    qt = gen.to_torch(q, "bf16", dev)
    kct, vct = gen.to_torch(kc, "bf16", dev), gen.to_torch(vc, "bf16", dev)
    tab = lambda a: torch.from_numpy(a).to(dev)
    lens_pre = tab(np.full(B, P, np.int32))
    lens_suf = tab(np.asarray(suffix, np.int32))
    lens_full = tab(np.asarray([P + s for s in suffix], np.int32))
    o1, m1, l1 = fa.fa_fwd_paged(qt, kct, vct, tab(pre_t), lens_pre, scale=scale, causal=False,
                                 return_stats=True)
    o2, m2, l2 = fa.fa_fwd_paged(qt, kct, vct, tab(suf_t), lens_suf, scale=scale, causal=True,
                                 return_stats=True)
    R = B * Hq * Nq
    o_parts = torch.stack([o1.float().reshape(R, d), o2.float().reshape(R, d)]).contiguous()
    m_parts = torch.stack([m1.reshape(R), m2.reshape(R)]).contiguous()
    l_parts = torch.stack([l1.reshape(R), l2.reshape(R)]).contiguous()
    o_c = fa.fa_merge(o_parts, m_parts, l_parts, out_dtype=torch.bfloat16)
    o_f = fa.fa_fwd_paged(qt, kct, vct, tab(full_t), lens_full, scale=scale, causal=True)
    torch.cuda.synchronize()
    o_ref, _, _ = oracle.prefill_paged(q, k_seqs, v_seqs, scale, True)
    assert_close(to_np(o_c).reshape(B, Hq, Nq, d), o_ref, "bf16", "cascade O")
    assert_close(to_np(o_f), o_ref, "bf16", "whole-history O")


def test_prefill_paged_workload_sampled_rows(dev):
    """The chunked-prefill workload at full size (4 sequences of 4K-16K cached tokens, 2048
    new ones, 32 query heads over 8 KV heads, d = 128), in the launch configuration the
    bench times; rows sampled across sequences, heads and query positions are compared with
    the oracle one by one (a single query at position p sees the p + 1 keys before it)."""
    cfg = gen.PREFILL_PAGED
    log_case(f"fa_fwd_paged full workload: {cfg.name}")
    x = gen.config_prefill_paged_inputs(cfg)
    t = upload(x, dev)
    o, m, l = run(t, x.scale, cfg.causal)
    o, m, l = to_np(o), to_np(m), to_np(l)
    assert np.isfinite(o).all()
    o2 = to_np(run(t, x.scale, cfg.causal, stats=False))  # the launch the bench times
    rng = np.random.default_rng(650)
    G = cfg.Hq // cfg.Hkv
    for _ in range(48):
        b = int(rng.integers(cfg.B))
        h = int(rng.integers(cfg.Hq))
        i = int(rng.choice([0, 1, cfg.Nq - 1, int(rng.integers(cfg.Nq))]))
        L = int(x.lens[b])
        pos = L - cfg.Nq + i
        ks = [x.k_seqs[b][h // G:h // G + 1, :pos + 1]]
        vs = [x.v_seqs[b][h // G:h // G + 1, :pos + 1]]
        o_ref, m_ref, l_ref = oracle.prefill_paged(x.q[b:b + 1, h:h + 1, i:i + 1], ks, vs, x.scale, True)
        assert_close(o[b, h, i], o_ref[0, 0, 0], "bf16", f"row (b={b}, h={h}, i={i})")
        assert_close(o2[b, h, i], o_ref[0, 0, 0], "bf16", f"row (b={b}, h={h}, i={i}) without statistics")
        assert abs(m[b, h, i] - m_ref[0, 0, 0]) <= 2e-3
        assert abs(l[b, h, i] - l_ref[0, 0, 0]) <= L_RTOL_BF16 * l_ref[0, 0, 0]


def test_prefill_paged_empty_calls_are_noops(dev):
    import torch

    q = torch.zeros((0, 4, 16, 128), dtype=torch.bfloat16, device=dev)
    kc = torch.zeros((1, 1, 16, 128), dtype=torch.bfloat16, device=dev)
    tab = torch.zeros((0, 1), dtype=torch.int32, device=dev)
    lens = torch.zeros((0,), dtype=torch.int32, device=dev)
    o = fa.fa_fwd_paged(q, kc, kc, tab, lens)
    assert o.shape == q.shape


@pytest.mark.parametrize("d", [128, 64])
def test_prefill_paged_per_sequence_query_counts(d, dev):
    """Different numbers of new tokens per sequence (q_lens), including none, more rows than
    one query block, and more new tokens than cached keys (its first rows see nothing): rows
    past a sequence's count keep what the output held."""
    import torch

    B, Hq, Hkv, Nq = 5, 8, 2, 600
    lens = [700, 300, 2000, 50, 90]
    q_lens = [600, 100, 257, 0, 120]
    log_case(f"fa_fwd_paged q_lens={q_lens} lens={lens} d={d}")
    x = gen.prefill_paged_inputs(B, Hq, Hkv, Nq, d, 16, seed=660 + d, lens=lens,
                                 max_pages_per_seq=-(-max(lens) // 16) + 1)
    t = upload(x, dev)
    ql = torch.tensor(q_lens, dtype=torch.int32, device=dev)
    sentinel = 7.0
    o = torch.full(t["q"].shape, sentinel, dtype=torch.bfloat16, device=dev)
    o, m, l = fa.fa_fwd_paged(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["seq_lens"],
                              scale=x.scale, causal=True, out=o, return_stats=True, q_lens=ql)
    torch.cuda.synchronize()
    o_ref, m_ref, l_ref = oracle.prefill_paged(x.q, x.k_seqs, x.v_seqs, x.scale, True, q_lens=q_lens)
    o, m, l = to_np(o), to_np(m), to_np(l)
    for b, n in enumerate(q_lens):
        if n:
            assert_close(o[b, :, :n], o_ref[b, :, :n], "bf16", f"sequence {b} O")
            check_stats(torch.from_numpy(m[b, :, :n]), torch.from_numpy(l[b, :, :n]),
                        m_ref[b, :, :n], l_ref[b, :, :n])
        assert np.all(o[b, :, n:] == sentinel), f"sequence {b}: rows past {n} were written"
