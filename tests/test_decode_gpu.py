"""fa_decode_splitk on the GPU against the float64 oracle (parity tests, through the C ABI)."""

import numpy as np
import pytest

import oracle
import exact_tiled_attention_24_amd as fa
from exact_tiled_attention_24_amd import inputs as gen
from helpers import assert_close, cuda_device, log_case, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return cuda_device()


def upload(x: gen.DecodeInputs, dev):
    import torch

    return dict(
        q=gen.to_torch(x.q, "bf16", dev),
        k_cache=gen.to_torch(x.k_cache, "bf16", dev),
        v_cache=gen.to_torch(x.v_cache, "bf16", dev),
        block_table=torch.from_numpy(x.block_table).to(dev),
        seq_lens=torch.from_numpy(x.lens.astype(np.int32)).to(dev),
    )


def run_decode(t, max_seq_len, scale, num_splits=0):
    import torch

    o = fa.fa_decode_splitk(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["seq_lens"],
                            max_seq_len, scale=scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return o


SMALL = [
    # B, Hq, Hkv, lens
    (3, 8, 8, [1, 16, 17]),
    (4, 8, 4, [15, 100, 255, 256]),
    (3, 16, 4, [1000, 4097, 33]),
    (2, 16, 2, [2000, 5]),
    (5, 32, 8, [16, 31, 1, 640, 2049]),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"B{c[0]}-Hq{c[1]}-Hkv{c[2]}")
@pytest.mark.parametrize("splits", [0, 1, 2, 7])
def test_decode_small(case, splits, dev):
    B, Hq, Hkv, lens = case
    seed = 200 + SMALL.index(case)
    log_case(f"fa_decode_splitk small {case} splits={splits} seed={seed}")
    x = gen.decode_inputs(B, Hq, Hkv, 128, 16, seed=seed, lens=lens,
                          max_pages_per_seq=-(-max(lens) // 16) + 3)
    t = upload(x, dev)
    o = run_decode(t, x.max_seq_len, x.scale, splits)
    o_ref, _, _ = oracle.decode(x.q, x.k_seqs, x.v_seqs, x.scale)
    assert_close(to_np(o), o_ref, "bf16", "decode O")


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"B{c[0]}-Hq{c[1]}-Hkv{c[2]}")
@pytest.mark.parametrize("splits", [3, 16])
def test_decode_split_counts(case, splits, dev):
    """Explicit split counts (the last chunk of every (sequence, KV head) merges in the same
    launch), against the oracle, on tables wider than the sequences."""
    B, Hq, Hkv, lens = case
    seed = 300 + SMALL.index(case)
    log_case(f"fa_decode_splitk {case} splits={splits} seed={seed}")
    x = gen.decode_inputs(B, Hq, Hkv, 128, 16, seed=seed, lens=lens,
                          max_pages_per_seq=-(-max(lens) // 16) + 3)
    t = upload(x, dev)
    o = run_decode(t, x.max_seq_len, x.scale, splits)
    o_ref, _, _ = oracle.decode(x.q, x.k_seqs, x.v_seqs, x.scale)
    assert_close(to_np(o), o_ref, "bf16", "decode O")


EDGE = [
    # B, Hq, Hkv, lens: the automatic plan on awkward length mixes
    (1, 8, 1, [40000]),                      # one (sequence, KV head) pair: many chunks
    (1, 4, 4, [20]),                         # two pages in all
    (6, 8, 2, [0, 300, 0, 0, 1, 5000]),      # empty sequences between and before others
    (70, 8, 2, None),                        # many sequences, a fifth of them empty
    (9, 16, 2, [17, 33, 4097, 16, 15, 2, 900, 1, 64]),
]


@pytest.mark.parametrize("case", EDGE, ids=lambda c: f"B{c[0]}-Hq{c[1]}-Hkv{c[2]}")
def test_decode_edge_lengths(case, dev):
    B, Hq, Hkv, lens = case
    seed = 400 + EDGE.index(case)
    if lens is None:
        rng = np.random.default_rng(seed)
        lens = [int(v) if rng.random() > 0.2 else 0 for v in rng.integers(1, 3000, size=B)]
    log_case(f"fa_decode_splitk edge {B, Hq, Hkv} lens={lens[:10]} seed={seed}")
    x = gen.decode_inputs(B, Hq, Hkv, 128, 16, seed=seed, lens=lens,
                          max_pages_per_seq=-(-max(max(lens), 1) // 16) + 2)
    t = upload(x, dev)
    o = to_np(run_decode(t, x.max_seq_len, x.scale))
    o_ref, _, _ = oracle.decode(x.q, x.k_seqs, x.v_seqs, x.scale)
    assert_close(o, o_ref, "bf16", "decode O")
    for b in range(B):
        if lens[b] == 0:
            assert np.all(o[b] == 0)


def test_decode_all_empty(dev):
    log_case("fa_decode_splitk, every length 0")
    x = gen.decode_inputs(3, 8, 2, 128, 16, seed=410, lens=[0, 0, 0], max_pages_per_seq=2)
    o = to_np(run_decode(upload(x, dev), 0, x.scale))
    assert np.all(o == 0)


def test_decode_length_clamped_to_table(dev):
    """Lengths beyond max_pages_per_seq * 16 are clamped (automatic and explicit splits): the
    result is that of the clamped sequence."""
    import torch

    log_case("fa_decode_splitk clamp")
    x = gen.decode_inputs(2, 8, 2, 128, 16, seed=411, lens=[64, 50])
    t = upload(x, dev)
    t["seq_lens"] = torch.tensor([100, 50], dtype=torch.int32, device=dev)  # beyond 4 pages
    o_ref, _, _ = oracle.decode(x.q, x.k_seqs, x.v_seqs, x.scale)
    for splits in (0, 2):
        o = fa.fa_decode_splitk(t["q"], t["k_cache"], t["v_cache"], t["block_table"],
                                t["seq_lens"], 64, scale=x.scale, num_splits=splits)
        torch.cuda.synchronize()
        assert_close(to_np(o), o_ref, "bf16", f"clamped, splits={splits}")


def test_decode_config5_full(dev):
    import torch

    cfg = gen.CONFIGS[5]
    log_case(f"fa_decode_splitk config: {cfg.name}")
    x = gen.config_decode_inputs(cfg)
    t = upload(x, dev)
    o = run_decode(t, cfg.len_max, x.scale)
    o2 = run_decode(t, cfg.len_max, x.scale)
    assert torch.equal(o, o2), "two runs differ: the kernel is not deterministic"
    o_ref, _, _ = oracle.decode(x.q, x.k_seqs, x.v_seqs, x.scale)
    assert_close(to_np(o), o_ref, "bf16", "config 5 O")
    for s in (1, 2, 7):
        log_case(f"fa_decode_splitk config 5 num_splits={s}")
        assert_close(to_np(run_decode(t, cfg.len_max, x.scale, s)), o_ref, "bf16", f"splits={s}")
    del t, o, o2
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fill", ["zeros", "ones", "random"])
def test_decode_workspace_contents_do_not_matter(fill, dev):
    """The workspace may hold anything on entry (the completion words included): the result
    is bitwise that of a fresh call, on every split count and on repeated calls."""
    import torch

    log_case(f"fa_decode_splitk workspace filled with {fill}")
    x = gen.decode_inputs(5, 32, 8, 128, 16, seed=305, lens=[3000, 17, 1500, 2049, 640])
    t = upload(x, dev)
    o_ref, _, _ = oracle.decode(x.q, x.k_seqs, x.v_seqs, x.scale)
    for splits in (0, 2, 5):
        need = fa.fa_decode_workspace_bytes(5, 32, 128, 16, x.max_seq_len, splits)
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        outs = []
        for rep in range(3):
            if fill == "zeros":
                ws.zero_()
            elif fill == "ones":
                ws.fill_(255)
            else:
                g = torch.Generator(device="cpu").manual_seed(1000 * splits + rep)
                ws.copy_(torch.randint(0, 256, (need,), dtype=torch.uint8, generator=g))
            o = fa.fa_decode_splitk(t["q"], t["k_cache"], t["v_cache"], t["block_table"],
                                    t["seq_lens"], x.max_seq_len, scale=x.scale,
                                    num_splits=splits, workspace=ws)
            torch.cuda.synchronize()
            outs.append(o)
        assert all(torch.equal(outs[0], u) for u in outs[1:])
        assert_close(to_np(outs[0]), o_ref, "bf16", f"splits={splits}")


def test_decode_physical_page_order_does_not_matter(dev):
    """Moving pages to other physical slots (and fixing the table) gives bitwise the same O."""
    import torch

    log_case("fa_decode_splitk page permutation")
    x = gen.decode_inputs(4, 16, 4, 128, 16, seed=301, lens=[700, 1, 64, 333])
    t1 = upload(x, dev)
    o1 = run_decode(t1, x.max_seq_len, x.scale)
    rng = np.random.default_rng(7)
    perm = rng.permutation(x.num_pages)  # old slot -> new slot
    k2 = np.empty_like(x.k_cache)
    v2 = np.empty_like(x.v_cache)
    k2[perm] = x.k_cache
    v2[perm] = x.v_cache
    table2 = np.where(x.block_table >= 0, perm[np.maximum(x.block_table, 0)], -1).astype(np.int32)
    x2 = gen.DecodeInputs(x.lens, x.q, x.k_seqs, x.v_seqs, k2, v2, table2, 16, x.scale)
    o2 = run_decode(upload(x2, dev), x.max_seq_len, x.scale)
    assert torch.equal(o1, o2)


def test_decode_zero_length_sequence(dev):
    log_case("fa_decode_splitk zero length")
    x = gen.decode_inputs(3, 8, 2, 128, 16, seed=302, lens=[0, 40, 0], max_pages_per_seq=4)
    o = to_np(run_decode(upload(x, dev), 40, x.scale))
    assert np.all(o[0] == 0) and np.all(o[2] == 0)
    o_ref, _, _ = oracle.decode(x.q, x.k_seqs, x.v_seqs, x.scale)
    assert_close(o[1], o_ref[1], "bf16", "decode O")


def test_decode_equals_last_row_of_causal_prefill(dev):
    """The one decode query is the newest token: same result as the last prefill row."""
    import torch

    log_case("fa_decode_splitk vs fa_fwd last row")
    L, Hq, Hkv = 777, 8, 2
    xf = gen.fwd_inputs(1, Hq, Hkv, L, 128, seed=303, dtype="bf16", causal=True)
    o_f = fa.fa_fwd(gen.to_torch(xf.q, "bf16", dev), gen.to_torch(xf.k, "bf16", dev),
                    gen.to_torch(xf.v, "bf16", dev), causal=True)
    xd = gen.decode_inputs(1, Hq, Hkv, 128, 16, seed=303, lens=[L])
    # overwrite the drawn sequence with the prefill's K/V and last query row
    npg = -(-L // 16)
    for cache, seq in ((xd.k_cache, xf.k[0]), (xd.v_cache, xf.v[0])):
        padded = np.full((Hkv, npg * 16, 128), np.nan, np.float32)
        padded[:, :L] = seq
        cache[xd.block_table[0, :npg]] = padded.reshape(Hkv, npg, 16, 128).transpose(1, 0, 2, 3)
    xd.q[0] = xf.q[0, :, L - 1]
    o_d = run_decode(upload(xd, dev), L, xd.scale)
    torch.cuda.synchronize()
    last = to_np(o_f)[0, :, L - 1]
    got = to_np(o_d)[0]
    np.testing.assert_allclose(got, last, atol=2e-2, rtol=1e-2)
    ref, _, _ = oracle.attention(xf.q[:, :, L - 1:], xf.k, xf.v, xf.scale, causal=False)
    assert_close(got, ref[0, :, 0], "bf16", "decode vs oracle")
