"""Host-side checks of the seeded input generators (CPU only)."""

import numpy as np
import torch

from exact_tiled_attention_24_amd import inputs as gen


def test_round_to_bf16_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100_000).astype(np.float32) * 10
    # exact ties: bf16 keeps 8 significant bits, so 1 + 2^-8 is halfway between neighbours
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -130, 3.0e38], np.float32)
    x = np.concatenate([x, ties])
    ours = gen.round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours, ref)
    assert gen.round_to_bf16(np.array([1 + 2 ** -8], np.float32))[0] == 1.0  # tie to even


def test_bf16_bits_roundtrip():
    x = gen.round_to_bf16(np.random.default_rng(1).standard_normal(1000).astype(np.float32))
    bits = gen.bf16_bits(x)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    np.testing.assert_array_equal(back, x)


def test_fwd_inputs_deterministic_and_exact():
    a = gen.fwd_inputs(2, 4, 2, 33, 16, seed=7, dtype="bf16", k_mult=2.0)
    b = gen.fwd_inputs(2, 4, 2, 33, 16, seed=7, dtype="bf16", k_mult=2.0)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v)):
        np.testing.assert_array_equal(x, y)
        np.testing.assert_array_equal(gen.round_to_bf16(x), x)
    assert a.q.shape == (2, 4, 33, 16) and a.k.shape == (2, 2, 33, 16)
    c = gen.fwd_inputs(2, 4, 2, 33, 16, seed=7, dtype="bf16", k_mult=1.0)
    np.testing.assert_array_equal(a.k, 2 * c.k)  # scaling by 2 commutes with rounding
    assert abs(a.scale - 0.25) < 1e-15


def test_config_table():
    c3 = gen.CONFIGS[3]
    assert (c3.B, c3.Hq, c3.N, c3.d, c3.causal, c3.k_mult) == (2, 32, 8192, 128, True, 2.0)
    assert abs(c3.flops() - 1.0996e12) / 1.0996e12 < 1e-3
    c4 = gen.CONFIGS[4]
    assert c4.Hq // c4.Hkv == 4 and c4.N == 32768
    c5 = gen.CONFIGS[5]
    assert (c5.B, c5.Hq, c5.Hkv, c5.page_size) == (8, 32, 8, 16)


def test_decode_pages_gather_back_to_logical():
    di = gen.decode_inputs(B=3, Hq=4, Hkv=2, d=8, page_size=16, seed=3, lens=[1, 16, 45],
                           max_pages_per_seq=5)
    assert di.block_table.shape == (3, 5)
    used = np.concatenate([di.block_table[b, :-(-L // 16)] for b, L in enumerate(di.lens)])
    assert sorted(used.tolist()) == list(range(di.num_pages))  # a permutation of all slots
    for b, L in enumerate(di.lens):
        npg = -(-int(L) // 16)
        assert np.all(di.block_table[b, npg:] == -1)
        for cache, seqs in ((di.k_cache, di.k_seqs), (di.v_cache, di.v_seqs)):
            pages = cache[di.block_table[b, :npg]]  # [npg, Hkv, 16, d]
            logical = pages.transpose(1, 0, 2, 3).reshape(2, npg * 16, 8)
            np.testing.assert_array_equal(logical[:, :L], seqs[b])
            assert np.all(np.isnan(logical[:, L:]))  # unused slots poison any stray read
    assert di.kv_bytes() == 2 * (1 + 16 + 45) * 2 * 8 * 2


def test_decode_lengths_drawn_inclusive_range():
    di = gen.decode_inputs(B=64, Hq=2, Hkv=1, d=4, page_size=16, seed=5, len_min=3, len_max=5)
    assert set(di.lens.tolist()) <= {3, 4, 5} and len(set(di.lens.tolist())) == 3


def test_e4m3_rounding_and_codes():
    """OCP e4m3: 1.0 = 0x38, 1.5 = 0x3c, 448 (largest finite) = 0x7e, 2^-6 (smallest normal) =
    0x08, 2^-9 (smallest subnormal) = 0x01; ties round to even; magnitudes past 448 saturate."""
    from exact_tiled_attention_24_amd import inputs as gen

    vals = np.array([1.0, 1.5, 448.0, 2.0 ** -6, 2.0 ** -9, -3.0, 0.0], np.float32)
    codes = [0x38, 0x3C, 0x7E, 0x08, 0x01, 0xC4, 0x00]
    assert np.array_equal(gen.round_to_e4m3(vals), vals)
    assert gen.e4m3_bits(vals).tolist() == codes
    # 1 + 1/16 lies halfway between 1 and 1.125: to even (1.0); 1 + 3/16 -> 1.25
    r = gen.round_to_e4m3(np.array([1.0625, 1.1875, 1000.0, -1000.0, 2.0 ** -10 * 3], np.float32))
    assert r.tolist() == [1.0, 1.25, 448.0, -448.0, 2.0 ** -9 * 2]
    # every code 0x00..0x7e decodes back to itself through the value grid
    x = np.random.default_rng(0).standard_normal(10000).astype(np.float32) * 8
    y = gen.round_to_e4m3(x)
    assert np.all(np.abs(y - x) <= np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10) + 1e-12)
    assert np.array_equal(gen.round_to_e4m3(y), y)
