"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module draws random numbers, rounds them to bfloat16 and lays K/V out in pages. It
holds none of the attention arithmetic, and neither the oracle nor the HIP path imports
the other through it.

Workloads (the shapes of prefill at 2K-32K tokens and long-context decode that the pages
discuss; every value is drawn from N(0, 1) with numpy's PCG64 ``default_rng(seed)``):

1. single-head forward, fp32: B=1, H=1, N=256, d=64, no mask, seed 1.
2. causal multi-head prefill, bf16: B=4, H=16, N=2048, d=64, seed 2.
3. causal multi-head prefill (long), bf16: B=2, H=32, N=8192, d=128, K scaled by 2 so that
   softmax rows are peaky, seed 3.
4. causal grouped-query prefill, bf16: B=1, 32 query heads over 8 KV heads, N=32768,
   d=128, seed 4.
5. split-K decode over a paged KV cache, bf16: B=8 sequences with one query token each,
   32 query heads over 8 KV heads, d=128, lengths uniform in [16384, 32768] (inclusive),
   16-token pages at randomly permuted physical slots named by an int32 block table,
   seed 5.

Beyond these five: chunked prefill over the paged cache (``PREFILL_PAGED``): 4 sequences of
4096 to 16384 cached tokens whose newest 2048 are the queries, 32 query heads over 8 KV
heads, d=128, causal with the diagonal at the bottom right, pages laid out as for decode,
seed 6.

Draw order: Q, then K, then V (forward); lengths, q, then K_b and V_b per sequence, then
the page permutation (decode and paged prefill). Values are rounded to bfloat16 with round-to-nearest-even
before anyone sees them, so both sides receive identical, exactly representable inputs.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BF16_NAN_BITS = 0x7FC0


@dataclass(frozen=True)
class FwdConfig:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    dtype: str  # "f32" or "bf16"
    causal: bool
    seed: int
    k_mult: float = 1.0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def flops(self) -> float:
        """Algorithmic FLOPs: 4*d per admissible (query, key) pair (two contractions)."""
        per_head = self.N * (self.N + 1) / 2 if self.causal else float(self.N) * self.N
        return 4.0 * self.d * per_head * self.B * self.Hq


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    page_size: int
    len_min: int
    len_max: int
    seed: int
    lens: tuple = field(default=())  # fixed lengths instead of drawing them

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


CONFIGS = {
    1: FwdConfig("single-head fwd fp32 B=1 H=1 N=256 d=64", 1, 1, 1, 256, 64, "f32", False, 1),
    2: FwdConfig("causal MHA prefill bf16 B=4 H=16 N=2048 d=64", 4, 16, 16, 2048, 64, "bf16", True, 2),
    3: FwdConfig("causal MHA prefill bf16 B=2 H=32 N=8192 d=128 (K x2)", 2, 32, 32, 8192, 128,
                 "bf16", True, 3, k_mult=2.0),
    4: FwdConfig("causal GQA prefill bf16 B=1 Hq=32 Hkv=8 N=32768 d=128", 1, 32, 8, 32768, 128,
                 "bf16", True, 4),
    5: DecodeConfig("paged split-K decode bf16 B=8 Hq=32 Hkv=8 d=128 L~U[16384,32768] page=16",
                    8, 32, 8, 128, 16, 16384, 32768, 5),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))
    rounded = (bits + bias) & np.uint32(0xFFFF0000)
    nan = np.isnan(x)
    if nan.any():
        rounded = np.where(nan, np.uint32(BF16_NAN_BITS << 16), rounded)
    return rounded.view(np.float32)


def round_to_e4m3(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest OCP fp8 e4m3 value (ties to even; 3 mantissa bits,
    exponent bias 7, subnormals below 2^-6 in steps of 2^-9, largest finite 448; larger
    magnitudes saturate to +-448). Returns float32 values that are e4m3-exact."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)                     # subnormal range shares the 2^-9 step
    step = np.exp2(e - 3.0)
    r = np.round(a / step) * step               # numpy rounds halves to even
    r = np.minimum(r, 448.0)
    return (np.sign(x) * r).astype(np.float32)


def e4m3_bits(x: np.ndarray) -> np.ndarray:
    """The uint8 e4m3 encodings of float32 values that are already e4m3-exact."""
    x = np.asarray(x, dtype=np.float64)
    sign = (np.signbit(x)).astype(np.uint8) << 7
    a = np.abs(x)
    normal = a >= 2.0 ** -6
    e = np.floor(np.log2(np.where(normal, a, 1.0))).astype(np.int64)
    mant_n = np.round((a / np.exp2(e) - 1.0) * 8).astype(np.int64)
    code_n = ((e + 7) << 3) | mant_n
    code_s = np.round(a / 2.0 ** -9).astype(np.int64)
    return (sign | np.where(normal, code_n, code_s).astype(np.uint8)).astype(np.uint8)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The uint16 bfloat16 encodings of float32 values that are already bf16-exact."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (bits >> np.uint32(16)).astype(np.uint16)


@dataclass
class FwdInputs:
    q: np.ndarray  # [B, Hq, N, d] float32 (bf16-exact when dtype == "bf16")
    k: np.ndarray  # [B, Hkv, N, d]
    v: np.ndarray  # [B, Hkv, N, d]
    scale: float
    causal: bool
    dtype: str


def fwd_inputs(B, Hq, Hkv, N, d, seed, dtype="bf16", causal=True, k_mult=1.0, scale=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, N, d), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, N, d), dtype=np.float32)
    if k_mult != 1.0:
        k *= np.float32(k_mult)
    v = rng.standard_normal((B, Hkv, N, d), dtype=np.float32)
    if dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    elif dtype != "f32":
        raise ValueError(dtype)
    return FwdInputs(q, k, v, 1.0 / math.sqrt(d) if scale is None else scale, causal, dtype)


def config_fwd_inputs(cfg: FwdConfig) -> FwdInputs:
    return fwd_inputs(cfg.B, cfg.Hq, cfg.Hkv, cfg.N, cfg.d, cfg.seed, cfg.dtype, cfg.causal,
                      cfg.k_mult)


@dataclass
class DecodeInputs:
    lens: np.ndarray  # [B] int32
    q: np.ndarray  # [B, Hq, d] float32, bf16-exact
    k_seqs: list  # per sequence [Hkv, L_b, d] (logical cache)
    v_seqs: list
    k_cache: np.ndarray  # [num_pages, Hkv, page_size, d]; unused slots hold NaN
    v_cache: np.ndarray
    block_table: np.ndarray  # [B, max_pages_per_seq] int32; unused entries are -1
    page_size: int
    scale: float

    @property
    def num_pages(self) -> int:
        return self.k_cache.shape[0]

    @property
    def max_seq_len(self) -> int:
        return int(self.lens.max()) if self.lens.size else 0

    def kv_bytes(self, elem_bytes=2) -> int:
        """Bytes of K and V a decode step must read: every admissible token once per KV head."""
        hkv, d = self.k_cache.shape[1], self.k_cache.shape[3]
        return int(2 * int(self.lens.sum()) * hkv * d * elem_bytes)


def _paged_cache(rng, lens, Hkv, d, page_size, max_pages_per_seq, unused_fill):
    """Draw each sequence's logical K_b and V_b, then scatter their 16-token pages to the
    physical slots of one seeded permutation. Returns (k_seqs, v_seqs, k_cache, v_cache,
    block_table)."""
    B = len(lens)
    k_seqs, v_seqs = [], []
    for b in range(B):
        k_seqs.append(round_to_bf16(rng.standard_normal((Hkv, int(lens[b]), d), dtype=np.float32)))
        v_seqs.append(round_to_bf16(rng.standard_normal((Hkv, int(lens[b]), d), dtype=np.float32)))
    pages = [-(-int(L) // page_size) for L in lens]
    total = int(sum(pages))
    perm = rng.permutation(total).astype(np.int32)
    width = max(pages + [1]) if max_pages_per_seq is None else max_pages_per_seq
    if width < max(pages + [0]):
        raise ValueError("max_pages_per_seq too small for the drawn lengths")
    block_table = np.full((B, width), -1, dtype=np.int32)
    k_cache = np.full((total, Hkv, page_size, d), unused_fill, dtype=np.float32)
    v_cache = np.full((total, Hkv, page_size, d), unused_fill, dtype=np.float32)
    offset = 0
    for b in range(B):
        npg, L = pages[b], int(lens[b])
        phys = perm[offset:offset + npg]
        block_table[b, :npg] = phys
        for cache, seq in ((k_cache, k_seqs[b]), (v_cache, v_seqs[b])):
            padded = np.full((Hkv, npg * page_size, d), unused_fill, dtype=np.float32)
            padded[:, :L] = seq
            cache[phys] = padded.reshape(Hkv, npg, page_size, d).transpose(1, 0, 2, 3)
        offset += npg
    return k_seqs, v_seqs, k_cache, v_cache, block_table


def decode_inputs(B, Hq, Hkv, d, page_size, seed, lens=None, len_min=None, len_max=None,
                  max_pages_per_seq=None, scale=None, unused_fill=np.nan):
    rng = np.random.default_rng(seed)
    if lens is None:
        lens = rng.integers(len_min, len_max + 1, size=B)
    lens = np.asarray(lens, dtype=np.int32)
    q = round_to_bf16(rng.standard_normal((B, Hq, d), dtype=np.float32))
    k_seqs, v_seqs, k_cache, v_cache, block_table = _paged_cache(
        rng, lens, Hkv, d, page_size, max_pages_per_seq, unused_fill)
    return DecodeInputs(lens, q, k_seqs, v_seqs, k_cache, v_cache, block_table, page_size,
                        1.0 / math.sqrt(d) if scale is None else scale)


def config_decode_inputs(cfg: DecodeConfig) -> DecodeInputs:
    lens = list(cfg.lens) if cfg.lens else None
    width = -(-cfg.len_max // cfg.page_size)
    return decode_inputs(cfg.B, cfg.Hq, cfg.Hkv, cfg.d, cfg.page_size, cfg.seed, lens=lens,
                         len_min=cfg.len_min, len_max=cfg.len_max, max_pages_per_seq=width)


@dataclass(frozen=True)
class PrefillPagedConfig:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    d: int
    page_size: int
    len_min: int
    len_max: int
    causal: bool
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


@dataclass
class PrefillPagedInputs:
    lens: np.ndarray  # [B] int32: cached tokens of each sequence, the Nq new ones included
    q: np.ndarray  # [B, Hq, Nq, d] float32, bf16-exact: the newest Nq tokens of each sequence
    k_seqs: list  # per sequence [Hkv, L_b, d] (logical cache)
    v_seqs: list
    k_cache: np.ndarray  # [num_pages, Hkv, page_size, d]; unused slots hold NaN
    v_cache: np.ndarray
    block_table: np.ndarray  # [B, max_pages_per_seq] int32; unused entries are -1
    page_size: int
    scale: float
    causal: bool

    @property
    def num_pages(self) -> int:
        return self.k_cache.shape[0]

    def pairs(self) -> int:
        """Admissible (query, key) pairs per query head."""
        nq = self.q.shape[2]
        total = 0
        for L in self.lens.tolist():
            pos = np.arange(L - nq, L)
            total += int(np.clip(pos + 1, 0, L).sum()) if self.causal else nq * L
        return total

    def flops(self) -> float:
        return 4.0 * self.q.shape[3] * self.pairs() * self.q.shape[1]


def prefill_paged_inputs(B, Hq, Hkv, Nq, d, page_size, seed, lens=None, len_min=None,
                         len_max=None, max_pages_per_seq=None, scale=None, causal=True,
                         unused_fill=np.nan):
    """Chunked prefill over a paged cache: each sequence's newest Nq tokens (q) against its
    L_b cached tokens. Draw order: lengths, q, then K_b and V_b per sequence, then the page
    permutation (as for decode)."""
    rng = np.random.default_rng(seed)
    if lens is None:
        lens = rng.integers(len_min, len_max + 1, size=B)
    lens = np.asarray(lens, dtype=np.int32)
    q = round_to_bf16(rng.standard_normal((B, Hq, Nq, d), dtype=np.float32))
    k_seqs, v_seqs, k_cache, v_cache, block_table = _paged_cache(
        rng, lens, Hkv, d, page_size, max_pages_per_seq, unused_fill)
    return PrefillPagedInputs(lens, q, k_seqs, v_seqs, k_cache, v_cache, block_table, page_size,
                              1.0 / math.sqrt(d) if scale is None else scale, causal)


# Chunked prefill over the paged cache (not one of the five workloads above): 4 sequences of
# 4096 to 16384 cached tokens (inclusive) whose newest 2048 are the queries, 32 query heads
# over 8 KV heads, d = 128, causal with the diagonal at the bottom right, seed 6.
PREFILL_PAGED = PrefillPagedConfig(
    "paged chunked prefill bf16 B=4 Hq=32 Hkv=8 Nq=2048 d=128 L~U[4096,16384] page=16",
    4, 32, 8, 2048, 128, 16, 4096, 16384, True, 6)


def config_prefill_paged_inputs(cfg: PrefillPagedConfig) -> PrefillPagedInputs:
    width = -(-cfg.len_max // cfg.page_size)
    return prefill_paged_inputs(cfg.B, cfg.Hq, cfg.Hkv, cfg.Nq, cfg.d, cfg.page_size, cfg.seed,
                                len_min=cfg.len_min, len_max=cfg.len_max,
                                max_pages_per_seq=width, causal=cfg.causal)


# ---- block masks for the block-sparse forward (256 query rows x 64 keys per block) ----

SPARSE_BQ, SPARSE_BK = 256, 64


def block_csr(rows):
    """Compressed rows (int32 offsets, int32 indices) from one key-block list per row."""
    offsets = np.zeros(len(rows) + 1, dtype=np.int32)
    offsets[1:] = np.cumsum([len(r) for r in rows])
    indices = np.asarray([j for r in rows for j in r], dtype=np.int32)
    return offsets, indices


def local_global_blocks(B, Hq, N, window, n_global, causal=True, bq=SPARSE_BQ, bk=SPARSE_BK):
    """Every head: query block qb lists the key blocks within `window` keys before its first
    row up to its last row (or to the end without the causal mask), and the first
    `n_global` key blocks."""
    nqb, nkb = -(-N // bq), -(-N // bk)
    rows = []
    for _ in range(B * Hq):
        for qb in range(nqb):
            lo = max(0, (qb * bq - window) // bk)
            hi = min(nkb, -(-min(N, (qb + 1) * bq) // bk)) if causal else min(nkb, -(-min(N, (qb + 1) * bq + window) // bk))
            rows.append(sorted(set(range(min(n_global, nkb))) | set(range(lo, hi))))
    return rows


def random_blocks(B, Hq, N, density, seed, bq=SPARSE_BQ, bk=SPARSE_BK):
    """Each (head, query block) lists each key block with probability `density`."""
    rng = np.random.default_rng(seed)
    nqb, nkb = -(-N // bq), -(-N // bk)
    return [sorted(np.flatnonzero(rng.random(nkb) < density).tolist()) for _ in range(B * Hq * nqb)]


def block_pairs(rows, B, Hq, N, causal, bq=SPARSE_BQ, bk=SPARSE_BK):
    """Admissible (query, key) pairs over all heads: the FLOP count's 4 d multiplier aside,
    the algorithmic work of the block-sparse forward."""
    nqb, nkb = -(-N // bq), -(-N // bk)
    total = 0
    for r, blocks in enumerate(rows):
        qb = r % nqb
        i = np.arange(qb * bq, min(N, (qb + 1) * bq))
        for kb in set(j for j in blocks if 0 <= j < nkb):
            j0, j1 = kb * bk, min(N, (kb + 1) * bk)
            if causal:
                total += int(np.clip(i + 1 - j0, 0, j1 - j0).sum())
            else:
                total += len(i) * (j1 - j0)
    return total


@dataclass(frozen=True)
class BlockSparseConfig:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    window: int
    n_global: int
    causal: bool
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


# Block-sparse forward (not one of the five workloads above): 2 x 32 query heads over 8 KV
# heads, N = 16384, d = 128, causal, each 256-row query block sees the 2048 keys before it,
# its own block and the first 256 keys (local window + global tokens), seed 7.
BLOCK_SPARSE = BlockSparseConfig(
    "block-sparse causal prefill bf16 B=2 Hq=32 Hkv=8 N=16384 d=128 window 2048 + 256 global",
    2, 32, 8, 16384, 128, 2048, 4, True, 7)


@dataclass
class Fp8Inputs:
    q: np.ndarray  # [B, Hq, N, d] float32, e4m3-exact
    k: np.ndarray  # [B, Hkv, N, d] float32, e4m3-exact
    v: np.ndarray  # [B, Hkv, N, d] float32, bf16-exact (or e4m3-exact)
    scale: float
    causal: bool


def fp8_fwd_inputs(B, Hq, Hkv, N, d, seed, causal=True, k_mult=1.0, scale=None, v_fp8=False):
    """The forward inputs of `fwd_inputs` with Q and K rounded to e4m3 instead of bf16, and V to
    e4m3 too when `v_fp8` (else bf16): the same draws, a different rounding."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, N, d), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, N, d), dtype=np.float32)
    if k_mult != 1.0:
        k *= np.float32(k_mult)
    v = rng.standard_normal((B, Hkv, N, d), dtype=np.float32)
    return Fp8Inputs(round_to_e4m3(q), round_to_e4m3(k), round_to_e4m3(v) if v_fp8 else round_to_bf16(v),
                     1.0 / math.sqrt(d) if scale is None else scale, causal)


def to_torch(x: np.ndarray, dtype: str, device="cuda"):
    """Upload a float32 array as a torch tensor of ``dtype`` ("f32", "bf16" or "e4m3", the last
    as uint8 codes), exactly."""
    import torch

    if dtype == "e4m3":
        return torch.from_numpy(e4m3_bits(x)).to(device).contiguous()
    if dtype == "bf16":
        bits = bf16_bits(x).view(np.int16)
        t = torch.from_numpy(bits).view(torch.bfloat16)
    elif dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    else:
        raise ValueError(dtype)
    return t.to(device).contiguous()
