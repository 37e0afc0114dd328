/*
 * fa.h - C ABI of libfa.so: exact tiled attention on AMD Instinct MI355X (gfx950).
 *
 * Three operations, each exact attention O = softmax(scale * Q K^T + M) V computed without
 * ever writing the N x N score matrix to device memory:
 *
 *   fa_fwd            tiled forward with the online softmax (running max m, running sum l,
 *                     rescaled accumulator O); "FlashAttention" (shubhamtatvamasi.com),
 *                     "The trick: tiles and an online softmax", and "FlashAttention,
 *                     explained." (vibeengines.com), the forward-pass statement.
 *   fa_decode_splitk  single-query decode over a paged KV cache read through a block table,
 *                     with the KV sequence split across workgroups and the partial (m, l, O)
 *                     results merged; "FlashAttention", "Decode is a different problem" and
 *                     the FlashAttention-family table (Flash-Decoding, paged variants).
 *   fa_merge          merge of partial (m, l, O) results over disjoint key sets with the
 *                     online-softmax rescale; "FlashAttention", "Decode is a different problem".
 *   fa_fwd_fp8        tiled forward with fp8 (e4m3) Q and K on the fp8 matrix cores; the
 *                     FP8 row of the FlashAttention-family table ("FlashAttention").
 *   fa_bwd            backward by recomputation (dQ, dK, dV from Q, K, V, O, dO and the saved
 *                     row statistics); "FlashAttention, explained." (vibeengines.com),
 *                     backward-pass section.
 *   fa_fwd_block_sparse  tiled forward that visits only the key blocks a block mask lists;
 *                     "FlashAttention, explained." (vibeengines.com), block-sparse section.
 *   fa_fwd_paged      tiled forward for the newest tokens of each sequence against its whole
 *                     paged KV cache (chunked prefill); the paged variants of the
 *                     FlashAttention-family table ("FlashAttention") with the update rule of
 *                     "The trick: tiles and an online softmax". A shared prefix is handled by
 *                     two calls (prefix unmasked, the rest causal) and fa_merge.
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller. The library allocates
 *     and frees nothing; the decode workspace is passed in by the caller.
 *   - Tensors are dense and row-major (C-contiguous) in the shapes stated per function.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Calls enqueue work
 *     on it and return; they never synchronise the device.
 *   - Arguments are validated on the host before any HIP call; a rejected call launches
 *     nothing and returns FA_ERR_INVALID_ARGUMENT or FA_ERR_UNSUPPORTED. A failed launch
 *     returns FA_ERR_HIP. Nothing is thrown across the ABI.
 *   - m is reported in natural-log units: m = max_j (scale * q.k_j); l = sum_j exp(s_j - m).
 *     A row with no admissible key yields O = 0, m = -inf, l = 0.
 *   - Results are deterministic: the same inputs give bitwise-identical outputs.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARGUMENT = 1,   /* NULL pointer, negative size, bad scale, ... */
    FA_ERR_UNSUPPORTED = 2,        /* valid request this build has no kernel for */
    FA_ERR_WORKSPACE_TOO_SMALL = 3,
    FA_ERR_HIP = 4                 /* the HIP runtime reported an error at launch */
} fa_status;

typedef enum {
    FA_F32 = 0,   /* IEEE binary32 */
    FA_BF16 = 1,  /* bfloat16 (round-to-nearest-even on output) */
    FA_E4M3 = 2   /* OCP fp8 e4m3: sign, 4 exponent bits (bias 7), 3 mantissa bits; max 448 */
} fa_dtype;

/*
 * fa_fwd - tiled attention forward (prefill).
 *
 *   q, o : [B, Hq, N, d]   in `dt`
 *   k, v : [B, Hkv, N, d]  in `dt`; query head h reads key/value head h / (Hq / Hkv)
 *   m_out, l_out : optional float32 [B, Hq, N] row statistics (NULL = not written)
 *
 * causal != 0 admits key j for query i iff j <= i (diagonal included); tiles entirely above
 * the diagonal are never loaded. The 1/sqrt(d) scale of the pages is passed as `scale`
 * (must be finite and > 0).
 * dt = FA_BF16: bf16 inputs, float32 accumulation and softmax, bf16 output.
 * dt = FA_F32: float32 throughout.
 * Supported: d in {64, 128}; Hq % Hkv == 0; N * d < 2^31, and for FA_BF16 N * d * 2 <= 2^30
 * (a head's K or V rows span at most 2^30 bytes: the kernel addresses them with 32-bit
 * offsets and keeps offsets at 2^31 and above as "outside the tile"; N <= 4M at d = 128);
 * else FA_ERR_UNSUPPORTED. B, Hq or N equal to 0 is a valid empty call (nothing is
 * launched).
 */
fa_status fa_fwd(fa_dtype dt, const void* q, const void* k, const void* v, void* o,
                 float* m_out, float* l_out, int B, int Hq, int Hkv, int N, int d,
                 float scale, int causal, void* stream);

/*
 * fa_decode_splitk - one query token per sequence against its paged KV cache.
 *
 *   q, o        : [B, Hq, d] bf16
 *   k_cache,
 *   v_cache     : [num_pages, Hkv, page_size, d] bf16; token t of sequence b lives in
 *                 physical page block_table[b][t / page_size], slot t % page_size
 *   block_table : int32 [B, max_pages_per_seq], device memory
 *   seq_lens    : int32 [B], device memory; every key of the sequence is admissible
 *   max_seq_len : host-side upper bound of seq_lens, used to plan the KV split
 *   num_splits  : 0 = automatic; otherwise the number of KV chunks the longest sequence is
 *                 split into (clamped to [1, pages of the longest sequence])
 *   workspace   : device scratch of at least fa_decode_workspace_bytes(...) bytes holding
 *                 one completion word per (sequence, KV head) and the float32 partial
 *                 (m, l, O) of every chunk; contents on entry are ignored (a completion
 *                 word carries a tag of the call that wrote it, so stale or arbitrary words
 *                 count as empty, and the last arrival leaves it at zero, so a launch
 *                 replayed from a captured graph, tag and all, starts clean as well)
 *
 * One launch: each chunk of a sequence's pages yields a partial; the last chunk of each
 * (sequence, KV head) to finish merges the partials, in chunk order, into o. Calls that
 * share one workspace must not overlap in time (enqueue them on one stream).
 *
 * Caller preconditions that are not checked on the device: seq_lens[b] <= max_seq_len, and
 * block_table[b][p] in [0, num_pages) for p < ceil(seq_lens[b] / page_size). The kernel
 * clamps each length to min(max_seq_len, max_pages_per_seq * page_size) and never
 * dereferences a table entry outside [0, num_pages) (such a page contributes nothing), so
 * a violated precondition gives a wrong result, never an out-of-bounds access. Table
 * entries past a sequence's last page are never read. A sequence of length 0 gets O = 0.
 * Supported: dt = FA_BF16; d = 128; page_size = 16; Hq / Hkv in {1, 2, 4, 8} (other exact
 * ratios return FA_ERR_UNSUPPORTED); Hq % Hkv != 0 is FA_ERR_INVALID_ARGUMENT.
 */
fa_status fa_decode_splitk(fa_dtype dt, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_table, const int32_t* seq_lens, void* o,
                           int B, int Hq, int Hkv, int d, int page_size, int num_pages,
                           int max_pages_per_seq, int max_seq_len, float scale, int num_splits,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_decode_splitk_noalloc - fa_decode_splitk without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation). Same arguments (minus workspace), semantics and results.
 *
 * The completion words and partials live in a static scratch array of the library, one copy
 * per device, of fa_decode_noalloc_max_bytes() bytes (16 MiB), held until the process ends.
 * A request whose partials would not fit (fa_decode_workspace_bytes(...) > that size, about
 * B * Hq * splits > 31K at d = 128) returns FA_ERR_WORKSPACE_TOO_SMALL and launches nothing.
 * The call allocates nothing (no hipMalloc, hipFree or allocating library routine); its
 * first call on a device looks up that device's scratch address once.
 * Every call on one device shares that device's scratch: calls that overlap in time on one
 * device (on different streams, or from different threads) race and give wrong results.
 * Enqueue them on one stream, or use fa_decode_splitk with a workspace per stream.
 */
fa_status fa_decode_splitk_noalloc(fa_dtype dt, const void* q, const void* k_cache,
                                   const void* v_cache, const int32_t* block_table,
                                   const int32_t* seq_lens, void* o, int B, int Hq, int Hkv, int d,
                                   int page_size, int num_pages, int max_pages_per_seq,
                                   int max_seq_len, float scale, int num_splits, void* stream);

/* Bytes of the static scratch fa_decode_splitk_noalloc uses (its largest workspace). */
size_t fa_decode_noalloc_max_bytes(void);

/* Workspace bytes fa_decode_splitk needs for these sizes (0 for an invalid request). */
size_t fa_decode_workspace_bytes(int B, int Hq, int d, int page_size, int max_seq_len,
                                 int num_splits);

/* The number of KV chunks the automatic plan gives the longest sequence (0 if invalid). */
int fa_decode_plan_splits(int B, int Hkv, int page_size, int max_seq_len);

/*
 * fa_fwd_fp8 - tiled forward with fp8 queries and keys, and optionally fp8 values.
 *
 *   q : [B, Hq, N, d] OCP fp8 e4m3 (one byte per element)
 *   k : [B, Hkv, N, d] e4m3
 *   v : [B, Hkv, N, d] in v_dt: FA_BF16 or FA_E4M3
 *   o : [B, Hq, N, d] bf16
 *   m_out, l_out : optional float32 [B, Hq, N] row statistics (NULL = not written)
 *
 * Computes what fa_fwd computes for the real values the codes stand for: the scores
 * scale * q.k are exact products of e4m3 values accumulated in float32, so a per-tensor
 * descale of q and k is passed by folding it into `scale` (finite, > 0). Softmax in float32.
 * v_dt = FA_BF16: P rounded to bf16 for P V on the bf16 matrix cores.
 * v_dt = FA_E4M3: P rounded to e4m3 (round to nearest even) and P V on the fp8 matrix cores;
 * l is the sum of the rounded weights, so O is a convex combination of V rows. The exponent
 * reference r of a row moves when a tile's maximum passes it by more than 2^8, and then to 2^4
 * below that maximum: a weight is at most 256 r (never saturated) and r is at most 2^-4 of
 * the row's largest weight. The rounding of P is the one added error: each weight w_j moves by
 * at most b_j = min(w_j, max(2^-4 w_j, 2^-14 max_i w_i)) (3 mantissa bits; e4m3 subnormals
 * step by 2^-9 r), which bounds |O - exact| elementwise by
 * sum_j b_j |v_j - O| / (1 - sum_j b_j) (w the exact softmax weights, normalised) and
 * |l / exact - 1| by sum_j b_j. A per-tensor descale of v multiplies O. float32 accumulation,
 * bf16 output.
 * causal as in fa_fwd. Supported: d = 128; Hq % Hkv == 0 (else FA_ERR_INVALID_ARGUMENT);
 * N * d * 2 <= 2^30. B, Hq or N equal to 0 is a valid empty call.
 */
fa_status fa_fwd_fp8(fa_dtype v_dt, const void* q, const void* k, const void* v, void* o,
                     float* m_out, float* l_out, int B, int Hq, int Hkv, int N, int d, float scale,
                     int causal, void* stream);

/*
 * fa_bwd - gradients of fa_fwd's output with respect to q, k and v.
 *
 *   q, o, dout, dq : [B, Hq, N, d] bf16;  k, v, dk, dv : [B, Hkv, N, d] bf16
 *   m, l           : float32 [B, Hq, N], the row statistics fa_fwd returned for (q, k, v)
 *   workspace      : device scratch of at least fa_bwd_workspace_bytes(B, Hq, N) bytes;
 *                    contents on entry are ignored
 *
 * With P = exp(scale q k^T + M - m) / l, D_i = sum_c dout_ic o_ic and dP = dout v^T:
 * dv = P^T dout, dS = P * (dP - D), dq = scale dS k, dk = scale dS^T q. A key/value head shared
 * by several query heads receives the sum of their gradients. `causal` and `scale` must be the
 * forward's. float32 accumulation; dq, dk, dv rounded to bf16 once. Rows with l = 0 contribute
 * nothing. Supported: dt = FA_BF16; d in {64, 128}; Hq % Hkv == 0 (else
 * FA_ERR_INVALID_ARGUMENT); N * d < 2^30 (a head's bytes fit a signed 32-bit count);
 * B * Hq < 65536. B, Hq or N equal to 0 is a valid empty call.
 */
fa_status fa_bwd(fa_dtype dt, const void* q, const void* k, const void* v, const void* o,
                 const void* dout, const float* m, const float* l, void* dq, void* dk, void* dv,
                 int B, int Hq, int Hkv, int N, int d, float scale, int causal, void* workspace,
                 size_t workspace_bytes, void* stream);

/* Workspace bytes fa_bwd needs (two float32 values per query row, a head's rows padded to a
 * multiple of 32; 0 for negative sizes). */
size_t fa_bwd_workspace_bytes(int B, int Hq, int N);

/* Block sizes of fa_fwd_block_sparse's mask: query rows per block, keys per block. */
#define FA_SPARSE_BLOCK_Q 256
#define FA_SPARSE_BLOCK_K 64

/*
 * fa_fwd_block_sparse - tiled forward restricted to listed (query block, key block) pairs.
 *
 *   q, o    : [B, Hq, N, d] bf16;  k, v : [B, Hkv, N, d] bf16 (GQA as in fa_fwd)
 *   m_out, l_out : optional float32 [B, Hq, N] row statistics (NULL = not written)
 *   block_offsets : int32 [B * Hq * ceil(N / 256) + 1], device memory
 *   block_indices : int32 [nnz], device memory
 *
 * Query block qb (rows 256 qb .. 256 qb + 255) of head (b, h) attends to the key blocks
 * (keys 64 kb .. 64 kb + 63) block_indices[block_offsets[r] .. block_offsets[r + 1]) with
 * r = (b * Hq + h) * ceil(N / 256) + qb, in that order; with causal != 0 key j is further
 * limited to j <= i. An index outside [0, ceil(N / 64)) names no key; a block listed twice
 * counts twice (the caller lists each at most once). A query that admits no key yields O = 0,
 * m = -inf, l = 0. Each list is clamped into [0, nnz], so no offset makes the kernel read
 * outside block_indices. Every listed block is computed: blocks that lie wholly above the
 * causal diagonal cost time and contribute nothing.
 * Supported: dt = FA_BF16; d in {64, 128}; Hq % Hkv == 0 (else FA_ERR_INVALID_ARGUMENT);
 * N * d * 2 <= 2^30 (as fa_fwd); nnz >= 0. B, Hq or N equal to 0 is a valid empty call.
 */
fa_status fa_fwd_block_sparse(fa_dtype dt, const void* q, const void* k, const void* v, void* o,
                              float* m_out, float* l_out, const int32_t* block_offsets,
                              const int32_t* block_indices, int nnz, int B, int Hq, int Hkv,
                              int N, int d, float scale, int causal, void* stream);

/*
 * fa_fwd_paged - tiled forward of each sequence's newest Nq tokens against its paged cache.
 *
 *   q, o        : [B, Hq, Nq, d] bf16; query i of sequence b is the token at position
 *                 seq_lens[b] - Nq + i (the chunk's own K/V are already in the cache)
 *   k_cache,
 *   v_cache     : [num_pages, Hkv, 16, d] bf16; token t of sequence b lives in physical page
 *                 block_table[b][t / 16], slot t % 16; query head h reads KV head h / (Hq / Hkv)
 *   block_table : int32 [B, max_pages_per_seq], device memory
 *   seq_lens    : int32 [B], device memory: cached tokens of each sequence, chunk included
 *   q_lens      : optional int32 [B], device memory: new tokens of each sequence, n_b =
 *                 clamp(q_lens[b], 0, Nq), in rows 0 .. n_b - 1 of q and o (NULL: n_b = Nq);
 *                 rows n_b .. Nq - 1 of o, m_out and l_out are not written
 *   m_out, l_out: optional float32 [B, Hq, Nq] row statistics (NULL = not written)
 *
 * causal != 0 admits key j for query i iff j <= seq_lens[b] - n_b + i (the diagonal aligned to
 * the bottom right); causal == 0 admits every j < seq_lens[b]. A query that admits no key
 * (seq_lens[b] < n_b, causal, or seq_lens[b] == 0) yields O = 0, m = -inf, l = 0. `scale`
 * must be finite and > 0. bf16 inputs, float32 accumulation and softmax, bf16 output.
 *
 * Caller preconditions that are not checked on the device: block_table[b][p] in
 * [0, num_pages) for p < ceil(seq_lens[b] / 16). Each length is clamped to
 * [0, max_pages_per_seq * 16]; a table entry outside [0, num_pages) is never dereferenced
 * (its page reads as zeros), so a violated precondition gives a wrong result, never an
 * out-of-bounds access. Entries past a sequence's last page are not used.
 * Supported: dt = FA_BF16; d in {64, 128}; page_size = 16; Hq % Hkv == 0 (else
 * FA_ERR_INVALID_ARGUMENT); Nq * d * 2 <= 2^30; each cache under 2 GiB (num_pages * Hkv * 16 *
 * d * 2 bytes < 2^31, about 1M tokens at Hkv = 8, d = 128), else FA_ERR_UNSUPPORTED.
 * B, Hq or Nq equal to 0 is a valid empty call.
 */
fa_status fa_fwd_paged(fa_dtype dt, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_table, const int32_t* seq_lens,
                       const int32_t* q_lens, void* o,
                       float* m_out, float* l_out, int B, int Hq, int Hkv, int Nq, int d,
                       int page_size, int num_pages, int max_pages_per_seq, float scale,
                       int causal, void* stream);

/*
 * fa_merge - merge S partial results over disjoint key sets, row by row.
 *
 *   o_parts : float32 [S, R, d], each partial normalised (O_s = sum p v / l_s)
 *   m_parts, l_parts : float32 [S, R], natural-log units as above
 *   o       : [R, d] in `out_dt` (FA_F32 or FA_BF16)
 *   m_out, l_out : optional float32 [R] merged statistics (NULL = not written)
 *
 * With m = max_s m_s and w_s = l_s * exp(m_s - m): l = sum_s w_s, O = sum_s w_s O_s / l.
 * A partial with l_s = 0 carries no weight. Supported: S >= 1, 1 <= d <= 1024.
 * R == 0 is a valid empty call.
 */
fa_status fa_merge(fa_dtype out_dt, const float* o_parts, const float* m_parts,
                   const float* l_parts, void* o, float* m_out, float* l_out, int S, int R,
                   int d, void* stream);

/* Static, human-readable text for a status code. */
const char* fa_status_string(fa_status s);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
