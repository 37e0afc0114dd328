// fa_api.hip - the C ABI declared in include/fa.h: argument validation, split planning and
// kernel dispatch. Validation happens before any HIP call, so a rejected request neither
// touches the device nor needs one.
#include <math.h>

#include <atomic>
#include <stdlib.h>
#include <string.h>

#include "fa.h"
#include "fa_internal.hpp"

namespace {

constexpr int kDecodePage = 16;
constexpr int kDecodeD = 128;

// The bf16 forward kernels address one head's K or V rows with 32-bit byte offsets and keep
// offsets at or above 2^31 (and, block-sparse, at 2^30) as "past the range" markers, so a
// head's rows may span at most 2^30 bytes: N d <= 2^29 (4M tokens at d = 128).
bool head_fits(long long N, long long d) { return N * d * 2 <= (1LL << 30); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool scale_ok(float s) { return isfinite(s) && s > 0.f; }

struct DecodePlan {
    int splits;        // chunks actually launched for the longest sequence
    int chunk_pages;   // pages per chunk
    int len_cap;       // lengths are clamped to this
    int bound;         // upper bound of `splits` over every Hkv >= 1 and shorter tables
};

// Chunks for the longest sequence: about two workgroups per CU of the device (one round of
// 4-wave chunks), since with few (sequence, KV head) pairs most CUs would otherwise idle;
// never more chunks than pages. A fixed plan keeps results deterministic.
DecodePlan plan_decode(int B, int Hkv, int max_pages_per_seq, int max_seq_len, int num_splits) {
    const long long target_wgs = 2LL * fa::device_cus();
    DecodePlan p;
    const long long cap = (long long)max_pages_per_seq * kDecodePage;
    p.len_cap = (int)(max_seq_len < cap ? max_seq_len : cap);
    const int pages = (p.len_cap + kDecodePage - 1) / kDecodePage;
    int s;
    if (num_splits > 0) {
        s = num_splits;
    } else {
        const long long units = (long long)B * Hkv;
        s = units > 0 ? (int)((target_wgs + units - 1) / units) : 1;
    }
    if (s > pages) s = pages;
    if (s < 1) s = 1;
    p.bound = s;
    p.chunk_pages = pages > 0 ? (pages + s - 1) / s : 1;
    p.splits = pages > 0 ? (pages + p.chunk_pages - 1) / p.chunk_pages : 1;
    return p;
}

// Workspace: completion words (one 8-byte word per query head, enough for every KV head),
// then the partials O [S][B*Hq][d], m [S][B*Hq] and l [S][B*Hq], all float32.
size_t decode_done_bytes(int B, int Hq) { return (size_t)B * (size_t)Hq * 8; }
size_t decode_ws_bytes(int B, int Hq, int d, int splits) {
    return decode_done_bytes(B, Hq) +
           (size_t)splits * (size_t)B * (size_t)Hq * ((size_t)d + 2) * sizeof(float);
}
fa::DecodeWorkspace decode_ws_layout(void* ws, int B, int Hq, int d, int splits) {
    fa::DecodeWorkspace w;
    w.done = static_cast<unsigned long long*>(ws);
    w.o = reinterpret_cast<float*>(static_cast<unsigned char*>(ws) + decode_done_bytes(B, Hq));
    w.m = w.o + (size_t)splits * B * Hq * d;
    w.l = w.m + (size_t)splits * B * Hq;
    return w;
}

}  // namespace

namespace fa {
int device_cus() {
    static std::atomic<int> cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kDefaultCUs;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n < 8)
            n = kDefaultCUs;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}
}  // namespace fa

extern "C" {

const char* fa_status_string(fa_status s) {
    switch (s) {
        case FA_OK: return "FA_OK: success";
        case FA_ERR_INVALID_ARGUMENT: return "FA_ERR_INVALID_ARGUMENT: invalid argument";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: no kernel for this request";
        case FA_ERR_WORKSPACE_TOO_SMALL: return "FA_ERR_WORKSPACE_TOO_SMALL: workspace too small";
        case FA_ERR_HIP: return "FA_ERR_HIP: HIP runtime error at launch";
    }
    return "unknown fa_status";
}

fa_status fa_fwd(fa_dtype dt, const void* q, const void* k, const void* v, void* o,
                 float* m_out, float* l_out, int B, int Hq, int Hkv, int N, int d, float scale,
                 int causal, void* stream) {
    if (dt != FA_F32 && dt != FA_BF16) return dt == FA_E4M3 ? FA_ERR_UNSUPPORTED : FA_ERR_INVALID_ARGUMENT;
    if (B < 0 || Hq < 0 || Hkv < 0 || N < 0) return FA_ERR_INVALID_ARGUMENT;
    if (!scale_ok(scale)) return FA_ERR_INVALID_ARGUMENT;
    if (Hq > 0 && (Hkv < 1 || Hq % Hkv != 0)) return FA_ERR_INVALID_ARGUMENT;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (B == 0 || Hq == 0 || N == 0) return FA_OK;
    if (!q || !k || !v || !o) return FA_ERR_INVALID_ARGUMENT;
    if ((long long)N * d >= (1LL << 31)) return FA_ERR_UNSUPPORTED;
    if (dt == FA_BF16 && !head_fits(N, d)) return FA_ERR_UNSUPPORTED;
    const long long rows_per_wg = dt == FA_BF16 ? 256 : 64;
    if (((long long)N + rows_per_wg - 1) / rows_per_wg * B * Hq >= (1LL << 31))
        return FA_ERR_UNSUPPORTED;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (dt == FA_BF16) {
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
            return FA_ERR_INVALID_ARGUMENT;
        e = fa::launch_fwd_bf16_sp(q, k, v, o, m_out, l_out, B, Hq, Hkv, N, d, scale,
                                   causal ? 1 : 0, st);
    } else {
        e = fa::launch_fwd_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                               static_cast<const float*>(v), static_cast<float*>(o), m_out, l_out,
                               B, Hq, Hkv, N, d, scale, causal ? 1 : 0, st);
    }
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_decode_plan_splits(int B, int Hkv, int page_size, int max_seq_len) {
    if (B < 0 || Hkv < 1 || page_size != kDecodePage || max_seq_len < 0) return 0;
    const int pages = (max_seq_len + kDecodePage - 1) / kDecodePage;
    return plan_decode(B, Hkv, pages, max_seq_len, 0).splits;
}

size_t fa_decode_workspace_bytes(int B, int Hq, int d, int page_size, int max_seq_len,
                                 int num_splits) {
    if (B < 0 || Hq < 1 || d < 1 || page_size != kDecodePage || max_seq_len < 0 || num_splits < 0)
        return 0;
    // The split count falls as B * Hkv or the table width grows, and the launched count never
    // exceeds the pre-rounding count, so planning with Hkv = 1 and a table wide enough for
    // max_seq_len bounds the splits of every valid call with these sizes.
    const int pages = (max_seq_len + kDecodePage - 1) / kDecodePage;
    const DecodePlan p = plan_decode(B, 1, pages, max_seq_len, num_splits);
    return decode_ws_bytes(B, Hq, d, p.bound);
}

// Checks shared by both decode entry points (everything but the workspace).
static fa_status decode_check(fa_dtype dt, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_table, const int32_t* seq_lens, void* o, int B, int Hq,
                       int Hkv, int d, int page_size, int num_pages, int max_pages_per_seq,
                       int max_seq_len, float scale, int num_splits) {
    if (dt != FA_F32 && dt != FA_BF16) return FA_ERR_INVALID_ARGUMENT;
    if (B < 0 || Hq < 1 || Hkv < 1 || d < 1 || page_size < 1 || num_pages < 0 ||
        max_pages_per_seq < 0 || max_seq_len < 0 || num_splits < 0)
        return FA_ERR_INVALID_ARGUMENT;
    if (Hq % Hkv != 0) return FA_ERR_INVALID_ARGUMENT;
    if (!scale_ok(scale)) return FA_ERR_INVALID_ARGUMENT;
    const int G = Hq / Hkv;
    if (dt != FA_BF16 || d != kDecodeD || page_size != kDecodePage ||
        (G != 1 && G != 2 && G != 4 && G != 8))
        return FA_ERR_UNSUPPORTED;
    if (B == 0) return FA_OK;
    if (!q || !o || !block_table || !seq_lens) return FA_ERR_INVALID_ARGUMENT;
    if (num_pages > 0 && (!k_cache || !v_cache)) return FA_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
        return FA_ERR_INVALID_ARGUMENT;
    if ((long long)B * Hkv >= (1LL << 31)) return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

fa_status fa_decode_splitk(fa_dtype dt, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_table, const int32_t* seq_lens, void* o, int B,
                           int Hq, int Hkv, int d, int page_size, int num_pages,
                           int max_pages_per_seq, int max_seq_len, float scale, int num_splits,
                           void* workspace, size_t workspace_bytes, void* stream) {
    const fa_status st = decode_check(dt, q, k_cache, v_cache, block_table, seq_lens, o, B, Hq,
                                      Hkv, d, page_size, num_pages, max_pages_per_seq,
                                      max_seq_len, scale, num_splits);
    if (st != FA_OK || B == 0) return st;
    if (!workspace) return FA_ERR_INVALID_ARGUMENT;
    if (!aligned16(workspace)) return FA_ERR_INVALID_ARGUMENT;
    const DecodePlan p = plan_decode(B, Hkv, max_pages_per_seq, max_seq_len, num_splits);
    if (p.splits > 65535) return FA_ERR_UNSUPPORTED;  // grid y holds the chunk
    const size_t need = decode_ws_bytes(B, Hq, d, p.splits);
    if (workspace_bytes < need) return FA_ERR_WORKSPACE_TOO_SMALL;
    const hipError_t e = fa::launch_decode_bf16_mx(
        q, k_cache, v_cache, block_table, seq_lens, o, B, Hq, Hkv, d, num_pages, max_pages_per_seq,
        p.len_cap, scale, p.splits, p.chunk_pages, decode_ws_layout(workspace, B, Hq, d, p.splits),
        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_decode_noalloc_max_bytes(void) { return fa::decode_scratch_bytes(); }

fa_status fa_decode_splitk_noalloc(fa_dtype dt, const void* q, const void* k_cache,
                                   const void* v_cache, const int32_t* block_table,
                                   const int32_t* seq_lens, void* o, int B, int Hq, int Hkv, int d,
                                   int page_size, int num_pages, int max_pages_per_seq,
                                   int max_seq_len, float scale, int num_splits, void* stream) {
    const fa_status st = decode_check(dt, q, k_cache, v_cache, block_table, seq_lens, o, B, Hq,
                                      Hkv, d, page_size, num_pages, max_pages_per_seq,
                                      max_seq_len, scale, num_splits);
    if (st != FA_OK || B == 0) return st;
    const DecodePlan p = plan_decode(B, Hkv, max_pages_per_seq, max_seq_len, num_splits);
    if (p.splits > 65535) return FA_ERR_UNSUPPORTED;  // grid y holds the chunk
    if (decode_ws_bytes(B, Hq, d, p.splits) > fa::decode_scratch_bytes())
        return FA_ERR_WORKSPACE_TOO_SMALL;
    void* scratch = nullptr;  // this device's copy of the library's static scratch
    if (fa::decode_scratch(&scratch) != hipSuccess) return FA_ERR_HIP;
    const hipError_t e = fa::launch_decode_bf16_mx(
        q, k_cache, v_cache, block_table, seq_lens, o, B, Hq, Hkv, d, num_pages, max_pages_per_seq,
        p.len_cap, scale, p.splits, p.chunk_pages, decode_ws_layout(scratch, B, Hq, d, p.splits),
        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_fwd_fp8(fa_dtype v_dt, const void* q, const void* k, const void* v, void* o,
                     float* m_out, float* l_out, int B, int Hq, int Hkv, int N, int d, float scale,
                     int causal, void* stream) {
    if (v_dt != FA_BF16 && v_dt != FA_E4M3) return FA_ERR_INVALID_ARGUMENT;
    if (B < 0 || Hq < 0 || Hkv < 0 || N < 0) return FA_ERR_INVALID_ARGUMENT;
    if (!scale_ok(scale)) return FA_ERR_INVALID_ARGUMENT;
    if (Hq > 0 && (Hkv < 1 || Hq % Hkv != 0)) return FA_ERR_INVALID_ARGUMENT;
    if (d != 128) return FA_ERR_UNSUPPORTED;
    if (B == 0 || Hq == 0 || N == 0) return FA_OK;
    if (!q || !k || !v || !o) return FA_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return FA_ERR_INVALID_ARGUMENT;
    if (!head_fits(N, d)) return FA_ERR_UNSUPPORTED;
    if (((long long)N + 255) / 256 * B * Hq >= (1LL << 31)) return FA_ERR_UNSUPPORTED;
    const hipError_t e = fa::launch_fwd_fp8qk_sp(q, k, v, v_dt == FA_E4M3 ? 1 : 0, o, m_out, l_out,
                                                 B, Hq, Hkv, N, d, scale, causal ? 1 : 0,
                                                 static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_workspace_bytes(int B, int Hq, int N) {
    if (B < 0 || Hq < 0 || N < 0) return 0;
    return fa::bwd_ld_bytes(B, Hq, N);
}

fa_status fa_bwd(fa_dtype dt, const void* q, const void* k, const void* v, const void* o,
                 const void* dout, const float* m, const float* l, void* dq, void* dk, void* dv,
                 int B, int Hq, int Hkv, int N, int d, float scale, int causal, void* workspace,
                 size_t workspace_bytes, void* stream) {
    if (dt != FA_F32 && dt != FA_BF16) return FA_ERR_INVALID_ARGUMENT;
    if (B < 0 || Hq < 0 || Hkv < 0 || N < 0) return FA_ERR_INVALID_ARGUMENT;
    if (!scale_ok(scale)) return FA_ERR_INVALID_ARGUMENT;
    if (Hq > 0 && (Hkv < 1 || Hq % Hkv != 0)) return FA_ERR_INVALID_ARGUMENT;
    if (dt != FA_BF16 || (d != 64 && d != 128)) return FA_ERR_UNSUPPORTED;
    if (B == 0 || Hq == 0 || N == 0) return FA_OK;
    if (!q || !k || !v || !o || !dout || !m || !l || !dq || !dk || !dv || !workspace)
        return FA_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
        !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace))
        return FA_ERR_INVALID_ARGUMENT;
    // a head's rows (N d bf16 values) are addressed with 32-bit signed byte counts
    if ((long long)N * d * 2 >= (1LL << 31)) return FA_ERR_UNSUPPORTED;
    if ((long long)B * Hq >= 65536 || ((long long)N + 127) / 128 >= (1LL << 31))
        return FA_ERR_UNSUPPORTED;  // grid y holds (batch, head)
    if (workspace_bytes < fa_bwd_workspace_bytes(B, Hq, N)) return FA_ERR_WORKSPACE_TOO_SMALL;
    const hipError_t e = fa::launch_bwd_bf16(q, k, v, o, dout, m, l, dq, dk, dv, B, Hq, Hkv, N, d,
                                             scale, causal ? 1 : 0, static_cast<float*>(workspace),
                                             static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_fwd_block_sparse(fa_dtype dt, const void* q, const void* k, const void* v, void* o,
                              float* m_out, float* l_out, const int32_t* block_offsets,
                              const int32_t* block_indices, int nnz, int B, int Hq, int Hkv,
                              int N, int d, float scale, int causal, void* stream) {
    if (dt != FA_F32 && dt != FA_BF16) return FA_ERR_INVALID_ARGUMENT;
    if (B < 0 || Hq < 0 || Hkv < 0 || N < 0 || nnz < 0) return FA_ERR_INVALID_ARGUMENT;
    if (!scale_ok(scale)) return FA_ERR_INVALID_ARGUMENT;
    if (Hq > 0 && (Hkv < 1 || Hq % Hkv != 0)) return FA_ERR_INVALID_ARGUMENT;
    if (dt != FA_BF16 || (d != 64 && d != 128)) return FA_ERR_UNSUPPORTED;
    if (B == 0 || Hq == 0 || N == 0) return FA_OK;
    if (!q || !k || !v || !o || !block_offsets || (nnz > 0 && !block_indices))
        return FA_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return FA_ERR_INVALID_ARGUMENT;
    if (!head_fits(N, d)) return FA_ERR_UNSUPPORTED;
    if (((long long)N + 255) / 256 * B * Hq >= (1LL << 31)) return FA_ERR_UNSUPPORTED;
    const hipError_t e = fa::launch_fwd_bf16_sp_block_sparse(
        q, k, v, o, m_out, l_out, block_offsets, block_indices, nnz, B, Hq, Hkv, N, d, scale,
        causal ? 1 : 0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_fwd_paged(fa_dtype dt, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_table, const int32_t* seq_lens,
                       const int32_t* q_lens, void* o,
                       float* m_out, float* l_out, int B, int Hq, int Hkv, int Nq, int d,
                       int page_size, int num_pages, int max_pages_per_seq, float scale,
                       int causal, void* stream) {
    if (dt != FA_F32 && dt != FA_BF16) return FA_ERR_INVALID_ARGUMENT;
    if (B < 0 || Hq < 0 || Hkv < 0 || Nq < 0 || num_pages < 0 || max_pages_per_seq < 0 ||
        page_size < 1)
        return FA_ERR_INVALID_ARGUMENT;
    if (!scale_ok(scale)) return FA_ERR_INVALID_ARGUMENT;
    if (Hq > 0 && (Hkv < 1 || Hq % Hkv != 0)) return FA_ERR_INVALID_ARGUMENT;
    if (dt != FA_BF16 || (d != 64 && d != 128) || page_size != kDecodePage) return FA_ERR_UNSUPPORTED;
    if (B == 0 || Hq == 0 || Nq == 0) return FA_OK;
    if (!q || !o || !block_table || !seq_lens) return FA_ERR_INVALID_ARGUMENT;
    if (num_pages > 0 && (!k_cache || !v_cache)) return FA_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
        return FA_ERR_INVALID_ARGUMENT;
    if (!head_fits(Nq, d)) return FA_ERR_UNSUPPORTED;
    if (((long long)Nq + 255) / 256 * B * Hq >= (1LL << 31)) return FA_ERR_UNSUPPORTED;
    if ((long long)max_pages_per_seq * page_size >= (1LL << 31)) return FA_ERR_UNSUPPORTED;
    // the kernel addresses each cache with 32-bit byte offsets below 2^31
    if ((long long)num_pages * Hkv * page_size * d * 2 >= (1LL << 31)) return FA_ERR_UNSUPPORTED;
    const hipError_t e = fa::launch_fwd_bf16_sp_paged(
        q, k_cache, v_cache, block_table, seq_lens, q_lens, o, m_out, l_out, B, Hq, Hkv, Nq, d, num_pages,
        max_pages_per_seq, scale, causal ? 1 : 0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_merge(fa_dtype out_dt, const float* o_parts, const float* m_parts,
                   const float* l_parts, void* o, float* m_out, float* l_out, int S, int R, int d,
                   void* stream) {
    if (out_dt != FA_F32 && out_dt != FA_BF16) return FA_ERR_INVALID_ARGUMENT;
    if (S < 1 || R < 0 || d < 1) return FA_ERR_INVALID_ARGUMENT;
    if (d > 1024) return FA_ERR_UNSUPPORTED;
    if (R == 0) return FA_OK;
    if (!o_parts || !m_parts || !l_parts || !o) return FA_ERR_INVALID_ARGUMENT;
    if ((long long)S * R * d >= (1LL << 40)) return FA_ERR_UNSUPPORTED;
    const hipError_t e = fa::launch_merge(o_parts, m_parts, l_parts, o, out_dt == FA_BF16 ? 1 : 0,
                                          m_out, l_out, S, R, d, 0,
                                          static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
