// decode_mx.hip - single-query attention over a paged KV cache, split across the KV sequence,
// with both products on the matrix cores.
//
// Method: "FlashAttention" (shubhamtatvamasi.com), "Decode is a different problem": with one
// query row per sequence there is no reuse on the query side and only batch x KV-head units
// of parallelism, so the KV sequence is split into chunks processed by separate workgroups;
// each chunk yields a partial (m, l, O) that is merged afterwards with the online-softmax
// rule. The cache is read through a block table (the paged variants of the family table on
// the same page, and its PagedAttention answer).
//
// CDNA4 design. The kernel is bound by HBM bandwidth; the point of the matrix cores here is
// to make the per-page work small, so that a wave gets back to issuing loads quickly:
//  * grid = (sequence x KV head, chunk); 4 waves per workgroup; wave w takes pages w, w+4,
//    ... of its chunk. The G <= 16 query heads that share a KV head form the 16 columns of
//    the matrix products (zero-padded past G), so each byte of the cache is read once per
//    KV head.
//  * A page of one KV head (16 tokens x 128 dims of K, and of V: 4 KiB each) goes from HBM
//    straight into LDS (buffer loads with the LDS bit), one page ahead of its use, into two
//    slots private to the wave: no workgroup barrier in the page loop.
//  * S^T (16 tokens x 16 queries) = K Q^T: four v_mfma_f32_16x16x32_bf16 with K from LDS.
//    The accumulator gives lane l the scores of query l % 16 for tokens 4 (l / 16) .. +3,
//    which, rounded to bf16, is exactly the A operand of O += P V with
//    v_mfma_f32_16x16x16_bf16 (eight MFMAs, one per 16 head dimensions); V's operand comes
//    out of row-major V through ds_read_b64_tr_b16.
//  * LDS reads are conflict free: the loads store each page's 16-byte chunks permuted by an
//    XOR with the token index (K) or twice its low three bits (V), and the reads undo it.
//  * Tokens past the sequence end get a score of -inf and a V operand of 0 (the cache slots
//    behind them may hold anything).
//  * Softmax per query: one exchange with lanes l ^ 16 and l ^ 32 gives the page maximum; the
//    exponent reference moves only when it is beaten by more than 2^8 (then O is rescaled).
//  * At the end the waves' states are merged through LDS and one normalised float32 partial
//    (m in log2 units, l, O) per (chunk, query head) is written to the workspace; the merge
//    kernel (merge.hip) combines the chunks.
#include <stdio.h>
#include <stdlib.h>

#include "fa_internal.hpp"
#include "gfx950.hpp"

namespace fa {
namespace {

constexpr int kD = 128;
constexpr int kPage = 16;
constexpr int kQ = 16;                          // query columns of the products
constexpr int kPiece = kPage * kD * 2;          // bytes of K (or V) of one page and KV head
constexpr int kSlot = 2 * kPiece;               // K then V
constexpr int kLoadsPerPage = 2 * kPiece / 1024;  // 1 KiB per load instruction
constexpr float kTau = 8.f;                     // lazy-rescale threshold, log2 units
constexpr int kBufferDword3 = 0x00020000;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef const __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef const __attribute__((address_space(3))) unsigned char* lds_cptr;

__device__ __forceinline__ float xlane_max(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float xlane_sum(float x) {
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}

// W waves per workgroup, S page slots per wave (S - 1 pages in flight while one is consumed).
template <int W, int S>
__global__ __launch_bounds__(64 * W) void decode_mx_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ table,
    const int32_t* __restrict__ lens, float* __restrict__ ws_o, float* __restrict__ ws_m,
    float* __restrict__ ws_l, int Hq, int Hkv, int G, int num_pages, int max_pages,
    int len_cap, float scale_log2, int chunk_pages) {
    constexpr int kWaves = W, kSlots = S, kThreads = 64 * W;
    static_assert(S >= 2 && (S - 1) * kLoadsPerPage <= 63, "vmcnt holds at most 63 loads");
    __shared__ __attribute__((aligned(16))) unsigned char smem[kWaves * kSlots * kSlot];
    lds_cptr const lds = (lds_cptr)smem;
    const unsigned lds_addr = (unsigned)(size_t)lds;

    // x = sequence x KV head (KV head fastest: the KV heads of one page sit next to each
    // other in memory and are streamed side by side), y = chunk
    const int split = blockIdx.y;
    const int bk = blockIdx.x;
    const int b = bk / Hkv;
    const int kvh = bk - b * Hkv;
    const int R = gridDim.x / Hkv * Hq;  // B * Hq
    const int row0 = b * Hq + kvh * G;

    int L = lens[b];
    L = L < 0 ? 0 : (L > len_cap ? len_cap : L);
    const int npages = (L + kPage - 1) / kPage;
    // This sequence gets ceil(npages / chunk_pages) chunks of near-equal size (they differ by
    // at most one page); splits past the sequence's chunk count are empty.
    const int n_chunks = (npages + chunk_pages - 1) / chunk_pages;
    const int p_begin = split < n_chunks ? (int)((long long)split * npages / n_chunks) : npages;
    const int p_end = split < n_chunks ? (int)((long long)(split + 1) * npages / n_chunks) : npages;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
    const int lane = tid & 63;
    const int l16 = lane & 15;  // query column (S^T, P) / head dimension in a block (O)
    const int g4 = lane >> 4;   // token group: tokens 4 g4 .. 4 g4 + 3

    f32x4 acc[kD / 16];  // O: lane holds queries 4 g4 + r, dims 16 blk + l16
#pragma unroll
    for (int i = 0; i < kD / 16; ++i) acc[i] = f32x4{};
    float m_ref = -INFINITY;  // exponent reference of query l16 (equal in its four lanes)
    float lsum = 0.f;         // this lane's part of query l16's sum

    const int n_mine = p_end - p_begin > wave ? (p_end - p_begin - wave + kWaves - 1) / kWaves : 0;
    if (n_mine > 0 && num_pages > 0) {
        // Q as the B operand of S^T = K Q^T: lane l holds query l16 (zero past G), dims
        // 32 m + 8 g4 .. +7.
        bf16x8 qb[kD / 32];
#pragma unroll
        for (int m = 0; m < kD / 32; ++m) {
            qb[m] = bf16x8{};
            if (l16 < G)
                qb[m] = *reinterpret_cast<const bf16x8*>(q + (size_t)(row0 + l16) * kD + 32 * m + 8 * g4);
        }
#pragma unroll
        for (int m = 0; m < kD / 32; ++m) asm volatile("" : "+v"(qb[m]));

        // LDS read offsets within a slot. K (A operand of the S^T MFMA): token l16, 16 bytes
        // of chunk 4 m + g4, stored at chunk (4 m + g4) ^ l16. V (B operand of the O MFMA,
        // ds_read_b64_tr_b16): source lane (q4, e) of group g4 reads token t = 4 g4 + e, 8
        // bytes of dims 16 blk + 4 q4 (chunk 2 blk + q4 / 2), stored at chunk ^ 2 (t & 7).
        int koff[kD / 32], voff[kD / 16];
#pragma unroll
        for (int m = 0; m < kD / 32; ++m) koff[m] = l16 * 256 + 16 * ((4 * m + g4) ^ l16);
        {
            const int q4 = lane & 3, t = 4 * g4 + ((lane & 15) >> 2);
#pragma unroll
            for (int blk = 0; blk < kD / 16; ++blk)
                voff[blk] = kPiece + t * 256 + 16 * ((2 * blk + (q4 >> 1)) ^ (2 * (t & 7))) + 8 * (q4 & 1);
        }
        // Load sources: load c of a piece fills slot bytes 1024 c + 16 lane: token
        // t = 4 c + lane / 16, stored chunk s = lane % 16, holding the piece's chunk s ^ t (K)
        // or s ^ 2 (t & 7) (V).
        int ksrc[kPiece / 1024], vsrc[kPiece / 1024];
#pragma unroll
        for (int c = 0; c < kPiece / 1024; ++c) {
            const int t = 4 * c + (lane >> 4), s = lane & 15;
            ksrc[c] = t * 256 + 16 * (s ^ t);
            vsrc[c] = t * 256 + 16 * (s ^ (2 * (t & 7)));
        }

        const size_t page_stride = (size_t)Hkv * kPage * kD;  // elements per physical page
        const int32_t* trow = table + (size_t)b * max_pages;
        const unsigned wave_lds = lds_addr + wave * kSlots * kSlot;
        // Block-table entries of this wave's pages, 64 at a time, read back with v_readlane
        // (scalar page bases). `ent` covers pages [w0, w0 + 64) of the wave's list.
        int w0 = 0;
        int ent = lane < n_mine ? trow[p_begin + wave + kWaves * lane] : -1;

        // Loads of the wave's page i into slot s: K and V of one KV head, 4 KiB each. Past the
        // wave's last page, or for an entry outside [0, num_pages), the descriptors have no
        // range: nothing is fetched and the slot fills with zeros (never read). Every call
        // issues the same kLoadsPerPage loads, so one vmcnt count waits for a page.
        auto issue = [&](int i, int s) {
            int phys = -1;
            if (i < n_mine) {
                if (i >= w0 + 64) {  // next 64 entries (once per 64 pages)
                    w0 += 64;
                    const int li = w0 + lane;
                    ent = li < n_mine ? trow[p_begin + wave + kWaves * li] : -1;
                }
                phys = __builtin_amdgcn_readlane(ent, i - w0);
            }
            const bool ok = phys >= 0 && phys < num_pages;
            const size_t off = ((size_t)(ok ? phys : 0) * page_stride + (size_t)kvh * kPage * kD);
            const int bytes = __builtin_amdgcn_readfirstlane(ok ? kPiece : 0);
            const __amdgpu_buffer_rsrc_t rk =
                __builtin_amdgcn_make_buffer_rsrc((void*)(kc + off), (short)0, bytes, kBufferDword3);
            const __amdgpu_buffer_rsrc_t rv =
                __builtin_amdgcn_make_buffer_rsrc((void*)(vc + off), (short)0, bytes, kBufferDword3);
            const unsigned dst = wave_lds + s * kSlot;
#pragma unroll
            for (int c = 0; c < kPiece / 1024; ++c)
                asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                             :
                             : "v"(ksrc[c]), "s"(rk), "{m0}"(dst + 1024 * c)
                             : "memory");
#pragma unroll
            for (int c = 0; c < kPiece / 1024; ++c)
                asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                             :
                             : "v"(vsrc[c]), "s"(rv), "{m0}"(dst + kPiece + 1024 * c)
                             : "memory");
            return phys;
        };

        // Consumes the wave's page i from slot s (physical page phys).
        auto process = [&](int i, int s, int phys) {
            const lds_cptr sl = lds + wave * kSlots * kSlot + s * kSlot;
            f32x4 sc = f32x4{};
#pragma unroll
            for (int m = 0; m < kD / 32; ++m)
                sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    *reinterpret_cast<const lds_bf16x8*>(sl + koff[m]), qb[m], sc, 0, 0, 0);
            // sc[r]: query l16, token 4 g4 + r of the page
            const int pidx = p_begin + wave + kWaves * i;
            const bool page_ok = phys >= 0 && phys < num_pages;
            const bool tail = !page_ok || (pidx + 1) * kPage > L;  // wave-uniform
            float x[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) x[r] = sc[r] * scale_log2;
            if (tail) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (!page_ok || pidx * kPage + 4 * g4 + r >= L) x[r] = -INFINITY;
            }
            const float mx = xlane_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
            if (__any(mx > m_ref + kTau)) {
                // move the reference of the queries that need it; O rows are held by other
                // lanes (query 4 g4 + r), so the factors are fetched from lanes 4 g4 + r
                const float m_new = mx > m_ref + kTau ? mx : m_ref;
                const float alpha = m_ref == -INFINITY ? 0.f : exp2_hw(m_ref - m_new);
                lsum *= alpha;
                m_ref = m_new;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float a = __shfl(alpha, 4 * g4 + r);
#pragma unroll
                    for (int blk = 0; blk < kD / 16; ++blk) acc[blk][r] *= a;
                }
            }
            float p[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) p[r] = m_ref == -INFINITY ? 0.f : exp2_hw(x[r] - m_ref);
            lsum += (p[0] + p[1]) + (p[2] + p[3]);
            const v4i16 pa = __builtin_bit_cast(v4i16, u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])});
            // V rows of tokens past the sequence end may hold anything (0 x NaN is NaN in the
            // product): on a tail page they are zeroed in the operand (element e of a lane's
            // V operand is token 4 g4 + e).
            bool vok[4] = {true, true, true, true};
            if (tail) {
#pragma unroll
                for (int e = 0; e < 4; ++e) vok[e] = page_ok && pidx * kPage + 4 * g4 + e < L;
            }
#pragma unroll
            for (int blk = 0; blk < kD / 16; ++blk) {
                v4i16 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(sl + voff[blk]));
                if (tail) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) vb[e] = vok[e] ? vb[e] : (short)0;
                }
                acc[blk] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, acc[blk], 0, 0, 0);
            }
        };

        // LDS loads are not tracked by the compiler's waits: wait for all but the newest
        // S - 1 pages' loads (vmcnt counts this wave's vector loads in issue order).
        auto wait_older = [&]() {
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kSlots - 1) * kLoadsPerPage) : "memory");
        };
        // Page i sits in slot i % S; page i + S - 1 is requested just before page i is
        // consumed. The loop is unrolled over the slots so every slot index is a constant.
        int ph[kSlots];
#pragma unroll
        for (int s = 0; s + 1 < kSlots; ++s) ph[s] = issue(s, s);
        int i = 0;
        for (bool more = true; more;) {
#pragma unroll
            for (int s = 0; s < kSlots; ++s) {
                if (more) {
                    const int sn = (s + kSlots - 1) % kSlots;
                    ph[sn] = issue(i + kSlots - 1, sn);
                    wait_older();
                    process(i, s, ph[s]);
                    more = ++i < n_mine;
                }
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the extra page's loads
    }
    __syncthreads();  // the slots are reused below

    // ---- merge the waves (lanes of a query: l16 = g, all g4) and write this chunk's
    // normalised partial ----
    float* sm_o = reinterpret_cast<float*>(smem);          // [wave][query][kD]
    float* sm_m = sm_o + kWaves * kQ * kD;                  // [wave][query]
    float* sm_l = sm_m + kWaves * kQ;
    const float lw = xlane_sum(lsum);
    if (g4 == 0 && l16 < G) {
        sm_m[wave * kQ + l16] = m_ref;
        sm_l[wave * kQ + l16] = lw;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int g = 4 * g4 + r;
        if (g < G) {
#pragma unroll
            for (int blk = 0; blk < kD / 16; ++blk)
                sm_o[(wave * kQ + g) * kD + 16 * blk + l16] = acc[blk][r];
        }
    }
    __syncthreads();
    for (int idx = tid; idx < G * kD; idx += kThreads) {
        const int g = idx / kD;
        const int d = idx - g * kD;
        float m = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
            if (sm_l[w * kQ + g] > 0.f) m = fmaxf(m, sm_m[w * kQ + g]);
        float lt = 0.f, ot = 0.f;
        if (m != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                // sm_o and sm_l are unnormalised sums relative to the wave's own reference
                const float ls = sm_l[w * kQ + g];
                const float rs = ls > 0.f ? exp2_hw(sm_m[w * kQ + g] - m) : 0.f;
                lt = __builtin_fmaf(rs, ls, lt);
                ot = __builtin_fmaf(rs, sm_o[(w * kQ + g) * kD + d], ot);
            }
        }
        const size_t prow = (size_t)split * R + row0 + g;
        ws_o[prow * kD + d] = lt > 0.f ? ot / lt : 0.f;
        if (d == 0) {
            ws_m[prow] = lt > 0.f ? m : -INFINITY;
            ws_l[prow] = lt;
        }
    }
}

}  // namespace

hipError_t launch_decode_bf16_mx(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_table, const int32_t* seq_lens, void* o,
                                 int B, int Hq, int Hkv, int d, int num_pages,
                                 int max_pages_per_seq, int len_cap, float scale, int splits,
                                 int chunk_pages, float* ws_o, float* ws_m, float* ws_l,
                                 hipStream_t stream) {
    (void)d;
    const dim3 grid((unsigned)(B * Hkv), (unsigned)splits);
    int W = 4, S = 2;
    if (const char* e = getenv("FA_DECODE_MX")) sscanf(e, "%d,%d", &W, &S);
#define FA_MX_CASE(w, s)                                                                         \
    if (W == w && S == s) {                                                                      \
        hipLaunchKernelGGL((decode_mx_kernel<w, s>), grid, dim3(64 * w), 0, stream,              \
                           static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache), \
                           static_cast<const uint16_t*>(v_cache), block_table, seq_lens, ws_o,   \
                           ws_m, ws_l, Hq, Hkv, Hq / Hkv, num_pages, max_pages_per_seq, len_cap, \
                           scale * kLog2e, chunk_pages);                                         \
    } else
    FA_MX_CASE(2, 3) FA_MX_CASE(2, 4) FA_MX_CASE(3, 3) FA_MX_CASE(3, 4) FA_MX_CASE(4, 3)
    FA_MX_CASE(4, 4) FA_MX_CASE(5, 4) FA_MX_CASE(6, 3) FA_MX_CASE(8, 2) FA_MX_CASE(4, 2)
    return hipErrorInvalidValue;
#undef FA_MX_CASE
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_merge(ws_o, ws_m, ws_l, o, 1, nullptr, nullptr, splits, B * Hq, kD, 1, stream);
}

}  // namespace fa
