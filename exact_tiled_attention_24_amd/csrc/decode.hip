// decode.hip - single-query attention over a paged KV cache, split across the KV sequence.
//
// Method: "FlashAttention" (shubhamtatvamasi.com), "Decode is a different problem": with one
// query row per sequence there is no reuse on the query side and only batch x KV-head
// units of parallelism, so the KV sequence is split into chunks processed by separate
// workgroups; each chunk yields a partial (m, l, O) that is merged afterwards with the
// online-softmax rule. The cache is read through a block table (the paged variants of the
// family table on the same page, and its PagedAttention answer).
//
// CDNA4 design. The kernel is bound by HBM bandwidth (about 4 FLOP per byte of K/V), so it
// is built around memory-level parallelism rather than the matrix cores:
//  * grid = (sequence x KV head, chunk); one workgroup of 4 waves per chunk; wave w takes
//    pages w, w+4, ... of its chunk. The G query heads that share a KV head are served by
//    the same pass over the K/V bytes (each byte of the cache is read once per KV head).
//  * lane l owns token slot l/8 of each 8-token half page and the 16 head dimensions
//    16*(l%8) .. +15, so a page is four 16-byte loads of K and four of V per lane, and
//    every load instruction covers contiguous 2 KiB halves of the page.
//  * the block-table entries of a wave's pages are fetched once into a VGPR and read back
//    with v_readlane, so every page address is a scalar; the next page is prefetched into
//    registers while the current one is consumed.
//  * q.k partial dot products use v_dot2_f32_bf16 and are summed over the 8 lanes of a token
//    with three DPP steps. Each lane keeps its own running (m, l, O) for its token slot with
//    a lazily moved reference maximum: the accumulator is rescaled only when a score exceeds
//    the reference by more than 2^8, which is exact up to rounding because the final
//    division by l cancels the reference.
//  * at the end the lanes' states are merged across token slots, then across waves through
//    LDS, and one normalised float32 partial (m in log2 units, l, O) per (chunk, query head)
//    is written to the workspace. A second kernel merges the chunks (merge.hip).
#include "fa_internal.hpp"
#include "gfx950.hpp"

namespace fa {
namespace {

constexpr int kD = 128;
constexpr int kPage = 16;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kTau = 8.f;  // lazy-rescale threshold, log2 units

__device__ __forceinline__ float dpp_sum8(float x) {
    // all-reduce over the 8 consecutive lanes of a half row
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xf, 0xf, false));
    return x;
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
}

struct PageRegs {
    u32x4 k[4];  // [half page][2 x 16 bytes]
    u32x4 v[4];
};

template <int G>
__global__ __launch_bounds__(kThreads) void decode_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ table,
    const int32_t* __restrict__ lens, float* __restrict__ ws_o, float* __restrict__ ws_m,
    float* __restrict__ ws_l, int Hq, int Hkv, int num_pages, int max_pages, int len_cap,
    float scale_log2, int chunk_pages) {
    __shared__ float sm_o[kWaves][G][kD];
    __shared__ float sm_m[kWaves][G];
    __shared__ float sm_l[kWaves][G];

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
    // at most one page), so the workgroups of one launch carry balanced work; splits past
    // the sequence's chunk count are empty.
    const int n_chunks = (npages + chunk_pages - 1) / chunk_pages;
    const int p_begin = split < n_chunks ? (int)((long long)split * npages / n_chunks) : npages;
    const int p_end = split < n_chunks ? (int)((long long)(split + 1) * npages / n_chunks) : npages;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
    const int lane = tid & 63;
    const int t8 = lane >> 3;
    const int qs = lane & 7;

    float acc[G][16];
    float mref[G], lsum[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        mref[g] = -INFINITY;
        lsum[g] = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[g][e] = 0.f;
    }

    if (p_begin < p_end && num_pages > 0) {
        uint32_t qw[G][8];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const u32x4* src =
                reinterpret_cast<const u32x4*>(q + (size_t)(row0 + g) * kD + 16 * qs);
            const u32x4 a = src[0], c = src[1];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                qw[g][w] = a[w];
                qw[g][4 + w] = c[w];
            }
        }
        // Complete the q loads before the page loop (see the note in fwd_bf16.hip).
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int w = 0; w < 8; ++w) asm volatile("" : "+v"(qw[g][w]));

        // pages of this wave: p_begin + wave + 4*i, i < n_mine
        const int n_mine = (p_end - p_begin - wave + kWaves - 1) / kWaves;
        const size_t kv_stride = (size_t)Hkv * kPage * kD;  // elements per physical page
        const size_t head_off = (size_t)kvh * kPage * kD + t8 * kD + 16 * qs;
        const int32_t* trow = table + (size_t)b * max_pages;

        // Loads are issued unconditionally (an invalid table entry reads page 0 and is
        // masked out arithmetically), so every page costs the same 8 loads and the waits
        // before consuming a buffer are exact.
        auto load_page = [&](int phys, PageRegs& r) {
            const bool ok = phys >= 0 && phys < num_pages;
            const size_t base = (size_t)(ok ? phys : 0) * kv_stride + head_off;
            const uint16_t* kp = kc + base;
            const uint16_t* vp = vc + base;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                r.k[2 * half] = *reinterpret_cast<const u32x4*>(kp + half * 8 * kD);
                r.k[2 * half + 1] = *reinterpret_cast<const u32x4*>(kp + half * 8 * kD + 8);
                r.v[2 * half] = *reinterpret_cast<const u32x4*>(vp + half * 8 * kD);
                r.v[2 * half + 1] = *reinterpret_cast<const u32x4*>(vp + half * 8 * kD + 8);
            }
        };
        // Consumes one page. Invalid tokens (past the sequence end, or an invalid table entry)
        // get s = -inf and their V is replaced by 0 at use; the loaded registers are never
        // overwritten, so no wait is needed beyond the page's own loads.
        auto process = [&](const PageRegs& cur, int phys, int i) {
            const int pidx = p_begin + wave + kWaves * i;
            const bool page_ok = phys >= 0 && phys < num_pages;
            const bool tail = !page_ok || (pidx + 1) * kPage > L;  // wave-uniform
            bool valid[2];
#pragma unroll
            for (int half = 0; half < 2; ++half)
                valid[half] = page_ok && pidx * kPage + 8 * half + t8 < L;
            float s[2][G];
#pragma unroll
            for (int half = 0; half < 2; ++half)
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    float d0 = 0.f;
#pragma unroll
                    for (int w = 0; w < 4; ++w) d0 = dot2_bf16(cur.k[2 * half][w], qw[g][w], d0);
#pragma unroll
                    for (int w = 0; w < 4; ++w)
                        d0 = dot2_bf16(cur.k[2 * half + 1][w], qw[g][4 + w], d0);
                    s[half][g] = d0;
                }
#pragma unroll
            for (int half = 0; half < 2; ++half)
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const float t = dpp_sum8(s[half][g]) * scale_log2;
                    s[half][g] = (tail && !valid[half]) ? -INFINITY : t;
                }

            float pr[2][G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float smax = fmaxf(s[0][g], s[1][g]);
                if (smax > mref[g] + kTau) {
                    const float alpha = exp2_hw(mref[g] - smax);
                    lsum[g] *= alpha;
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[g][e] *= alpha;
                    mref[g] = smax;
                }
#pragma unroll
                for (int half = 0; half < 2; ++half)
                    pr[half][g] = (s[half][g] == -INFINITY) ? 0.f : exp2_hw(s[half][g] - mref[g]);
                lsum[g] += pr[0][g] + pr[1][g];
            }

            auto accumulate = [&](bool masked) {
#pragma unroll
                for (int half = 0; half < 2; ++half)
#pragma unroll
                    for (int w = 0; w < 8; ++w) {
                        const uint32_t word = cur.v[2 * half + (w >> 2)][w & 3];
                        float v0 = bf16_lo(word), v1 = bf16_hi(word);
                        if (masked) {
                            v0 = valid[half] ? v0 : 0.f;
                            v1 = valid[half] ? v1 : 0.f;
                        }
#pragma unroll
                        for (int g = 0; g < G; ++g) {
                            acc[g][2 * w] = __builtin_fmaf(pr[half][g], v0, acc[g][2 * w]);
                            acc[g][2 * w + 1] = __builtin_fmaf(pr[half][g], v1, acc[g][2 * w + 1]);
                        }
                    }
            };
            if (tail)
                accumulate(true);
            else
                accumulate(false);
        };

        for (int g0 = 0; g0 < n_mine; g0 += 64) {
            // block-table entries of up to 64 pages, broadcast later with v_readlane
            const int cnt = min_(64, n_mine - g0);
            int entry = lane < cnt ? trow[p_begin + wave + kWaves * (g0 + lane)] : -1;
            asm volatile("" : "+v"(entry));
            // Ping-pong page buffers. Every iteration issues both prefetches (re-reading the
            // current page when there is no next one, an L2 hit), so the number of loads in
            // flight is the same on every path and each buffer is waited for exactly.
            PageRegs ra, rb;
            int pa = __builtin_amdgcn_readlane(entry, 0);
            load_page(pa, ra);
            for (int i = 0; i < cnt; i += 2) {
                const bool has_b = i + 1 < cnt;
                const int pb = has_b ? __builtin_amdgcn_readlane(entry, min_(i + 1, 63)) : pa;
                load_page(pb, rb);
                process(ra, pa, g0 + i);
                const int pn = i + 2 < cnt ? __builtin_amdgcn_readlane(entry, min_(i + 2, 63)) : pb;
                load_page(pn, ra);
                if (has_b) process(rb, pb, g0 + i + 1);
                pa = pn;
            }
        }
    }

    // ---- merge the 8 token slots of the wave (lanes with equal qs) ----
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float mw = mref[g];
        mw = fmaxf(mw, __shfl_xor(mw, 8));
        mw = fmaxf(mw, __shfl_xor(mw, 16));
        mw = fmaxf(mw, __shfl_xor(mw, 32));
        const float f = (mref[g] == -INFINITY) ? 0.f : exp2_hw(mref[g] - mw);
        float lw = lsum[g] * f;
        lw += __shfl_xor(lw, 8);
        lw += __shfl_xor(lw, 16);
        lw += __shfl_xor(lw, 32);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            float x = acc[g][e] * f;
            x += __shfl_xor(x, 8);
            x += __shfl_xor(x, 16);
            x += __shfl_xor(x, 32);
            acc[g][e] = x;
        }
        if (t8 == 0) {
#pragma unroll
            for (int e = 0; e < 16; ++e) sm_o[wave][g][16 * qs + e] = acc[g][e];
        }
        if (lane == 0) {
            sm_m[wave][g] = mw;
            sm_l[wave][g] = lw;
        }
    }
    __syncthreads();

    // ---- merge the waves and write this chunk's normalised partial ----
    for (int idx = tid; idx < G * kD; idx += kThreads) {
        const int g = idx / kD;
        const int d = idx - g * kD;
        float m = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
            if (sm_l[w][g] > 0.f) m = fmaxf(m, sm_m[w][g]);
        float lt = 0.f, ot = 0.f;
        if (m != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                // sm_o and sm_l are unnormalised sums relative to the wave's own maximum
                const float rs = sm_l[w][g] > 0.f ? exp2_hw(sm_m[w][g] - m) : 0.f;
                lt = __builtin_fmaf(rs, sm_l[w][g], lt);
                ot = __builtin_fmaf(rs, sm_o[w][g][d], ot);
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

hipError_t launch_decode_bf16(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* seq_lens, void* o,
                              int B, int Hq, int Hkv, int d, int num_pages, int max_pages_per_seq,
                              int len_cap, float scale, int splits, int chunk_pages,
                              float* ws_o, float* ws_m, float* ws_l, hipStream_t stream) {
    (void)d;
    const dim3 grid((unsigned)(B * Hkv), (unsigned)splits);
    const float sl2 = scale * kLog2e;
    auto qp = static_cast<const uint16_t*>(q);
    auto kp = static_cast<const uint16_t*>(k_cache);
    auto vp = static_cast<const uint16_t*>(v_cache);
    const int G = Hq / Hkv;
#define FA_DECODE_LAUNCH(GG)                                                                     \
    hipLaunchKernelGGL(decode_bf16_kernel<GG>, grid, dim3(kThreads), 0, stream, qp, kp, vp,      \
                       block_table, seq_lens, ws_o, ws_m, ws_l, Hq, Hkv, num_pages,             \
                       max_pages_per_seq, len_cap, sl2, chunk_pages)
    switch (G) {
        case 1: FA_DECODE_LAUNCH(1); break;
        case 2: FA_DECODE_LAUNCH(2); break;
        case 4: FA_DECODE_LAUNCH(4); break;
        default: FA_DECODE_LAUNCH(8); break;
    }
#undef FA_DECODE_LAUNCH
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_merge(ws_o, ws_m, ws_l, o, 1, nullptr, nullptr, splits, B * Hq, kD, 1, stream);
}

}  // namespace fa
