// fwd_bf16.hip - tiled attention forward, bf16 in / bf16 out, on the gfx950 matrix cores.
//
// Method: "FlashAttention" (shubhamtatvamasi.com), "The trick: tiles and an online softmax":
// Q is split into row blocks and K/V into column blocks; each score tile lives only on chip
// and is folded into a running row maximum m, running sum l and rescaled accumulator O, and
// the block's output is O / l. Scheduling follows the FlashAttention-2 row of the family
// table on the same page (parallel over query blocks; normalise once at the end). Causal
// tiles strictly above the diagonal are never loaded ("The trick", streaming demo).
//
// CDNA4 design (one workgroup = 4 waves = 128 query rows; one K/V tile = 64 keys):
//  * Each wave owns 32 query rows and computes the TRANSPOSED score tile S^T = K Q^T with
//    v_mfma_f32_32x32x16_bf16, so every lane holds the scores of ONE query row: the row
//    maximum and row sum are in-lane reductions plus one exchange with lane l ^ 32.
//  * The S^T accumulator is converted to bf16 in registers and used directly as the B
//    operand of O^T += V^T P^T. K rows are fetched in a permuted order (bits 2 and 3 of the
//    row index swapped) so that the accumulator's register order already equals the key
//    order the second MFMA expects; no LDS round trip for P.
//  * K is staged in LDS row-major, V transposed ([d][key]); both with an XOR swizzle of the
//    16-byte chunk index so that the MFMA operand reads and the staging writes are free of
//    bank conflicts on gfx950's LDS (64 banks of 4 bytes, 128 bytes per cycle). The next tile is
//    prefetched into registers while the current one is consumed (double-buffered LDS, one
//    barrier per tile).
//  * Scores are kept in the log2 domain: p = exp2(s * scale * log2(e) - m), one FMA and one
//    v_exp_f32 per score. The exponent reference moves only when a row maximum beats it by
//    more than 2^8, so the O rescale is rare.
//  * Grid: one workgroup per (query block, head). Each XCD gets a contiguous run of work
//    items ordered by KV head, so it streams about one head's K/V at a time from its own
//    L2; query heads sharing a KV head (GQA) run together; heaviest causal blocks first.
#include "fa_internal.hpp"
#include "gfx950.hpp"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBr = 32 * kWaves;  // query rows per workgroup
constexpr int kBc = 64;           // keys per tile
constexpr int kXcds = 8;          // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr float kLazy = 8.f;      // reference-max slack (log2 units) before O is rescaled
// Word 3 of a raw (untyped, unswizzled) buffer resource descriptor on gfx9-family GPUs.
constexpr int kBufferDword3 = 0x00020000;

// Row permutation within each 16-row group: swap bits 2 and 3.
__device__ __forceinline__ int kappa(int m) {
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

template <int D>
struct Tile {
    static constexpr int kChunks = D / 8;                          // 16-byte chunks per K row
    static constexpr int kKBytes = kBc * D * 2;
    static constexpr int kVBytes = D * kBc * 2;
    static constexpr int kStage = kKBytes + kVBytes;
    static constexpr int kKLoads = kBc * kChunks / kThreads;       // 16-byte loads per thread
    static constexpr int kVQuads = D / 4;                          // 4-column groups per V row
    static constexpr int kVKeys = kBc * kVQuads / kThreads;        // keys per thread (V): 8 or 4
};

// XOR swizzle of the 16-byte chunk index of row d of the transposed V tile. Under the LDS
// banking measured on gfx950 (64 banks of 4 bytes, 128 bytes per cycle) it keeps both the
// MFMA operand reads (8 consecutive rows per cycle) and the transposed writes (rows
// 4q + j for 8 consecutive q per cycle) conflict free.
__device__ __forceinline__ int vt_swz(int d) { return ((d >> 2) & 7) ^ ((d & 3) << 1); }

template <int D>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ m_out, float* __restrict__ l_out, int B, int Hq,
    int Hkv, int N, float scale_log2, int causal, int nqb) {
    using T = Tile<D>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * T::kStage];

    // ---- work item ----
    // Items are ordered (KV group, query block from the last to the first, head in group).
    // Workgroups are dealt round-robin over the 8 XCDs, so XCD x receives ids x, x+8, ...;
    // mapping its i-th workgroup to item x*per_xcd + i gives every XCD one contiguous run of
    // items: it works through about one KV head at a time (K/V stay in its L2), the query
    // heads sharing that KV head run side by side, and within a head the heaviest causal
    // query blocks come first.
    const int G = Hq / Hkv;
    const int per_unit = nqb * G;
    const int total = B * Hkv * per_unit;
    const int per_xcd = (total + kXcds - 1) / kXcds;
    const int item = (int)(blockIdx.x % kXcds) * per_xcd + (int)(blockIdx.x / kXcds);
    if (item >= total) return;
    const int kvg = item / per_unit;
    const int rem = item - kvg * per_unit;
    const int qb = causal ? (nqb - 1 - rem / G) : rem / G;
    const int gi = rem - (rem / G) * G;
    const int b = kvg / Hkv;
    const int kvh = kvg - b * Hkv;
    const int h = kvh * G + gi;

    const size_t qoff = ((size_t)(b * Hq + h) * N) * D;
    const size_t koff = ((size_t)(b * Hkv + kvh) * N) * D;
    const uint16_t* qh = q + qoff;
    const uint16_t* kh = k + koff;
    const uint16_t* vh = v + koff;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    const int row0 = qb * kBr + wave * 32;  // first query row of this wave
    const int qrow = row0 + l32;            // the query row this lane's column holds

    // ---- Q^T fragments (B operand), kept in registers for the whole kernel ----
    bf16x8 qf[D / 16];
    {
        const uint16_t* src = qh + (size_t)min_(qrow, N - 1) * D + 8 * hh;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            qf[kk] = *reinterpret_cast<const bf16x8*>(src + 16 * kk);
    }
    // Complete the Q loads here: the empty asm redefines the fragments, so the wait for the
    // loads lands before the loop. Otherwise the loop header merges "possibly pending" state
    // from before the loop and every tile's MFMAs wait on that tile's K/V prefetch instead.
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) asm volatile("" : "+v"(qf[kk]));

    f32x16 acc_o[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) acc_o[i] = f32x16{};
    float m_run = -INFINITY;  // running max of scale*log2(e)*s for row qrow
    float m_ref = -INFINITY;  // reference the exponentials are taken against (<= m_run)
    float l_part = 0.f;       // running sum over this lane's half of every tile

    const int kv_end = causal ? min_(N, qb * kBr + kBr) : N;
    const int n_tiles = (kv_end + kBc - 1) / kBc;

    // ---- global -> register staging of one K/V tile ----
    // Buffer loads: each tile gets a scalar resource descriptor (base = the tile's first key,
    // size = the keys left in the head), and every thread reads at offsets fixed for the
    // whole kernel, so a load costs no vector address arithmetic. Keys past the head's end
    // read as zero through the descriptor's range check (and are masked anyway).
    u32x4 kreg[T::kKLoads];
    u32x2 vreg[T::kVKeys];
    const int k_r0 = tid / T::kChunks;               // K: rows k_r0 + (kThreads/kChunks)*i
    const int k_ch = tid % T::kChunks;
    const int v_dq = tid % T::kVQuads;                // V: keys v_kg*kVKeys + i, columns 4*v_dq..
    const int v_kg = tid / T::kVQuads;
    constexpr int kRowsPerLoad = kThreads / T::kChunks;
    int k_boff[T::kKLoads];
#pragma unroll
    for (int i = 0; i < T::kKLoads; ++i) k_boff[i] = ((k_r0 + i * kRowsPerLoad) * D + k_ch * 8) * 2;
    const int v_boff = (v_kg * T::kVKeys * D + v_dq * 4) * 2;
    auto load_tile = [&](int j) {
        const int kv0 = j * kBc;
        const int bytes = min_(N - kv0, kBc) * D * 2;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(kh + (size_t)kv0 * D), (short)0, bytes, kBufferDword3);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(vh + (size_t)kv0 * D), (short)0, bytes, kBufferDword3);
#pragma unroll
        for (int i = 0; i < T::kKLoads; ++i)
            kreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, k_boff[i], 0, 0));
#pragma unroll
        for (int i = 0; i < T::kVKeys; ++i)
            vreg[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rv, v_boff + i * D * 2, 0, 0));
    };
    auto store_tile = [&](int buf) {
        unsigned char* ks = smem + buf * T::kStage;
        unsigned char* vs = ks + T::kKBytes;
#pragma unroll
        for (int i = 0; i < T::kKLoads; ++i) {
            const int r = k_r0 + i * kRowsPerLoad;
            const int sw = kappa(r & 15) & (T::kChunks - 1);
            *reinterpret_cast<u32x4*>(ks + r * (D * 2) + ((k_ch ^ sw) << 4)) = kreg[i];
        }
        // V transposed: row d of the [d][key] tile gets this thread's kVKeys keys; each
        // word pairs two keys of one column (one v_perm_b32).
        const int key0 = v_kg * T::kVKeys;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d = v_dq * 4 + j;
            const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
            uint32_t w[T::kVKeys / 2];
#pragma unroll
            for (int i = 0; i < T::kVKeys / 2; ++i)
                w[i] = __builtin_amdgcn_perm(vreg[2 * i + 1][j >> 1], vreg[2 * i][j >> 1], sel);
            unsigned char* dst = vs + d * (kBc * 2) + (((key0 >> 3) ^ vt_swz(d)) << 4) + (key0 & 7) * 2;
            if constexpr (T::kVKeys == 8) {
                *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
            } else {
                *reinterpret_cast<u32x2*>(dst) = u32x2{w[0], w[1]};
            }
        }
    };

    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int j = 0; j < n_tiles; ++j) {
        const bool has_next = j + 1 < n_tiles;
        if (has_next) load_tile(j + 1);

        const int kv0 = j * kBc;
        const bool active = !causal || kv0 <= row0 + 31;
        if (active) {
            const unsigned char* ks = smem + (j & 1) * T::kStage;
            const unsigned char* vs = ks + T::kKBytes;

            // S^T = K Q^T for two 32-key blocks.
            f32x16 s[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int krow = 32 * kb + kappa(l32);
                const int sw = (l32 & 15) & (T::kChunks - 1);
                const unsigned char* base = ks + krow * (D * 2);
                f32x16 acc = f32x16{};
#pragma unroll
                for (int kk = 0; kk < D / 16; ++kk) {
                    const bf16x8 a =
                        *reinterpret_cast<const bf16x8*>(base + (((2 * kk + hh) ^ sw) << 4));
                    acc = mfma_32x32x16(a, qf[kk], acc);
                }
                s[kb] = acc;
            }

            // Mask: causal diagonal tiles and the ragged key tail.
            const bool need_mask = (causal && kv0 + kBc - 1 > row0) || (kv0 + kBc > N);
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kv0 + 32 * kb + 16 * (r >> 3) + 8 * hh + (r & 7);
                        const bool bad = key >= N || (causal && key > qrow);
                        s[kb][r] = bad ? -INFINITY : s[kb][r];
                    }
            }

            // Online softmax (log2 domain).
            float mx = s[0][0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
            mx = pair32_max(mx) * scale_log2;
            m_run = fmaxf(m_run, mx);
            // Lazy rescale: p is taken relative to a reference m_ref that moves only when
            // a row's maximum exceeds it by more than 2^8, so p <= 256 and the O rescale is
            // rare. Exact up to rounding: the final O / l cancels the reference.
            float alpha = 1.f;
            const bool move = mx > m_ref + kLazy;
            if (__any(move)) {
                const float r_new = move ? mx : m_ref;
                alpha = exp2_hw(m_ref - r_new);
                m_ref = r_new;
#pragma unroll
                for (int i = 0; i < D / 32; ++i) acc_o[i] *= alpha;
            }
            const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;

            uint32_t pk[2][8];
            float rs = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const float p0 = exp2_hw(__builtin_fmaf(s[kb][r], scale_log2, -m_use));
                    const float p1 = exp2_hw(__builtin_fmaf(s[kb][r + 1], scale_log2, -m_use));
                    rs += p0 + p1;
                    pk[kb][r >> 1] = pack_bf16x2(p0, p1);
                }
            l_part = l_part * alpha + rs;

            // O^T += V^T P^T.
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    u32x4 pw = {pk[kb][4 * t], pk[kb][4 * t + 1], pk[kb][4 * t + 2], pk[kb][4 * t + 3]};
                    const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
                    const int chunk = 4 * kb + 2 * t + hh;
#pragma unroll
                    for (int db = 0; db < D / 32; ++db) {
                        const int d = 32 * db + l32;
                        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                            vs + d * (kBc * 2) + ((chunk ^ vt_swz(d)) << 4));
                        acc_o[db] = mfma_32x32x16(a, pb, acc_o[db]);
                    }
                }
        }

        if (has_next) store_tile((j + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue: O / l, bf16, and the optional row statistics ----
    const float l_tot = pair32_sum(l_part);
    if (qrow < N) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        uint16_t* dst = o + qoff + (size_t)qrow * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * db + 8 * g + 4 * hh;
                u32x2 w = {pack_bf16x2(acc_o[db][4 * g] * inv, acc_o[db][4 * g + 1] * inv),
                           pack_bf16x2(acc_o[db][4 * g + 2] * inv, acc_o[db][4 * g + 3] * inv)};
                *reinterpret_cast<u32x2*>(dst + d) = w;
            }
        if (hh == 0) {
            const size_t ridx = (size_t)(b * Hq + h) * N + qrow;
            if (m_out) m_out[ridx] = (l_tot > 0.f) ? m_run * kLn2 : -INFINITY;
            if (l_out) l_out[ridx] = (l_tot > 0.f) ? l_tot * exp2_hw(m_ref - m_run) : 0.f;
        }
    }
}

}  // namespace

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* m_out,
                           float* l_out, int B, int Hq, int Hkv, int N, int d, float scale,
                           int causal, hipStream_t stream) {
    const int nqb = (N + kBr - 1) / kBr;
    const long long items = (long long)nqb * B * Hq;
    const long long grid = (items + kXcds - 1) / kXcds * kXcds;
    const float sl2 = scale * kLog2e;
    auto qp = static_cast<const uint16_t*>(q);
    auto kp = static_cast<const uint16_t*>(k);
    auto vp = static_cast<const uint16_t*>(v);
    auto op = static_cast<uint16_t*>(o);
    if (d == 128)
        hipLaunchKernelGGL(fwd_bf16_kernel<128>, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                           qp, kp, vp, op, m_out, l_out, B, Hq, Hkv, N, sl2, causal, nqb);
    else
        hipLaunchKernelGGL(fwd_bf16_kernel<64>, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                           qp, kp, vp, op, m_out, l_out, B, Hq, Hkv, N, sl2, causal, nqb);
    return hipGetLastError();
}

}  // namespace fa
