// fwd_bf16_pipe.hip - software-pipelined tiled attention forward, bf16 in / bf16 out.
//
// Same method as fwd_bf16.hip ("FlashAttention" (shubhamtatvamasi.com), "The trick: tiles
// and an online softmax"; FA-2 schedule from the family table on the same page), with a
// CDNA4 schedule built for one wave per SIMD:
//  * 4 waves x 64 query rows = 256 rows per workgroup. Each wave holds two 32-row query
//    blocks, so every K or V operand fragment read from LDS feeds two MFMAs: half the LDS
//    bytes per FLOP of a 32-row wave.
//  * Software pipelining over 32-key half tiles: while the wave turns half tile i's scores
//    into probabilities (VALU: FMA, v_exp_f32, row sums, bf16 packing), it issues half tile
//    i+1's S^T = K Q^T MFMAs, which do not depend on them; both streams sit in one basic
//    block so the scheduler can interleave them. O += V^T P^T of half tile i follows.
//  * LDS staging is per 64-key tile with one barrier per tile: K has three stages (K_j and
//    K_{j+1} are read during tile j while K_{j+2} is written), V two (V_j read, V_{j+1}
//    written): 80 KiB.
//  * Layouts, swizzles, buffer loads, log2-domain lazy-reference softmax and the XCD-aware
//    work order are those of fwd_bf16.hip.
#include "fa_internal.hpp"
#include "gfx950.hpp"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQB = 2;                   // 32-row query blocks per wave
constexpr int kBr = 32 * kQB * kWaves;   // query rows per workgroup
constexpr int kBc = 64;                  // keys per tile
constexpr int kXcds = 8;
constexpr float kLazy = 8.f;
constexpr int kBufferDword3 = 0x00020000;

__device__ __forceinline__ int kappa(int m) {
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}
__device__ __forceinline__ int vt_swz(int d) { return ((d >> 2) & 7) ^ ((d & 3) << 1); }

template <int D>
struct Tile {
    static constexpr int kChunks = D / 8;
    static constexpr int kKBytes = kBc * D * 2;
    static constexpr int kVBytes = D * kBc * 2;
    static constexpr int kKLoads = kBc * kChunks / kThreads;
    static constexpr int kVQuads = D / 4;
    static constexpr int kVKeys = kBc * kVQuads / kThreads;
};

template <int D>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_pipe_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ m_out, float* __restrict__ l_out, int B, int Hq,
    int Hkv, int N, float scale_log2, int causal, int nqb) {
    using T = Tile<D>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[3 * T::kKBytes + 2 * T::kVBytes];
    unsigned char* const kbuf = smem;
    unsigned char* const vbuf = smem + 3 * T::kKBytes;

    // ---- work item (see fwd_bf16.hip): XCD-contiguous runs, heaviest blocks first ----
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
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int row0 = qb * kBr + wave * 32 * kQB;  // first query row of this wave

    // ---- Q^T fragments of both query blocks ----
    bf16x8 qf[kQB][D / 16];
#pragma unroll
    for (int c = 0; c < kQB; ++c) {
        const uint16_t* src = qh + (size_t)min_(row0 + 32 * c + l32, N - 1) * D + 8 * hh;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            qf[c][kk] = *reinterpret_cast<const bf16x8*>(src + 16 * kk);
    }
#pragma unroll
    for (int c = 0; c < kQB; ++c)
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) asm volatile("" : "+v"(qf[c][kk]));

    f32x16 acc_o[kQB][D / 32];
    float m_run[kQB], m_ref[kQB], l_part[kQB];
#pragma unroll
    for (int c = 0; c < kQB; ++c) {
#pragma unroll
        for (int i = 0; i < D / 32; ++i) acc_o[c][i] = f32x16{};
        m_run[c] = -INFINITY;
        m_ref[c] = -INFINITY;
        l_part[c] = 0.f;
    }

    const int kv_end = causal ? min_(N, qb * kBr + kBr) : N;
    const int n_tiles = (kv_end + kBc - 1) / kBc;
    // last tile holding a key this wave's rows may attend
    const int last_tile = causal ? min_(n_tiles - 1, (row0 + 32 * kQB - 1) / kBc) : n_tiles - 1;

    // ---- staging (buffer loads, constant per-thread offsets) ----
    u32x4 kreg[T::kKLoads];
    u32x2 vreg[T::kVKeys];
    const int k_r0 = tid / T::kChunks;
    const int k_ch = tid % T::kChunks;
    const int v_dq = tid % T::kVQuads;
    const int v_kg = tid / T::kVQuads;
    constexpr int kRowsPerLoad = kThreads / T::kChunks;
    int k_boff[T::kKLoads];
#pragma unroll
    for (int i = 0; i < T::kKLoads; ++i) k_boff[i] = ((k_r0 + i * kRowsPerLoad) * D + k_ch * 8) * 2;
    const int v_boff = (v_kg * T::kVKeys * D + v_dq * 4) * 2;

    auto rsrc = [&](const uint16_t* base, int j) {
        const int kv0 = j * kBc;
        return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (size_t)kv0 * D), (short)0,
                                                 min_(N - kv0, kBc) * D * 2, kBufferDword3);
    };
    auto load_k = [&](int j) {
        const __amdgpu_buffer_rsrc_t r = rsrc(kh, j);
#pragma unroll
        for (int i = 0; i < T::kKLoads; ++i)
            kreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, k_boff[i], 0, 0));
    };
    auto load_v = [&](int j) {
        const __amdgpu_buffer_rsrc_t r = rsrc(vh, j);
#pragma unroll
        for (int i = 0; i < T::kVKeys; ++i)
            vreg[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, v_boff + i * D * 2, 0, 0));
    };
    auto store_k = [&](int buf) {
        unsigned char* ks = kbuf + buf * T::kKBytes;
#pragma unroll
        for (int i = 0; i < T::kKLoads; ++i) {
            const int r = k_r0 + i * kRowsPerLoad;
            const int sw = kappa(r & 15) & (T::kChunks - 1);
            *reinterpret_cast<u32x4*>(ks + r * (D * 2) + ((k_ch ^ sw) << 4)) = kreg[i];
        }
    };
    auto store_v = [&](int buf) {
        unsigned char* vs = vbuf + buf * T::kVBytes;
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

    // S^T = K Q^T for half tile i (32 keys of tile i/2, both query blocks).
    auto compute_s = [&](int i, f32x16 (&s)[kQB]) {
        const int j = i >> 1;
        const unsigned char* ks = kbuf + (j % 3) * T::kKBytes;
        const int sw = (l32 & 15) & (T::kChunks - 1);
        const unsigned char* base = ks + (32 * (i & 1) + kappa(l32)) * (D * 2);
#pragma unroll
        for (int c = 0; c < kQB; ++c) s[c] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(base + (((2 * kk + hh) ^ sw) << 4));
#pragma unroll
            for (int c = 0; c < kQB; ++c) s[c] = mfma_32x32x16(a, qf[c][kk], s[c]);
        }
    };

    // One pipeline step: softmax and O update of half tile i (scores in `cur`), while the
    // scores of half tile i+1 are computed into `nxt`.
    auto step = [&](int i, f32x16 (&cur)[kQB], f32x16 (&nxt)[kQB]) {
        const int j = i >> 1;
        const int kb = i & 1;
        const int kv0 = j * kBc + 32 * kb;  // first key of the half tile
        if (kb == 0) {
            if (j + 2 < n_tiles) load_k(j + 2);
            if (j + 1 < n_tiles) load_v(j + 1);
        }
        if (j <= last_tile) {
            float m_use[kQB], alpha[kQB];
#pragma unroll
            for (int c = 0; c < kQB; ++c) {
                const int r0 = row0 + 32 * c;
                const bool need_mask = (causal && kv0 + 31 > r0) || (kv0 + 32 > N);
                if (need_mask) {
                    const int qrow = r0 + l32;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kv0 + 16 * (r >> 3) + 8 * hh + (r & 7);
                        const bool bad = key >= N || (causal && key > qrow);
                        cur[c][r] = bad ? -INFINITY : cur[c][r];
                    }
                }
                float mx = cur[c][0];
#pragma unroll
                for (int r = 1; r < 16; ++r) mx = fmaxf(mx, cur[c][r]);
                mx = pair32_max(mx) * scale_log2;
                m_run[c] = fmaxf(m_run[c], mx);
                alpha[c] = 1.f;
                const bool move = mx > m_ref[c] + kLazy;
                if (__any(move)) {
                    const float r_new = move ? mx : m_ref[c];
                    alpha[c] = exp2_hw(m_ref[c] - r_new);
                    m_ref[c] = r_new;
#pragma unroll
                    for (int d4 = 0; d4 < D / 32; ++d4) acc_o[c][d4] *= alpha[c];
                }
                m_use[c] = (m_ref[c] == -INFINITY) ? 0.f : m_ref[c];
            }

            // ---- one basic block: S MFMAs of half tile i+1 beside the probabilities of i ----
            compute_s(i + 1, nxt);  // unused when past the wave's last tile (stale stage)

            uint32_t pk[kQB][8];
#pragma unroll
            for (int c = 0; c < kQB; ++c) {
                float rs = 0.f;
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const float p0 = exp2_hw(__builtin_fmaf(cur[c][r], scale_log2, -m_use[c]));
                    const float p1 = exp2_hw(__builtin_fmaf(cur[c][r + 1], scale_log2, -m_use[c]));
                    rs += p0 + p1;
                    pk[c][r >> 1] = pack_bf16x2(p0, p1);
                }
                l_part[c] = l_part[c] * alpha[c] + rs;
            }

            // O^T += V^T P^T for half tile i; each V fragment feeds both query blocks.
            const unsigned char* vs = vbuf + (j & 1) * T::kVBytes;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                bf16x8 pb[kQB];
#pragma unroll
                for (int c = 0; c < kQB; ++c) {
                    u32x4 pw = {pk[c][4 * t], pk[c][4 * t + 1], pk[c][4 * t + 2], pk[c][4 * t + 3]};
                    pb[c] = __builtin_bit_cast(bf16x8, pw);
                }
                const int chunk = 4 * kb + 2 * t + hh;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const int d = 32 * db + l32;
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                        vs + d * (kBc * 2) + ((chunk ^ vt_swz(d)) << 4));
#pragma unroll
                    for (int c = 0; c < kQB; ++c) acc_o[c][db] = mfma_32x32x16(a, pb[c], acc_o[c][db]);
                }
            }
        }
        if (kb == 1) {
            // K_{j+2} goes to the stage K_{j-1} used (last read during tile j-1); V_{j+1}
            // replaces V_{j-1}. Tile j's own stages are untouched.
            if (j + 2 < n_tiles) store_k((j + 2) % 3);
            if (j + 1 < n_tiles) store_v((j + 1) & 1);
            __syncthreads();
        }
    };

    // ---- prologue: K0, V0, K1 staged; scores of half tile 0 ----
    load_k(0);
    load_v(0);
    store_k(0);
    store_v(0);
    if (n_tiles > 1) {
        load_k(1);
        store_k(1);
    }
    __syncthreads();
    f32x16 sa[kQB], sb[kQB];
    compute_s(0, sa);

    const int n_half = 2 * n_tiles;
    for (int i = 0; i < n_half; i += 2) {
        step(i, sa, sb);
        step(i + 1, sb, sa);
    }

    // ---- epilogue ----
#pragma unroll
    for (int c = 0; c < kQB; ++c) {
        const int qrow = row0 + 32 * c + l32;
        const float l_tot = pair32_sum(l_part[c]);
        if (qrow < N) {
            const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
            uint16_t* dst = o + qoff + (size_t)qrow * D;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d = 32 * db + 8 * g + 4 * hh;
                    u32x2 w = {pack_bf16x2(acc_o[c][db][4 * g] * inv, acc_o[c][db][4 * g + 1] * inv),
                               pack_bf16x2(acc_o[c][db][4 * g + 2] * inv, acc_o[c][db][4 * g + 3] * inv)};
                    *reinterpret_cast<u32x2*>(dst + d) = w;
                }
            if (hh == 0) {
                const size_t ridx = (size_t)(b * Hq + h) * N + qrow;
                if (m_out) m_out[ridx] = (l_tot > 0.f) ? m_run[c] * kLn2 : -INFINITY;
                if (l_out) l_out[ridx] = (l_tot > 0.f) ? l_tot * exp2_hw(m_ref[c] - m_run[c]) : 0.f;
            }
        }
    }
}

}  // namespace

hipError_t launch_fwd_bf16_pipe(const void* q, const void* k, const void* v, void* o, float* m_out,
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
        hipLaunchKernelGGL(fwd_bf16_pipe_kernel<128>, dim3((unsigned)grid), dim3(kThreads), 0,
                           stream, qp, kp, vp, op, m_out, l_out, B, Hq, Hkv, N, sl2, causal, nqb);
    else
        hipLaunchKernelGGL(fwd_bf16_pipe_kernel<64>, dim3((unsigned)grid), dim3(kThreads), 0,
                           stream, qp, kp, vp, op, m_out, l_out, B, Hq, Hkv, N, sl2, causal, nqb);
    return hipGetLastError();
}

}  // namespace fa
