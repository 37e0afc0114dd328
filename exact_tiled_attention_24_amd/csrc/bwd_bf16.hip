// bwd_bf16.hip - attention backward by recomputation, bf16 in / bf16 out, fp32 accumulation.
//
// Method: "FlashAttention, explained." (vibeengines.com), the backward-pass section: nothing of
// size N x N is stored by the forward; the backward recomputes the probabilities tile by tile
// from Q, K and the saved row statistics, P = exp(s - m) / l, and uses D_i = rowsum(dO_i * O_i)
// so that dS = P * (dP - D) needs no second pass over the keys. With dP = dO V^T:
//     dV = P^T dO,   dK = scale dS^T Q,   dQ = scale dS K.
//
// Three kernels:
//  * bwd_prep: D_i and the log2-domain normaliser L_i = (m_i + ln l_i) log2 e of every query
//    row, so that P = exp2(scale log2e q.k - L) (L = +inf for a row with no key: P = 0).
//  * bwd_dkdv: one workgroup per (128-key block, KV head); each wave keeps its 32 keys' K and V
//    in registers and walks the query chunks (32 rows of Q and dO staged in LDS) of every
//    query head of the KV group, accumulating dV^T and dK^T.
//  * bwd_dq: one workgroup per (128-query block, query head); each wave keeps its 32 queries'
//    Q and dO in registers and walks the key chunks (32 rows of K and V in LDS).
// Chunks are double-buffered: the next chunk's rows load straight into the other LDS buffer
// while the current chunk's products run, with one barrier per chunk.
// All products use v_mfma_f32_32x32x16_bf16. As in the forward kernel, the score tile is
// computed with the rows of its A operand read in an order that swaps bits 2 and 3 of the row
// index, so that the accumulator, rounded to bf16, is directly the B operand of the next
// product (no LDS round trip for P or dS); the transposed operands (Q^T, dO^T, K^T) come out
// of row-major LDS tiles through ds_read_b64_tr_b16.
#include "fa_internal.hpp"
#include "gfx950.hpp"

namespace fa {
namespace {

constexpr int kThreads = 256;  // 4 waves
// 32-row sub-chunks per staged chunk: one in both kernels, so that each fits two waves per
// SIMD (two sub-chunks in dK/dV interleave their products but leave it one wave per SIMD,
// which measured slower)
constexpr int kSubKV = 1, kSubQ = 1;
constexpr int kBlock = 128;    // keys (dK/dV) or queries (dQ) per workgroup: 32 per wave

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef const __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef const __attribute__((address_space(3))) unsigned char* lds_cptr;

// Word 3 of a raw buffer descriptor (no format, no swizzle) for the loads into LDS.
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ int kappa(int m) {
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Natural row index of accumulator register r in lane half h when the A operand's rows were
// read in kappa order: registers 0-7 hold rows 8h .. 8h + 7, registers 8-15 rows 16 + 8h ..
__device__ __forceinline__ int acc_row(int r, int h) { return 16 * (r >> 3) + 8 * h + (r & 7); }

template <int D, int SUB>
struct Stage {
    static constexpr int kChunk = 32 * SUB;  // rows of a staged chunk
    static constexpr int kRow = D * 2;       // row, bytes (unpadded; chunks swizzled)
    static constexpr int kTile = kChunk * kRow;
};

// A staged row's 16-byte chunk c sits at chunk position c ^ swz(row). With 64 four-byte
// banks this keeps every access of a tile conflict-free: the row reads (16 lanes, 16 rows,
// one chunk) find 16 different bank groups, and so do the transposing reads (32 lanes, 4 rows,
// 4 adjacent chunks each), which a row pad cannot give together with the row reads.
// d = 128 (a row fills the banks once): the chunk index is XORed with (row bits 0-1) << 2 |
// row bits 2-3. d = 64 (two rows per bank line): with row bit 1 << 2 | row bits 2-3.
template <int D>
__device__ __forceinline__ int swz(int r) {
    return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// A staged tile loaded straight from global memory into LDS (buffer_load ... lds, 1 KiB per
// instruction, no registers held while the data flies). Instruction k fills tile bytes
// 1024 k ..: lane l writes the 16 bytes at 1024 k + 16 l, i.e. row (1024 k + 16 l) / R at
// chunk position p, so it loads that row's logical chunk p ^ swz(row). Rows past the end of
// the descriptor's range read as zeros. Each of the 4 waves issues a quarter of the
// instructions; the caller waits with s_waitcnt vmcnt before the barrier that publishes the
// tile.
template <int D, int SUB>
struct TileDma {
    static constexpr int kRow = Stage<D, SUB>::kRow;
    static constexpr int kPerWave = Stage<D, SUB>::kTile / 1024 / 4;
    static_assert(Stage<D, SUB>::kTile % 4096 == 0, "whole 1 KiB loads per wave");
    unsigned off[kPerWave];  // this lane's byte offset in the tile's rows, per instruction
    __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
        for (int j = 0; j < kPerWave; ++j) {
            const int byte = 1024 * (wave * kPerWave + j) + 16 * lane;
            const int row = byte / kRow, p = (byte - row * kRow) / 16;
            off[j] = (unsigned)(row * kRow + 16 * (p ^ swz<D>(row)));
        }
    }
    // rows from byte row0 of the buffer r into the tile at LDS address lds_tile
    __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t r, unsigned row0, unsigned lds_tile,
                                          int wave) const {
        const unsigned dst = lds_tile + 1024u * (unsigned)(wave * kPerWave);
#pragma unroll
        for (int j = 0; j < kPerWave; ++j)
            asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                         :
                         : "v"(row0 + off[j]), "s"(r), "{m0}"(dst + 1024u * j)
                         : "memory");
    }
};

// A operand of a 32 x 16 slice (K-dim chunk kk) of a staged tile, rows in kappa order.
template <int D>
__device__ __forceinline__ bf16x8 rows_frag(lds_cptr tile, int lane, int kk) {
    const int r = kappa(lane & 31);
    return *reinterpret_cast<const lds_bf16x8*>(tile + r * Stage<D, 1>::kRow +
                                                 16 * ((2 * kk + (lane >> 5)) ^ swz<D>(r)));
}

// A operand of the transposed tile X^T (rows = head dimensions 32 db .., K-dim = the tile's
// rows 16 t ..): ds_read_b64_tr_b16 transposes within each 16-lane group, so two reads give
// a lane its 8 consecutive rows of one head dimension.
template <int D>
__device__ __forceinline__ bf16x8 trans_frag(lds_cptr tile, int lane, int t, int db) {
    constexpr int R = Stage<D, 1>::kRow;
    // the lane's 8 bytes: row r (+ 4 for the second read), head dimensions 32 db + 16 g +
    // 4 (lane & 3) .., i.e. chunk 4 db + 2 g + (lane & 3) / 2, byte 8 (lane & 1) of it
    const int r = 8 * (lane >> 5) + ((lane & 15) >> 2);
    const int c = 4 * db + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const lds_cptr row = tile + 16 * t * R + 8 * (lane & 1);
    const lds_cptr plo = row + r * R + 16 * (c ^ swz<D>(r));
    const lds_cptr phi = row + (r + 4) * R + 16 * (c ^ swz<D>(r + 4));
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)plo);
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)phi);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Accumulator registers 8 t .. 8 t + 7, rounded to bf16: the B operand (K-dim rows 16 t ..).
__device__ __forceinline__ bf16x8 acc_operand(const float (&x)[16], int t) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(x[8 * t + 2 * i], x[8 * t + 2 * i + 1]);
    return __builtin_bit_cast(bf16x8, w);
}

// Workgroups are dealt to the 8 XCDs round robin by linear id. xcd_position maps the linear
// id to a position in (head, block) order so that each XCD receives a contiguous run of
// positions: the ~32 workgroups one XCD runs at a time then share one or two heads, whose
// staged operands (4 MiB per head at N = 8192, d = 128) its L2 can hold. A bijection on
// 0 .. total - 1: XCD k holds the ids k, k + 8, .. and gets positions k q + min(k, r) on.
__device__ __forceinline__ int xcd_position(int total) {
    const int id = blockIdx.x + gridDim.x * blockIdx.y;
    const int k = id & 7, j = id >> 3, q = total >> 3, r = total & 7;
    return k * q + min_(k, r) + j;
}

// ---- D_i = rowsum(dO * O) and L_i = (m_i + ln l_i) log2 e, 4 threads per row ----
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(const uint16_t* __restrict__ o,
                                                            const uint16_t* __restrict__ dout,
                                                            const float* __restrict__ m,
                                                            const float* __restrict__ l,
                                                            float* __restrict__ lse2,
                                                            float* __restrict__ dsum, long long rows) {
    const long long row = (long long)blockIdx.x * (kThreads / 4) + threadIdx.x / 4;
    const int part = threadIdx.x & 3;
    float acc = 0.f;
    if (row < rows) {
        const uint16_t* po = o + row * D + part * (D / 4);
        const uint16_t* pd = dout + row * D + part * (D / 4);
#pragma unroll
        for (int c = 0; c < D / 4; c += 8) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(po + c);
            const u32x4 b = *reinterpret_cast<const u32x4*>(pd + c);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc = __builtin_fmaf(bf16_lo(a[i]), bf16_lo(b[i]), acc);
                acc = __builtin_fmaf(bf16_hi(a[i]), bf16_hi(b[i]), acc);
            }
        }
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    if (row < rows && part == 0) {
        dsum[row] = acc;
        const float lr = l[row];
        lse2[row] = lr > 0.f ? (m[row] + logf(lr)) * kLog2e : INFINITY;
    }
}

struct BwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* dout;
    const float* lse2;  // [B, Hq, N]
    const float* dsum;  // [B, Hq, N]
    uint16_t* dq;
    uint16_t* dk;
    uint16_t* dv;
    int Hq, Hkv, N;
    float scale, scale_log2;
    int causal;
};

// ---- dK, dV: workgroup = 128 keys of one KV head; wave = 32 keys ----
// (two waves per SIMD: the register budget is 256 per lane, with a small spill)
template <int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_dkdv_kernel(BwdArgs a) {
    constexpr int kSub = kSubKV;
    using S = Stage<D, kSub>;
    constexpr int kChunk = S::kChunk;
    // two buffers, each: Q chunk, dO chunk, L and D of its 32 queries
    constexpr int kBuf = 2 * S::kTile + 2 * kChunk * 4;
    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kBuf];

    const int N = a.N, G = a.Hq / a.Hkv;
    const int pos = xcd_position(gridDim.x * gridDim.y);
    const int bk = pos / gridDim.x;  // b * Hkv + kvh
    const int b = bk / a.Hkv, kvh = bk - b * a.Hkv;
    const int kb0 = (pos - bk * gridDim.x) * kBlock;  // (causal: the first blocks see the most queries)
    const int lane = threadIdx.x & 63, h = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int key = kb0 + 32 * wave + (lane & 31);  // this lane's key (accumulator column)

    // K and V of the lane's key as B operands (K-dim = head dimension 16 kk + 8 h ..)
    const size_t kvoff = (size_t)bk * N * D;
    bf16x8 kf[D / 16], vf[D / 16];
    {
        const int kr = min_(key, N - 1);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            kf[kk] = *reinterpret_cast<const bf16x8*>(a.k + kvoff + (size_t)kr * D + 16 * kk + 8 * h);
            vf[kk] = *reinterpret_cast<const bf16x8*>(a.v + kvoff + (size_t)kr * D + 16 * kk + 8 * h);
        }
    }
    f32x16 acc_dk[D / 32], acc_dv[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) acc_dk[i] = acc_dv[i] = f32x16{};

    // causal: queries before the block's first key see none of its keys. The chunks of all
    // query heads of the KV group form one sequence it = 0 .. G * nch - 1.
    const int q_first = a.causal ? (kb0 / kChunk) * kChunk : 0;
    const int nch = (N - q_first + kChunk - 1) / kChunk;
    const int total = G * nch;
    float rl = INFINITY, rd = 0.f;
    auto chunk_rows = [&](int it, size_t& qoff) {  // first query row; qoff = head's row base
        const int g = it / nch;
        qoff = ((size_t)b * a.Hq + kvh * G + g) * N;
        return q_first + (it - g * nch) * kChunk;
    };
    // The Q and dO rows of a chunk go straight into LDS; L and D go through registers.
    constexpr int R = S::kRow;
    TileDma<D, kSub> dma;
    dma.init(wave, lane);
    const unsigned lds_base = (unsigned)(size_t)(lds_cptr)smem;
    const int head_bytes = N * D * 2;
    auto load_chunk = [&](int it, int buf) {
        size_t qoff;
        const int qc0 = chunk_rows(it, qoff);
        const __amdgpu_buffer_rsrc_t rsq =
            __builtin_amdgcn_make_buffer_rsrc((void*)(a.q + qoff * D), (short)0, head_bytes, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t rsdo =
            __builtin_amdgcn_make_buffer_rsrc((void*)(a.dout + qoff * D), (short)0, head_bytes, kRsrcWord3);
        const unsigned row0 = (unsigned)qc0 * R, tile = lds_base + (unsigned)(buf * kBuf);
        dma.issue(rsq, row0, tile, wave);
        dma.issue(rsdo, row0, tile + (unsigned)S::kTile, wave);
        if (threadIdx.x < kChunk) {
            const int qi = qc0 + threadIdx.x;
            rl = qi < N ? a.lse2[qoff + qi] : INFINITY;
            rd = qi < N ? a.dsum[qoff + qi] : 0.f;
        }
    };
    // L and D into LDS; then this wave's loads into LDS are waited for (vmcnt counts the
    // wave's vector loads in issue order) before the barrier that publishes the chunk
    auto store_chunk = [&](int buf) {
        unsigned char* base = smem + buf * kBuf;
        if (threadIdx.x < kChunk) {
            reinterpret_cast<float*>(base + 2 * S::kTile)[threadIdx.x] = rl;
            reinterpret_cast<float*>(base + 2 * S::kTile)[kChunk + threadIdx.x] = rd;
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };
    if (total > 0) {
        load_chunk(0, 0);
        store_chunk(0);
    }
    __syncthreads();
    for (int it = 0; it < total; ++it) {
        // the other buffer was last read before the previous barrier
        if (it + 1 < total) load_chunk(it + 1, (it + 1) & 1);  // in flight during this chunk's products
        size_t qoff_chunk;  // (the head's row base; the chunk's rows are already staged)
        const int qc0 = chunk_rows(it, qoff_chunk);
        const unsigned char* base = smem + (it & 1) * kBuf;
        lds_cptr const lq = (lds_cptr)base;
        lds_cptr const ldo = (lds_cptr)(base + S::kTile);
        const float* s_l = reinterpret_cast<const float*>(base + 2 * S::kTile);
        const float* s_d = s_l + kChunk;

        // S = Q K^T and dP = dO V^T for each 32-query sub-chunk x the wave's 32 keys; the
        // sub-chunks are independent until the accumulations, so their matrix and vector work
        // can interleave
        f32x16 sc[kSub], dp[kSub];
#pragma unroll
        for (int u = 0; u < kSub; ++u) {
            sc[u] = f32x16{};
            dp[u] = f32x16{};
            const lds_cptr tq = lq + 32 * u * S::kRow, tdo = ldo + 32 * u * S::kRow;
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                sc[u] = mfma_32x32x16(rows_frag<D>(tq, lane, kk), kf[kk], sc[u]);
                dp[u] = mfma_32x32x16(rows_frag<D>(tdo, lane, kk), vf[kk], dp[u]);
            }
        }
        // No score of this chunk is masked when the wave's 32 keys and the chunk's queries all
        // lie inside the sequence and (causal) the chunk's first query follows the wave's last
        // key; then the probabilities take no predicate (a wave-uniform branch)
        const int kw0 = kb0 + 32 * wave;
        const bool plain = kw0 + 32 <= N && qc0 + kChunk <= N && (!a.causal || qc0 >= kw0 + 31);
#pragma unroll
        for (int u = 0; u < kSub; ++u) {
            float p[16], ds[16];
            if (plain) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    p[r] = exp2_hw(__builtin_fmaf(sc[u][r], a.scale_log2, -s_l[32 * u + acc_row(r, h)]));
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int qr = 32 * u + acc_row(r, h);
                    const int qi = qc0 + qr;
                    const bool ok = key < N && qi < N && (!a.causal || key <= qi);
                    const float e = exp2_hw(__builtin_fmaf(sc[u][r], a.scale_log2, -s_l[qr]));
                    p[r] = ok ? e : 0.f;
                }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) ds[r] = p[r] * (dp[u][r] - s_d[32 * u + acc_row(r, h)]);
            // dV^T += dO^T P and dK^T += Q^T dS (K-dim = the sub-chunk's queries)
            const lds_cptr tq = lq + 32 * u * S::kRow, tdo = ldo + 32 * u * S::kRow;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const bf16x8 pb = acc_operand(p, t), sb = acc_operand(ds, t);
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    acc_dv[db] = mfma_32x32x16(trans_frag<D>(tdo, lane, t, db), pb, acc_dv[db]);
                    acc_dk[db] = mfma_32x32x16(trans_frag<D>(tq, lane, t, db), sb, acc_dk[db]);
                }
            }
        }
        if (it + 1 < total) store_chunk((it + 1) & 1);
        __syncthreads();
    }
    // accumulator register r of block db: head dimension 32 db + 8 (r / 4) + 4 h + r % 4
    if (key < N) {
        uint16_t* pk = a.dk + kvoff + (size_t)key * D;
        uint16_t* pv = a.dv + kvoff + (size_t)key * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int d0 = 32 * db + 8 * gq + 4 * h;
                u32x2 wk = {pack_bf16x2(a.scale * acc_dk[db][4 * gq], a.scale * acc_dk[db][4 * gq + 1]),
                            pack_bf16x2(a.scale * acc_dk[db][4 * gq + 2], a.scale * acc_dk[db][4 * gq + 3])};
                u32x2 wv = {pack_bf16x2(acc_dv[db][4 * gq], acc_dv[db][4 * gq + 1]),
                            pack_bf16x2(acc_dv[db][4 * gq + 2], acc_dv[db][4 * gq + 3])};
                *reinterpret_cast<u32x2*>(pk + d0) = wk;
                *reinterpret_cast<u32x2*>(pv + d0) = wv;
            }
    }
}

// ---- dQ: workgroup = 128 queries of one query head; wave = 32 queries ----
template <int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(BwdArgs a) {
    constexpr int kSub = kSubQ;
    using S = Stage<D, kSub>;
    constexpr int kChunk = S::kChunk;
    // two buffers, each: K chunk, V chunk
    __shared__ __attribute__((aligned(16))) unsigned char smem[4 * S::kTile];

    const int N = a.N, G = a.Hq / a.Hkv;
    const int pos = xcd_position(gridDim.x * gridDim.y);
    const int bh = pos / gridDim.x;  // b * Hq + hq
    const int b = bh / a.Hq, hq = bh - b * a.Hq;
    const int kvh = hq / G;
    // last query block first: under the causal mask it sees the most keys
    const int qb0 = (gridDim.x - 1 - (pos - bh * gridDim.x)) * kBlock;
    const int lane = threadIdx.x & 63, h = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int query = qb0 + 32 * wave + (lane & 31);  // this lane's query (accumulator column)

    const size_t qoff = (size_t)bh * N;
    const size_t kvoff = ((size_t)b * a.Hkv + kvh) * N * D;
    bf16x8 qf[D / 16], dof[D / 16];
    {
        const int qr = min_(query, N - 1);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            qf[kk] = *reinterpret_cast<const bf16x8*>(a.q + (qoff + qr) * D + 16 * kk + 8 * h);
            dof[kk] = *reinterpret_cast<const bf16x8*>(a.dout + (qoff + qr) * D + 16 * kk + 8 * h);
        }
    }
    const float lse = query < N ? a.lse2[qoff + query] : INFINITY;
    const float dsum = query < N ? a.dsum[qoff + query] : 0.f;
    f32x16 acc_dq[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) acc_dq[i] = f32x16{};

    const int k_end = a.causal ? min_(N, qb0 + kBlock) : N;  // keys past the block's last query
    const int total = (k_end + kChunk - 1) / kChunk;
    // K and V chunks go straight into LDS (two buffers, each: K chunk, V chunk)
    TileDma<D, kSub> dma;
    dma.init(wave, lane);
    const unsigned lds_base = (unsigned)(size_t)(lds_cptr)smem;
    const int head_bytes = N * D * 2;
    const __amdgpu_buffer_rsrc_t rsk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + kvoff), (short)0, head_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rsv =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.v + kvoff), (short)0, head_bytes, kRsrcWord3);
    auto load_chunk = [&](int it) {
        const unsigned row0 = (unsigned)(it * kChunk * S::kRow);
        const unsigned tile = lds_base + (unsigned)(2 * (it & 1) * S::kTile);
        dma.issue(rsk, row0, tile, wave);
        dma.issue(rsv, row0, tile + (unsigned)S::kTile, wave);
    };
    auto store_chunk = [&](int) { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
    if (total > 0) {
        load_chunk(0);
        store_chunk(0);
    }
    __syncthreads();
    for (int it = 0; it < total; ++it) {
        // the other buffer was last read before the previous barrier
        if (it + 1 < total) load_chunk(it + 1);  // in flight during this chunk's products
        const int kc0 = it * kChunk;
        lds_cptr const lk = (lds_cptr)(smem + 2 * (it & 1) * S::kTile);
        lds_cptr const lv = (lds_cptr)(smem + (2 * (it & 1) + 1) * S::kTile);

        // S^T = K Q^T and dP^T = V dO^T: each 32-key sub-chunk x the wave's 32 queries
        f32x16 sc[kSub], dp[kSub];
#pragma unroll
        for (int u = 0; u < kSub; ++u) {
            sc[u] = f32x16{};
            dp[u] = f32x16{};
            const lds_cptr tk = lk + 32 * u * S::kRow, tv = lv + 32 * u * S::kRow;
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                sc[u] = mfma_32x32x16(rows_frag<D>(tk, lane, kk), qf[kk], sc[u]);
                dp[u] = mfma_32x32x16(rows_frag<D>(tv, lane, kk), dof[kk], dp[u]);
            }
        }
        // No score of this chunk is masked when the wave's 32 queries and the chunk's keys all
        // lie inside the sequence and (causal) the chunk's last key precedes the wave's first
        // query; then the probabilities take no predicate (a wave-uniform branch)
        const int qw0 = qb0 + 32 * wave;
        const bool plain = qw0 + 32 <= N && kc0 + kChunk <= N && (!a.causal || kc0 + kChunk - 1 <= qw0);
#pragma unroll
        for (int u = 0; u < kSub; ++u) {
            float ds[16];
            if (plain) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    ds[r] = exp2_hw(__builtin_fmaf(sc[u][r], a.scale_log2, -lse)) * (dp[u][r] - dsum);
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int kj = kc0 + 32 * u + acc_row(r, h);
                    const bool ok = kj < N && query < N && (!a.causal || kj <= query);
                    const float e = exp2_hw(__builtin_fmaf(sc[u][r], a.scale_log2, -lse));
                    ds[r] = (ok ? e : 0.f) * (dp[u][r] - dsum);
                }
            }
            // dQ^T += K^T dS^T (K-dim = the sub-chunk's keys)
            const lds_cptr tk = lk + 32 * u * S::kRow;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const bf16x8 sb = acc_operand(ds, t);
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
                    acc_dq[db] = mfma_32x32x16(trans_frag<D>(tk, lane, t, db), sb, acc_dq[db]);
            }
        }
        if (it + 1 < total) store_chunk((it + 1) & 1);
        __syncthreads();
    }
    if (query < N) {
        uint16_t* pq = a.dq + (qoff + query) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int d0 = 32 * db + 8 * gq + 4 * h;
                u32x2 w = {pack_bf16x2(a.scale * acc_dq[db][4 * gq], a.scale * acc_dq[db][4 * gq + 1]),
                           pack_bf16x2(a.scale * acc_dq[db][4 * gq + 2], a.scale * acc_dq[db][4 * gq + 3])};
                *reinterpret_cast<u32x2*>(pq + d0) = w;
            }
    }
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, const uint16_t* o, const float* m, const float* l,
                        float* lse2, float* dsum, int B, hipStream_t stream) {
    const long long rows = (long long)B * a.Hq * a.N;
    hipLaunchKernelGGL(bwd_prep_kernel<D>, dim3((unsigned)((rows + 63) / 64)), dim3(kThreads), 0,
                       stream, o, a.dout, m, l, lse2, dsum, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned blocks = (unsigned)((a.N + kBlock - 1) / kBlock);
    hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3(blocks, (unsigned)(B * a.Hkv)), dim3(kThreads), 0,
                       stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3(blocks, (unsigned)(B * a.Hq)), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* m, const float* l, void* dq, void* dk,
                           void* dv, int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                           float* lse2, float* dsum, hipStream_t stream) {
    BwdArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.dout = static_cast<const uint16_t*>(dout);
    a.lse2 = lse2;
    a.dsum = dsum;
    a.dq = static_cast<uint16_t*>(dq);
    a.dk = static_cast<uint16_t*>(dk);
    a.dv = static_cast<uint16_t*>(dv);
    a.Hq = Hq, a.Hkv = Hkv, a.N = N;
    a.scale = scale;
    a.scale_log2 = scale * kLog2e;
    a.causal = causal;
    const uint16_t* op = static_cast<const uint16_t*>(o);
    return d == 128 ? launch_bwd_d<128>(a, op, m, l, lse2, dsum, B, stream)
                    : launch_bwd_d<64>(a, op, m, l, lse2, dsum, B, stream);
}

}  // namespace fa
