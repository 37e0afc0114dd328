// bwd_bf16.hip - attention backward by recomputation, bf16 in / bf16 out, fp32 accumulation.
//
// Method: "FlashAttention, explained." (vibeengines.com), the backward-pass section: nothing of
// size N x N is stored by the forward; the backward recomputes the probabilities tile by tile
// from Q, K and the saved row statistics, P = exp(s - m) / l, and uses D_i = rowsum(dO_i * O_i)
// so that dS = P * (dP - D) needs no second pass over the keys. With dP = dO V^T:
//     dV = P^T dO,   dK = scale dS^T Q,   dQ = scale dS K.
//
// Two kernels, dQ first:
//  * bwd_dq: one workgroup per (128-query block, query head); each wave keeps its 32 queries'
//    Q and dO in registers, computes their D_i and log2-domain normaliser
//    L_i = (m_i + ln l_i) log2 e, so that P = exp2(scale log2e q.k - L) (L = +inf for a row
//    with no key: P = 0), writes both for the next kernel and walks the key chunks (32 rows of
//    K and V in LDS).
//  * bwd_dkdv: one workgroup per (128-key block, KV head); each wave keeps its 32 keys' K and V
//    in registers and walks the query chunks (32 rows of Q and dO staged in LDS, with their L
//    and D) of every query head of the KV group, accumulating dV^T and dK^T.
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
typedef const __attribute__((address_space(3))) f32x4 lds_f32x4;
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
    // instruction j of this wave's share: rows from byte row0 of the buffer r into the tile at
    // LDS address lds_tile
    __device__ __forceinline__ void issue_one(__amdgpu_buffer_rsrc_t r, unsigned row0, unsigned lds_tile,
                                              int wave, int j) const {
        asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                     :
                     : "v"(row0 + off[j]), "s"(r),
                       "{m0}"(lds_tile + 1024u * (unsigned)(wave * kPerWave + j))
                     : "memory");
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

// The same reads from lane offsets computed once: the byte offsets, from the LDS base, of this
// lane's row reads (per K-dim chunk kk) and transposing reads (two per head-dim block db) in a
// tile at byte `base`. They are held opaque to the compiler, so each read of a tile at base +
// an immediate is one register plus that immediate, not an address recomputed per read.
template <int D>
struct LaneOffsets {
    unsigned ro[D / 16];
    unsigned tr[D / 32][2];
    __device__ __forceinline__ void init(int lane, unsigned base) {
        constexpr int R = Stage<D, 1>::kRow;
        const int rr = kappa(lane & 31);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            ro[kk] = base + (unsigned)(rr * R + 16 * ((2 * kk + (lane >> 5)) ^ swz<D>(rr)));
            asm volatile("" : "+v"(ro[kk]));
        }
        const int r = 8 * (lane >> 5) + ((lane & 15) >> 2);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const int c = 4 * db + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
            tr[db][0] = base + (unsigned)(8 * (lane & 1) + r * R + 16 * (c ^ swz<D>(r)));
            tr[db][1] = base + (unsigned)(8 * (lane & 1) + (r + 4) * R + 16 * (c ^ swz<D>(r + 4)));
            asm volatile("" : "+v"(tr[db][0]), "+v"(tr[db][1]));
        }
    }
    // rows_frag of the tile `at` bytes past `base`
    __device__ __forceinline__ bf16x8 rows(lds_cptr lds, int at, int kk) const {
        return *reinterpret_cast<const lds_bf16x8*>(lds + ro[kk] + at);
    }
    // trans_frag of the tile `at` bytes past `base`
    __device__ __forceinline__ bf16x8 trans(lds_cptr lds, int at, int t, int db) const {
        constexpr int R = Stage<D, 1>::kRow;
        const int o = at + 16 * t * R;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds + tr[db][0] + o));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds + tr[db][1] + o));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
};

// The products of the dK, dV loop, written out so that each keeps the register file it needs:
// S and dP in VGPRs, which the vector work reads directly, the dK and dV accumulators in
// AGPRs, which only the products touch. The compiler does not know these for matrix
// instructions and adds no wait states around them: every read of a product's result stands
// a product and a dozen instructions or more after it (in the loop, a step later; before the
// epilogue's reads an explicit wait), and the A operands come from LDS reads whose counter
// waits the compiler places as for any instruction that reads the registers.
__device__ __forceinline__ void mma_v0(f32x16& d, bf16x8 a, bf16x8 b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mma_v(f32x16& d, bf16x8 a, bf16x8 b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mma_a(f32x16& d, bf16x8 a, bf16x8 b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}

// Accumulator registers 8 t .. 8 t + 7, rounded to bf16: the B operand (K-dim rows 16 t ..).
__device__ __forceinline__ bf16x8 acc_operand(const float (&x)[16], int t) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(x[8 * t + 2 * i], x[8 * t + 2 * i + 1]);
    return __builtin_bit_cast(bf16x8, w);
}

// A wave's 32 output rows, from 32 x 32 accumulators (lane (r, h), register 4 g + i of block db:
// row r, column 32 db + 8 g + 4 h + i) times s, rounded to bf16 and stored whole through LDS:
// the wave writes them row-major into its own block blk (32 rows of 2 D bytes; chunk c of row r
// at c ^ (r mod 16), d = 128, or c ^ (r / 2 mod 8), d = 64: conflict-free both ways), reads
// back 16 contiguous bytes a lane and stores rows 0 .. n_valid - 1 at dst, so that one store
// instruction covers 1 KiB of the output (the accumulator layout gives a lane 8 bytes in each
// of 16 places).
template <int D>
__device__ __forceinline__ void store_rows(const f32x16 (&acc)[D / 32], float s,
                                           __attribute__((address_space(3))) unsigned char* blk,
                                           uint16_t* dst, int n_valid, int lane) {
    typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
    typedef const __attribute__((address_space(3))) u32x4 lds_u32x4;
    constexpr int kRowB = 2 * D, kCh = kRowB / 16, kRowsPer = 1024 / kRowB;
    auto sw = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };
    const int r0 = lane & 31, h = lane >> 5, s0 = sw(r0);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            u32x2 w = {pack_bf16x2(s * acc[db][4 * g], s * acc[db][4 * g + 1]),
                       pack_bf16x2(s * acc[db][4 * g + 2], s * acc[db][4 * g + 3])};
            *(lds_u32x2*)(blk + r0 * kRowB + 16 * ((4 * db + g) ^ s0) + 8 * h) = w;
        }
    // (a wave's LDS accesses complete in order: its reads below see all its lanes' writes)
    __builtin_amdgcn_wave_barrier();
    const int rr = lane / kCh, ch = lane % kCh;
#pragma unroll
    for (int i = 0; i < 32 / kRowsPer; ++i) {
        const int r = kRowsPer * i + rr;
        const u32x4 v = *(lds_u32x4*)(blk + r * kRowB + 16 * (ch ^ sw(r)));
        if (r < n_valid) *reinterpret_cast<u32x4*>(dst + (size_t)r * D + 8 * ch) = v;
    }
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

// ---- D_i = rowsum(dO * O) and L_i = (m_i + ln l_i) log2 e ----
// Layout of L and D (written by the dQ kernel, read by the dK/dV kernel): per head, per 32-row
// chunk, the chunk's 32 L values then its 32 D values (256 bytes), so that one 4-byte-per-lane
// load moves a chunk's L and D together. A head's rows are padded to a multiple of 32; padding
// rows get L = +inf, D = 0 (P = 0 there).
constexpr int kLdChunk = 32;
__host__ __device__ constexpr long long ld_rows(int N) { return ((long long)N + kLdChunk - 1) / kLdChunk * kLdChunk; }
__device__ __forceinline__ long long ld_index(long long head, int N, int row) {
    return head * 2 * ld_rows(N) + (long long)(row / kLdChunk) * (2 * kLdChunk) + row % kLdChunk;
}

struct BwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* dout;
    const uint16_t* o;  // the forward's output and row statistics (natural-log units)
    const float* m;
    const float* l;
    float* ld;          // L and D of every query row, in 32-row chunks (see ld_index)
    uint16_t* dq;
    uint16_t* dk;
    uint16_t* dv;
    int Hq, Hkv, N;
    float scale, scale_log2;
    int causal;
};

// ---- dK, dV: workgroup = 128 keys of one KV head; wave = 32 keys; one wave per SIMD ----
// Each wave keeps its 32 keys' K and V rows in registers as B operands and walks 32-query
// chunks of every query head of the KV group. The walk is software-pipelined: the step of
// chunk c runs S = Q K^T and dP = dO V^T of chunk c + 1 (16 products, Q and dO rows read from
// LDS), dV^T += dO^T P and dK^T += Q^T dS of chunk c - 1 (16 products, dO^T and Q^T through
// transposing LDS reads, P and dS of that chunk as B operands), and between them the vector
// work of chunk c (P = exp2(s scale log2e - L), dS = P (dP - D), both rounded to bf16 as the
// B operands of the next step). With one wave per SIMD the wave has the whole register file:
// the accumulators live in AGPRs and K, V and two chunks of scores fit beside them.
// Chunks stream through a ring of kRing LDS stages (Q rows, dO rows, L and D), each loaded
// straight from global memory kAhead chunks before its first use; one barrier per step. The
// loop is unrolled over the ring, so every LDS address is a loop-invariant lane offset plus
// an immediate; the walk is padded to a whole number of rounds with chunks whose loads lie
// past every buffer and fill zeros (zero Q and dO rows contribute nothing), and a zero chunk
// stands before the first one.
// Query chunks are walked from the last one down: the workgroups of one head, started
// together, read the same chunks at about the same time and find them in L2.
template <int D>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(BwdArgs a) {
    using S = Stage<D, 1>;
    using Dma = TileDma<D, 1>;
    constexpr int kChunk = S::kChunk;
    constexpr int kT = S::kTile;                          // bytes of a chunk's Q (or dO) rows
    constexpr int kRing = 6;
    constexpr int kAhead = kRing - 2;                     // chunks c - 1 .. c + 1 are in use
    constexpr int kOps = 2 * Dma::kPerWave + 1;           // loads per wave and chunk
    constexpr int kA = 3;                                 // LDS operand reads kept in flight
    constexpr int kLdB = 2 * kChunk * 4;                  // L and D of a chunk's rows
    // the ring: the L and D of every stage, then the Q rows of every stage, then the dO rows;
    // each region spans less than the 64 KiB that an LDS instruction's immediate offset
    // reaches from one lane offset
    constexpr int kQ0 = kRing * kLdB, kDo0 = kQ0 + kRing * kT;
    auto ld_at = [](int st) { return st * kLdB; };
    // The workgroup's K and V rows come in through LDS (whole 1 KiB loads), each wave's 32 K
    // rows and 32 V rows in blocks of kKV bytes past the ring; where the LDS runs out, the
    // last block sits in stage 4's Q rows, first loaded after the prologue's barrier.
    constexpr int kKV = 32 * 2 * D, kRingEnd = kDo0 + kRing * kT;
    constexpr int kKVInRing = kRingEnd + 8 * kKV <= 160 * 1024 ? 0 : 1;
    static_assert(kKVInRing == 0 || (kKV == kT && kRing > kAhead + 1), "a block fits stage 4's Q rows");
    auto kv_block = [](int blk) {  // blocks 0 .. 3: K of waves 0 .. 3; 4 .. 7: V
        return blk < 8 - kKVInRing ? kRingEnd + blk * kKV : kQ0 + kAhead * kT;
    };
    __shared__ __attribute__((aligned(16))) unsigned char smem[kRingEnd + (8 - kKVInRing) * kKV];

    const int N = a.N, G = a.Hq / a.Hkv;
    const int pos = xcd_position(gridDim.x * gridDim.y);
    const int bk = pos / gridDim.x;  // b * Hkv + kvh
    const int b = bk / a.Hkv, kvh = bk - b * a.Hkv;
    const int kb0 = (pos - bk * gridDim.x) * kBlock;  // (causal: the first blocks see the most queries)
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, h = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int key = kb0 + 32 * wave + (lane & 31);  // this lane's key (accumulator column)
    const int kw0 = kb0 + 32 * wave;

    // K and V of the lane's key as B operands (K-dim = head dimension 16 kk + 8 h ..), read
    // from the wave's LDS blocks after the prologue's wait: chunk c of row r stored at chunk
    // c ^ (r mod 16) (d = 128) or c ^ (r / 2 mod 8) (d = 64); rows past N read zero
    const size_t kvoff = (size_t)bk * N * D;
    bf16x8 kf[D / 16], vf[D / 16];
    auto kv_sw = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };
    {
        const unsigned base = (unsigned)(size_t)(lds_cptr)smem;
        const __amdgpu_buffer_rsrc_t rk =
            __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + kvoff), (short)0, N * D * 2, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc((void*)(a.v + kvoff), (short)0, N * D * 2, kRsrcWord3);
#pragma unroll
        for (int i = 0; i < kKV / 1024; ++i) {
            const int slot = 1024 * i + 16 * lane;
            const int r = slot / (2 * D), cs = (slot % (2 * D)) / 16;
            const unsigned src = unsigned((kw0 + r) * 2 * D + 16 * (cs ^ kv_sw(r)));
            asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                         :
                         : "v"(src), "s"(rk), "{m0}"(base + (unsigned)kv_block(wave) + 1024u * i)
                         : "memory");
            asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                         :
                         : "v"(src), "s"(rv), "{m0}"(base + (unsigned)kv_block(4 + wave) + 1024u * i)
                         : "memory");
        }
    }
    f32x16 acc_dk[D / 32], acc_dv[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) acc_dk[i] = acc_dv[i] = f32x16{};

    // causal: queries before the block's first key see none of its keys. Chunk it = g nch + j
    // of the walk is query head kvh G + g, rows qtop - 32 j ..; chunks from `total` on (and
    // chunk -1) are zero chunks.
    const int q_first = a.causal ? (kb0 / kChunk) * kChunk : 0;
    const int nch = (N - q_first + kChunk - 1) / kChunk;
    const int qtop = q_first + (nch - 1) * kChunk;
    const int total = G * nch;
    const int rounds = (total + kRing - 1) / kRing;
    constexpr int R = S::kRow;
    Dma dma;
    dma.init(wave, lane);
    const unsigned lds_base = (unsigned)(size_t)(lds_cptr)smem;
    const int head_bytes = N * D * 2;
    const int ld_bytes = (int)(ld_rows(N) * 8);
    // The loads of one chunk: this wave's share of its Q and dO rows (kPerWave instructions
    // each) and the chunk's L and D (256 bytes, one dword per lane; every wave loads the same
    // bytes, so each wave issues kOps loads per chunk and one vmcnt count serves all). A chunk
    // past the walk (or before it) reads from past every range and fills zeros.
    struct Heads {  // the buffers of one query head: Q rows, dO rows, L and D
        __amdgpu_buffer_rsrc_t rq, rdo, rld;
    };
    struct Loads {
        Heads hd;
        unsigned row0, ldo, st;
    };
    const size_t hq0 = (size_t)b * a.Hq + (size_t)kvh * G;  // the group's first query head
    auto head_buffers = [&](int g) -> Heads {
        const size_t hq = hq0 + (size_t)g;
        Heads r;
        r.rq = __builtin_amdgcn_make_buffer_rsrc((void*)(a.q + hq * N * D), (short)0, head_bytes, kRsrcWord3);
        r.rdo = __builtin_amdgcn_make_buffer_rsrc((void*)(a.dout + hq * N * D), (short)0, head_bytes, kRsrcWord3);
        r.rld = __builtin_amdgcn_make_buffer_rsrc((void*)(a.ld + hq * 2 * ld_rows(N)), (short)0, ld_bytes,
                                                  kRsrcWord3);
        return r;
    };
    // chunk cursors (wave-uniform), kept incrementally so that a step spends a few scalar
    // instructions on them: the next chunk to load as (walk index, query head, byte offsets
    // of its rows and of its L and D in that head, the head's buffers, rebuilt only when the
    // walk moves on to the next head), and the walk index and first query row of the next
    // step's chunk
    const unsigned row_top = (unsigned)qtop * R, row_first = (unsigned)q_first * R;
    int ld_it = 0, ld_g = 0, st_it = 0, st_q = qtop;
    unsigned ld_row = row_top, ld_ldo = (unsigned)qtop * 8u;
    Heads ld_h = head_buffers(0);
    // the loads of the next chunk into stage st; advance_load() moves on after its last load
    auto load_of = [&](int st) -> Loads {
        const bool real = ld_it < total;
        return Loads{ld_h, real ? ld_row : 0x80000000u, real ? ld_ldo : 0x80000000u, (unsigned)st};
    };
    auto advance_load = [&]() {
        ++ld_it;
        if (ld_row == row_first) {
            ld_row = row_top;
            ld_ldo = (unsigned)qtop * 8u;
            if (++ld_g < G) ld_h = head_buffers(ld_g);
        } else {
            ld_row -= (unsigned)(kChunk * R);
            ld_ldo -= (unsigned)(kChunk * 8);
        }
    };
    auto next_load = [&](int st) -> Loads {
        const Loads l = load_of(st);
        advance_load();
        return l;
    };
    // load k (0 .. kOps - 1) of a chunk
    auto issue_op = [&](const Loads& l, int k) {
        constexpr int P = Dma::kPerWave;
        if (k < P) {
            dma.issue_one(l.hd.rq, l.row0, lds_base + (unsigned)kQ0 + l.st * (unsigned)kT, wave, k);
        } else if (k < 2 * P) {
            dma.issue_one(l.hd.rdo, l.row0, lds_base + (unsigned)kDo0 + l.st * (unsigned)kT, wave, k - P);
        } else {
            asm volatile("buffer_load_dword %0, %1, 0 offen lds"
                         :
                         : "v"(l.ldo + 4u * (unsigned)lane), "s"(l.hd.rld),
                           "{m0}"(lds_base + l.st * (unsigned)kLdB)
                         : "memory");
        }
    };
    auto issue_all = [&](const Loads& l) {
#pragma unroll
        for (int k = 0; k < kOps; ++k) issue_op(l, k);
    };
    const lds_cptr lds = (lds_cptr)smem;
    LaneOffsets<D> oq, odo;  // the Q and the dO region
    oq.init(lane, kQ0);
    odo.init(lane, kDo0);

    // products of slot sl of a step: the first half S / dP of the next chunk (S in even
    // slots, head dims 16 (sl / 2) ..), the second half dV / dK of the previous chunk (query
    // group t, head-dim block db), so that the next step's first reads of the scores come
    // kSlots / 2 products after the last one that wrote them (products that depend on the one
    // just before run at full rate)
    constexpr int kSlots = 2 * (D / 8);  // 16 next-chunk products + 16 previous-chunk ones (D = 128)
    constexpr int kPrev = D / 8;         // previous-chunk products: 2 (t) x D / 32 (db) x 2 (dV, dK)
    static_assert(kSlots == 2 * kPrev, "as many previous-chunk products as next-chunk ones");
    constexpr int kSpread = kSlots / 16; // slots per score of the vector work

    // One step: chunk it's vector work (its scores sc_c, dp_c -> operands pb_c, sb_c), the next
    // chunk's scores into (sc_n, dp_n) and the previous chunk's gradient products with pb_p,
    // sb_p; the loads `ld` of a later chunk go out one at a time between the products.
    // st_c: chunk it's ring stage.
    auto step = [&](auto st_c, f32x16& sc_c, f32x16& dp_c, f32x16& sc_n, f32x16& dp_n,
                    const bf16x8 (&pb_p)[2], const bf16x8 (&sb_p)[2], bf16x8 (&pb_c)[2],
                    bf16x8 (&sb_c)[2], int st_load) {
        constexpr int Pc = decltype(st_c)::value;
        constexpr int Pn = (Pc + 1) % kRing, Pp = (Pc + kRing - 1) % kRing;
        const lds_cptr s_l = lds + ld_at(Pc), s_d = s_l + 4 * kChunk;  // L, D
        // keys past the query get the score -inf where the chunk reaches above the wave's keys
        // (causal; a wave-uniform branch, rare: zero chunks and most chunks need none)
        if (a.causal && st_it < total && st_q < kw0 + 31) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sc_c[r] = key <= st_q + acc_row(r, h) ? sc_c[r] : -INFINITY;
        }
        ++st_it;
        st_q = st_q == q_first ? qtop : st_q - kChunk;
        // L and D of register r's row acc_row(r, h): element r % 4 of the 16-byte run at row
        // 16 (r / 8) + 8 h + 4 ((r / 4) % 2)
        auto ld4 = [&](lds_cptr base, int r) -> f32x4 {
            const int row = 16 * (r >> 3) + 8 * h + 4 * ((r >> 2) & 1);
            return *reinterpret_cast<const lds_f32x4*>(base + 4 * row);
        };
        auto operand = [&](int sl) -> bf16x8 {
            // next chunk: Q rows (S) and dO rows (dP); previous chunk: dO^T (dV) and Q^T (dK)
            const bool nx = sl < kSlots / 2;
            const int i = nx ? sl : sl - kSlots / 2;
            if (nx) return ((i & 1) ? odo : oq).rows(lds, Pn * kT, i >> 1);
            const int t = i / (kPrev / 2), db = (i >> 1) % (D / 32);
            return ((i & 1) ? oq : odo).trans(lds, Pp * kT, t, db);
        };
        bf16x8 op[kSlots];
        // The vector work of score r in three parts, pipelined over the slots so that each
        // slot's instructions take about as long to issue as its product takes to run (one
        // wave per SIMD issues in order: work beyond that delays the next product):
        //   A(r): the scores out of the accumulator registers, x = s scale log2e - L, u = dP - D
        //   B(r): p = exp2(x)
        //   C(r): dS = p u; pairs (r - 1, r) packed to bf16 in a later slot
        // With two slots per score (d = 128) slot 2 r holds A(r) and C(r - 1), slot 2 r + 1
        // holds B(r) and the pack of the pair before; with one slot per score (d = 64) a slot
        // does all of score r. The empty asm statements keep each part in its slot (without
        // them the compiler gathers the chunk's vector work ahead of the products).
        // L and D of registers 4 g .. 4 g + 3 are read four scores ahead of their first use.
        f32x4 lq = ld4(s_l, 0), dq4 = ld4(s_d, 0);   // L, D of registers 0 .. 3
        f32x4 lqn = ld4(s_l, 4), dqn = ld4(s_d, 4);  // of registers 4 .. 7
        float xs[16], us[16], ps[16], dss[16];
        auto part_a = [&](int r, float sr, float dpr) {
            if (r >= 4 && (r & 3) == 0) {
                lq = lqn;
                dq4 = dqn;
                if (r + 4 < 16) {
                    lqn = ld4(s_l, r + 4);
                    dqn = ld4(s_d, r + 4);
                }
            }
            xs[r] = __builtin_fmaf(sr, a.scale_log2, -lq[r & 3]);
            us[r] = dpr - dq4[r & 3];
            asm volatile("" : "+v"(xs[r]), "+v"(us[r]));
        };
        auto part_b = [&](int r) {
            ps[r] = exp2_hw(xs[r]);
            asm volatile("" : "+v"(ps[r]));
        };
        auto part_c = [&](int r) {
            dss[r] = ps[r] * us[r];
            asm volatile("" : "+v"(dss[r]));
        };
        // the pair (r - 1, r) into the operands
        auto pack = [&](int r) {
            const int w = (r >> 1) & 3, t = r >> 3;
            u32x4 pw = __builtin_bit_cast(u32x4, pb_c[t]);
            u32x4 sw = __builtin_bit_cast(u32x4, sb_c[t]);
            uint32_t wp = pack_bf16x2(ps[r - 1], ps[r]), wd = pack_bf16x2(dss[r - 1], dss[r]);
            asm volatile("" : "+v"(wp), "+v"(wd));  // packed here, not at their first use
            pw[w] = wp;
            sw[w] = wd;
            pb_c[t] = __builtin_bit_cast(bf16x8, pw);
            sb_c[t] = __builtin_bit_cast(bf16x8, sw);
        };
        Loads ld;  // the loads of this step's chunk kAhead ahead (set up after the first products)
#pragma unroll
        for (int sl = 0; sl < kA; ++sl) op[sl] = operand(sl);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int sl = 0; sl < kSlots; ++sl) {
            // A(r)'s scores, taken at the slot's start. Slot 0 reads what the step before wrote
            // in its slots kSlots / 2 - 2 and kSlots / 2 - 1, with kSlots / 2 products and their
            // vector work issued since: far more wait states than a matrix instruction's result
            // needs before a vector read (the prologue's products are padded explicitly).
            const bool has_a = kSpread == 1 || (sl & 1) == 0;
            const int r = sl / kSpread;
            float sr = 0.f, dpr = 0.f;
            if (has_a) {
                sr = sc_c[r];
                dpr = dp_c[r];
                asm volatile("" : "+v"(sr), "+v"(dpr));
            }
            if (sl + kA < kSlots) op[sl + kA] = operand(sl + kA);
            const int i = sl < kSlots / 2 ? sl : sl - kSlots / 2;
            if (sl < kSlots / 2) {
                f32x16& acc = (i & 1) ? dp_n : sc_n;
                const bf16x8 b = (i & 1) ? vf[i >> 1] : kf[i >> 1];
                if (i < 2) mma_v0(acc, op[sl], b);
                else mma_v(acc, op[sl], b);
            } else {
                const int t = i / (kPrev / 2), db = (i >> 1) % (D / 32);
                if ((i & 1) == 0) mma_a(acc_dv[db], op[sl], pb_p[t]);
                else mma_a(acc_dk[db], op[sl], sb_p[t]);
            }
            // the loads' descriptors in slot 1 (scalar work beside the products), load k in
            // slot 4 k + 2
            if (sl == 1) ld = load_of(st_load);
            if ((sl & 3) == 2 && (sl >> 2) < kOps) issue_op(ld, sl >> 2);
            if (sl == 4 * (kOps - 1) + 3) advance_load();
            if (kSpread == 1) {
                part_a(r, sr, dpr);
                part_b(r);
                part_c(r);
                if (r & 1) pack(r);
            } else if (has_a) {
                part_a(r, sr, dpr);
                if (r >= 1) part_c(r - 1);
            } else {
                part_b(r);
                if (r >= 2 && (r & 1) == 0) pack(r - 1);
                if (r == 15) {
                    part_c(15);
                    pack(15);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    static_assert(4 * (kOps - 1) + 2 < kSlots, "every load of a chunk has its slot");
    // before a step: wait for the next chunk (this wave's loads; the kAhead - 2 chunks after it
    // stay in flight), barrier; the step then loads the chunk kAhead ahead into stage st_load,
    // the one chunk it - 2 used
    auto advance = [&](int st_load) -> int {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kAhead - 2) * kOps) : "memory");
        __syncthreads();
        return st_load;
    };

    if (total > 0) {
        // prologue: the zero chunk -1 into stage kRing - 1, chunks 0 .. kAhead - 1 into stages
        // 0 .. kAhead - 1; wait for chunks -1 and 0; chunk 0's scores
        issue_all(Loads{ld_h, 0x80000000u, 0x80000000u, (unsigned)(kRing - 1)});
#pragma unroll
        for (int c = 0; c < kAhead; ++c) issue_all(next_load(c));
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kAhead - 1) * kOps) : "memory");
        {
            // the wave's K and V blocks have landed (issued before the chunks waited for)
            const int r0 = lane & 31;
            const lds_cptr bk_ = (lds_cptr)smem + kv_block(wave) + r0 * 2 * D;
            const lds_cptr bv_ = (lds_cptr)smem + kv_block(4 + wave) + r0 * 2 * D;
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                kf[kk] = *(const lds_bf16x8*)(bk_ + 16 * ((2 * kk + h) ^ kv_sw(r0)));
                vf[kk] = *(const lds_bf16x8*)(bv_ + 16 * ((2 * kk + h) ^ kv_sw(r0)));
            }
        }
        __syncthreads();
        f32x16 sa{}, da{}, sb2{}, db2{};
        const bf16x8 zero8 = {};
        bf16x8 pa[2] = {zero8, zero8}, qa[2] = {zero8, zero8};   // P, dS of even chunks
        bf16x8 pb[2] = {zero8, zero8}, qb[2] = {zero8, zero8};   // of odd chunks (and chunk -1)
        {
            mma_v0(sa, oq.rows(lds, 0, 0), kf[0]);
            mma_v0(da, odo.rows(lds, 0, 0), vf[0]);
#pragma unroll
            for (int kk = 1; kk < D / 16; ++kk) {
                mma_v(sa, oq.rows(lds, 0, kk), kf[kk]);
                mma_v(da, odo.rows(lds, 0, kk), vf[kk]);
            }
            // the wait states between these products and the first step's reads of their
            // results (the masking at its start, or its slot 0)
            asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
        }
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2>;
        using I3 = std::integral_constant<int, 3>;
        using I4 = std::integral_constant<int, 4>;
        using I5 = std::integral_constant<int, 5>;
        // rounds of kRing steps; step it's loads go to stage (it + kAhead) % kRing
        for (int rd = 0; rd < rounds; ++rd) {
            step(I0{}, sa, da, sb2, db2, pb, qb, pa, qa, advance(4));
            step(I1{}, sb2, db2, sa, da, pa, qa, pb, qb, advance(5));
            step(I2{}, sa, da, sb2, db2, pb, qb, pa, qa, advance(0));
            step(I3{}, sb2, db2, sa, da, pa, qa, pb, qb, advance(1));
            step(I4{}, sa, da, sb2, db2, pb, qb, pa, qa, advance(2));
            step(I5{}, sb2, db2, sa, da, pa, qa, pb, qb, advance(3));
        }
        // dV, dK of the last chunk of the walk (an odd chunk, in stage kRing - 1)
        {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    mma_a(acc_dv[db], odo.trans(lds, (kRing - 1) * kT, t, db), pb[t]);
                    mma_a(acc_dk[db], oq.trans(lds, (kRing - 1) * kT, t, db), qb[t]);
                }
        }
        // no load may still be writing LDS when the workgroup ends
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        // the wait states between the last products and the reads of their accumulators
        // (the accumulators pass through, so that no read moves ahead of the wait)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) asm volatile("" : "+a"(acc_dv[db]), "+a"(acc_dk[db]));
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
        for (int db = 0; db < D / 32; ++db) asm volatile("" : "+a"(acc_dv[db]), "+a"(acc_dk[db]));
    }
    // dK and dV rows through LDS (every wave is done with the ring after the barrier, and no
    // load is in flight, not even the K and V rows' without a walk): the wave's dK block, then
    // its dV block
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    {
        typedef __attribute__((address_space(3))) unsigned char* lds_ptr;
        lds_ptr const blk = (lds_ptr)smem + wave * 2 * 32 * 2 * D;
        store_rows<D>(acc_dk, a.scale, blk, a.dk + kvoff + (size_t)kw0 * D, N - kw0, lane);
        store_rows<D>(acc_dv, 1.f, blk + 32 * 2 * D, a.dv + kvoff + (size_t)kw0 * D, N - kw0, lane);
    }
}

// ---- dQ: workgroup = 128 queries of one query head; wave = 32 queries ----
// Each wave keeps its 32 queries' Q and dO rows in registers as B operands and walks 32-key
// chunks of K and V, software-pipelined like the dK/dV kernel: the step of chunk c runs
// S^T = K Q^T and dP^T = V dO^T of chunk c + 1 (16 products, K and V rows from LDS), dQ^T +=
// K^T dS^T of chunk c - 1 (8 products, K^T through transposing LDS reads) and the vector work
// of chunk c. K and V chunks stream through a ring of kRing LDS stages (K rows, then V rows),
// loaded kAhead chunks ahead, one load per few products; the loop is unrolled over the ring
// and the walk padded to whole rounds with zero chunks (zero K rows add nothing to dQ).
// Two waves per SIMD.
template <int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(BwdArgs a) {
    using S = Stage<D, 1>;
    using Dma = TileDma<D, 1>;
    constexpr int kChunk = S::kChunk;
    constexpr int kT = S::kTile;            // bytes of a chunk's K (or V) rows
    constexpr int kRing = 4;
    constexpr int kAhead = kRing - 2;       // chunks c - 1 and c + 1 are in use during step c
    constexpr int kOps = 2 * Dma::kPerWave; // loads per wave and chunk
    constexpr int kA = 3;                   // LDS operand reads kept in flight
    constexpr int kStB = 2 * kT;            // a stage: K rows, V rows
    __shared__ __attribute__((aligned(16))) unsigned char smem[kRing * kStB];

    const int N = a.N, G = a.Hq / a.Hkv;
    const int pos = xcd_position(gridDim.x * gridDim.y);
    const int bh = pos / gridDim.x;  // b * Hq + hq
    const int b = bh / a.Hq, hq = bh - b * a.Hq;
    const int kvh = hq / G;
    // last query block first: under the causal mask it sees the most keys
    const int qb0 = (gridDim.x - 1 - (pos - bh * gridDim.x)) * kBlock;
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, h = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int query = qb0 + 32 * wave + (lane & 31);  // this lane's query (accumulator column)
    const int qw0 = qb0 + 32 * wave;

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
    // L = (m + ln l) log2 e and D = dO . O of the lane's query, computed here and written to the
    // workspace for the dK/dV kernel, which runs after this one (a padding row, past N, gets
    // L = +inf and D = 0, so that its P is 0). The wave's 32 queries are one chunk of the
    // layout: lane q writes the chunk's L value q, lane 32 + q its D value q.
    float lse = INFINITY, dsum = 0.f;
    {
        const int qr = min_(query, N - 1);
        float part = 0.f;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            const u32x4 ov = *reinterpret_cast<const u32x4*>(a.o + (qoff + qr) * D + 16 * kk + 8 * h);
            const u32x4 dv = __builtin_bit_cast(u32x4, dof[kk]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                part = __builtin_fmaf(bf16_lo(ov[i]), bf16_lo(dv[i]), part);
                part = __builtin_fmaf(bf16_hi(ov[i]), bf16_hi(dv[i]), part);
            }
        }
        part += __shfl_xor(part, 32);  // the other half of the row's head dimensions
        if (query < N) {
            const float lr = a.l[qoff + query];
            lse = lr > 0.f ? (a.m[qoff + query] + logf(lr)) * kLog2e : INFINITY;
            dsum = part;
        }
        if (qw0 < N) a.ld[ld_index((long long)bh, N, qw0) + lane] = h == 0 ? lse : dsum;
    }
    f32x16 acc_dq[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) acc_dq[i] = f32x16{};

    const int k_end = a.causal ? min_(N, qb0 + kBlock) : N;  // keys past the block's last query
    const int total = (k_end + kChunk - 1) / kChunk;
    const int rounds = (total + kRing - 1) / kRing;
    Dma dma;
    dma.init(wave, lane);
    const unsigned lds_base = (unsigned)(size_t)(lds_cptr)smem;
    const int head_bytes = N * D * 2;
    const __amdgpu_buffer_rsrc_t rsk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + kvoff), (short)0, head_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rsv =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.v + kvoff), (short)0, head_bytes, kRsrcWord3);
    // load k (0 .. kOps - 1) of chunk it into stage st (a chunk past the walk, or before it,
    // reads from past the range and fills zeros)
    auto issue_op = [&](int it, int st, int k) {
        constexpr int P = Dma::kPerWave;
        const unsigned row0 = (it >= 0 && it < total) ? (unsigned)(it * kChunk * S::kRow) : 0x80000000u;
        const unsigned tile = lds_base + (unsigned)(st * kStB);
        if (k < P) dma.issue_one(rsk, row0, tile, wave, k);
        else dma.issue_one(rsv, row0, tile + (unsigned)kT, wave, k - P);
    };
    const lds_cptr lds = (lds_cptr)smem;

    // slots of a step: first the (S^T, dP^T) pairs of the next chunk (head dims 16 k ..),
    // then the dQ^T products k of the previous chunk (key group t = k / (D / 32), head-dim
    // block db), so that the next step's first reads of the scores come kDq products after
    // the last one that wrote them (products that depend on the one just before run at full
    // rate)
    constexpr int kNext = D / 16;                // S^T / dP^T pairs
    constexpr int kDq = 2 * (D / 32);            // dQ^T products: 2 (t) x D / 32 (db)
    static_assert(kNext == kDq, "one dQ product per (S, dP) pair");
    constexpr int kSlots = 3 * kNext;
    // product k and kind m (0: S^T, 1: dP^T, 2: dQ^T) of slot sl
    auto slot_k = [](int sl) { return sl < 2 * kNext ? sl >> 1 : sl - 2 * kNext; };
    auto slot_m = [](int sl) { return sl < 2 * kNext ? (sl & 1) : 2; };
    // vector work of score r in slot slot_of(r): spread over the step
    auto slot_of = [](int r) { return (r * kSlots) / 16; };
    static_assert((15 * kSlots) / 16 < kSlots, "every score has its slot");

    // One step: chunk it's vector work (scores sc_c, dp_c -> dS operands sb_c), the next
    // chunk's scores into (sc_n, dp_n), the previous chunk's dQ products with sb_p; loads of
    // chunk it + kAhead into stage st_load. st_c: chunk it's stage.
    auto step = [&](int it, auto st_c, f32x16& sc_c, f32x16& dp_c, f32x16& sc_n, f32x16& dp_n,
                    const bf16x8 (&sb_p)[2], bf16x8 (&sb_c)[2], int st_load) {
        constexpr int Pc = decltype(st_c)::value;
        constexpr int Pn = (Pc + 1) % kRing, Pp = (Pc + kRing - 1) % kRing;
        const lds_cptr tnk = lds + Pn * kStB, tnv = tnk + kT;  // next chunk's K, V rows
        const lds_cptr tpk = lds + Pp * kStB;                  // previous chunk's K rows
        // keys past the query get the score -inf where the chunk reaches past the wave's first
        // query (causal; a wave-uniform branch)
        const int kc0 = it * kChunk;
        if (a.causal && it < total && kc0 + kChunk - 1 > qw0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sc_c[r] = kc0 + acc_row(r, h) <= query ? sc_c[r] : -INFINITY;
        }
        auto operand = [&](int sl) -> bf16x8 {
            const int k = slot_k(sl), m = slot_m(sl);
            if (m == 0) return rows_frag<D>(tnk, lane, k);
            if (m == 1) return rows_frag<D>(tnv, lane, k);
            return trans_frag<D>(tpk, lane, k / (D / 32), k % (D / 32));
        };
        bf16x8 op[kSlots];
        float d0 = 0.f;  // the first dS of a pair
        sc_n = f32x16{};
        dp_n = f32x16{};
#pragma unroll
        for (int sl = 0; sl < kA; ++sl) op[sl] = operand(sl);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int sl = 0; sl < kSlots; ++sl) {
            if (sl + kA < kSlots) op[sl + kA] = operand(sl + kA);
            const int k = slot_k(sl), m = slot_m(sl);
            if (m == 0) sc_n = mfma_32x32x16(op[sl], qf[k], sc_n);
            else if (m == 1) dp_n = mfma_32x32x16(op[sl], dof[k], dp_n);
            else acc_dq[k % (D / 32)] = mfma_32x32x16(op[sl], sb_p[k / (D / 32)], acc_dq[k % (D / 32)]);
            // load k of the chunk kAhead ahead in slot 4 k + 1
            if ((sl & 3) == 1 && (sl >> 2) < kOps) issue_op(it + kAhead, st_load, sl >> 2);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if (slot_of(r) != sl) continue;
                // (the empty asm statements keep this work in its slot)
                float sr = sc_c[r], dpr = dp_c[r];
                asm volatile("" : "+v"(sr), "+v"(dpr));
                float dr = exp2_hw(__builtin_fmaf(sr, a.scale_log2, -lse)) * (dpr - dsum);
                asm volatile("" : "+v"(dr));
                if (r & 1) {
                    const int w = (r >> 1) & 3, t = r >> 3;
                    u32x4 sw = __builtin_bit_cast(u32x4, sb_c[t]);
                    sw[w] = pack_bf16x2(d0, dr);
                    sb_c[t] = __builtin_bit_cast(bf16x8, sw);
                } else {
                    d0 = dr;
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    static_assert(4 * (kOps - 1) + 1 < kSlots, "every load of a chunk has its slot");
    // before the step of chunk it: wait for chunk it + 1 (this wave's loads; the chunks after
    // it, kAhead - 2 of them, stay in flight), barrier
    auto advance = [&]() {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kAhead - 2) * kOps) : "memory");
        __syncthreads();
    };

    if (total > 0) {
        // prologue: the zero chunk -1 into stage kRing - 1, chunks 0 .. kAhead - 1 into stages
        // 0 .. kAhead - 1; wait for chunks -1 and 0; chunk 0's scores
#pragma unroll
        for (int k = 0; k < kOps; ++k) issue_op(-1, kRing - 1, k);
#pragma unroll
        for (int c = 0; c < kAhead; ++c)
#pragma unroll
            for (int k = 0; k < kOps; ++k) issue_op(c, c, k);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kAhead - 1) * kOps) : "memory");
        __syncthreads();
        f32x16 sa{}, da{}, sb2{}, db2{};
        const bf16x8 zero8 = {};
        bf16x8 qa[2] = {zero8, zero8}, qb[2] = {zero8, zero8};  // dS of even / odd chunks
        {
            const lds_cptr tk = lds, tv = lds + kT;
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                sa = mfma_32x32x16(rows_frag<D>(tk, lane, kk), qf[kk], sa);
                da = mfma_32x32x16(rows_frag<D>(tv, lane, kk), dof[kk], da);
            }
        }
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2>;
        using I3 = std::integral_constant<int, 3>;
        static_assert(kRing == 4, "the loop below is unrolled over a ring of four stages");
        for (int rd = 0; rd < rounds; ++rd) {
            const int it = rd * kRing;
            advance();
            step(it, I0{}, sa, da, sb2, db2, qb, qa, 2);
            advance();
            step(it + 1, I1{}, sb2, db2, sa, da, qa, qb, 3);
            advance();
            step(it + 2, I2{}, sa, da, sb2, db2, qb, qa, 0);
            advance();
            step(it + 3, I3{}, sb2, db2, sa, da, qa, qb, 1);
        }
        // dQ of the last chunk of the walk (an odd chunk, in stage kRing - 1)
        {
            const lds_cptr tk = lds + (kRing - 1) * kStB;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
                    acc_dq[db] = mfma_32x32x16(trans_frag<D>(tk, lane, t, db), qb[t], acc_dq[db]);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load may still be writing LDS
    }
    // dQ rows through LDS (every wave is done with the ring after the barrier)
    __syncthreads();
    {
        typedef __attribute__((address_space(3))) unsigned char* lds_ptr;
        store_rows<D>(acc_dq, a.scale, (lds_ptr)smem + wave * 32 * 2 * D, a.dq + (qoff + qw0) * D,
                      N - qw0, lane);
    }
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, int B, hipStream_t stream) {
    // dQ first: it writes the L and D rows that dK/dV reads
    const unsigned blocks = (unsigned)((a.N + kBlock - 1) / kBlock);
    hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3(blocks, (unsigned)(B * a.Hq)), dim3(kThreads), 0,
                       stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3(blocks, (unsigned)(B * a.Hkv)), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* m, const float* l, void* dq, void* dk,
                           void* dv, int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                           float* ld, hipStream_t stream) {
    BwdArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.dout = static_cast<const uint16_t*>(dout);
    a.o = static_cast<const uint16_t*>(o);
    a.m = m;
    a.l = l;
    a.ld = ld;
    a.dq = static_cast<uint16_t*>(dq);
    a.dk = static_cast<uint16_t*>(dk);
    a.dv = static_cast<uint16_t*>(dv);
    a.Hq = Hq, a.Hkv = Hkv, a.N = N;
    a.scale = scale;
    a.scale_log2 = scale * kLog2e;
    a.causal = causal;
    return d == 128 ? launch_bwd_d<128>(a, B, stream) : launch_bwd_d<64>(a, B, stream);
}

}  // namespace fa
