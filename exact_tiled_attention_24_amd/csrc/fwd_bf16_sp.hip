// fwd_bf16_sp.hip - tiled attention forward, bf16 in / bf16 out, software-pipelined so that
// every wave keeps the matrix cores and the vector ALUs busy at the same time.
//
// Method: "FlashAttention" (shubhamtatvamasi.com), "The trick: tiles and an online softmax":
// Q is split into row blocks and K/V into key blocks; each score block lives only on chip
// and is folded into a running row maximum, running sum and rescaled accumulator, and the
// output is O / l. Scheduling follows the FlashAttention-2 row of the family table on the
// same page (parallel over query blocks; normalise once at the end); causal tiles strictly
// above the workgroup's diagonal are never loaded.
//
// Schedule. A wave owns 32 query rows and walks the keys in 32-key half tiles h. Step h
// issues, in one basic block, the MFMAs of O^T += V^T P^T for half tile h-1 and of
// S^T = K Q^T for half tile h+1 (16 MFMAs, about 512 cycles) together with the vector work
// that turns the scores of half tile h into probabilities (about 90 instructions). The two
// streams are independent, so the SIMD runs them side by side; the scheduler is told to
// interleave them (one MFMA, one LDS operand read, a few vector instructions, repeated).
// Two such waves share each SIMD (8 waves, 256 query rows per workgroup), and each needs
// only about 16 bytes of LDS operand per cycle, half of what one wave can draw.
//
// CDNA4 details:
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: a lane holds the scores of one query row,
//    so row max and sum are in-lane plus one exchange with lane l ^ 32. The S^T
//    accumulator, converted to bf16, is directly the B operand of O^T += V^T P^T: the MFMA
//    reads K rows in an order that swaps bits 2 and 3 of the row index, so the
//    accumulator's register order is the key order the second MFMA needs.
//  * K is staged in LDS row-major, V transposed ([d][key]), rows padded by 16 bytes: on
//    gfx950's LDS (64 banks of 4 bytes) the MFMA operand reads and the staging writes are
//    conflict free, and every operand address is one per-lane base plus an immediate.
//  * Three LDS stages per operand: K and V of tile j+2 / j+1 are written while tiles j and
//    j+1 are being read, with one workgroup barrier per 64-key tile. Threads 0-255 move K,
//    256-511 move V (register-staged buffer loads, issued one tile ahead).
//  * Scores in the log2 domain; the exponent reference moves only when a row maximum beats
//    it by more than 2^8, so the O rescale (a branch after the MFMAs) is rare.
//  * Every wave runs every half tile of its workgroup (those past its own diagonal are
//    fully masked and contribute nothing), so all waves follow one branch-free schedule.
//  * Grid: one workgroup per (256-row query block, head), XCD-contiguous work order.
#include <type_traits>

#include "fa_internal.hpp"
#include "gfx950.hpp"

namespace fa {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBr = 32 * kWaves;  // query rows per workgroup
constexpr int kBc = 64;           // keys per tile (two 32-key half tiles)
constexpr int kStages = 3;
constexpr int kXcds = 8;
constexpr float kLazy = 8.f;
constexpr int kAhead = 5;         // LDS operand reads kept in flight
constexpr int kBufferDword3 = 0x00020000;

__device__ __forceinline__ int kappa(int m) {
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Workgroup barrier that orders LDS accesses only: global loads in flight stay in flight.
__device__ __forceinline__ void barrier_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int D>
struct Tile {
    static constexpr int kChunks = D / 8;                             // 16-byte chunks per K row
    static constexpr int kKRow = D * 2 + 16;                          // padded K row, bytes
    static constexpr int kVRow = kBc * 2 + 16;                        // padded V^T row, bytes
    static constexpr int kKBytes = kBc * kKRow;
    static constexpr int kVBytes = D * kVRow;
    static constexpr int kStageBytes = kKBytes + kVBytes;
    static constexpr int kKLoads = kBc * kChunks / kThreads;          // b128 K loads per thread
    static constexpr int kRowsPerLoad = kThreads / kChunks;
    static constexpr int kVKeys = kBc * (D / 4) / kThreads;           // V keys per thread
    static constexpr int kVGroups = kBc / kVKeys;                     // key groups per V tile
    static constexpr int kStageOps = kKLoads + 4 + 1;                 // see stage_op
};

template <int D>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_sp_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ m_out, float* __restrict__ l_out, int B, int Hq,
    int Hkv, int N, float scale_log2, int causal, int nqb) {
    using T = Tile<D>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[kStages * T::kStageBytes];

    // ---- work item: XCD-contiguous runs ordered (KV group, query block heaviest first,
    // head in group); see fwd_bf16.hip ----
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
    const int row0 = qb * kBr + 32 * wave;
    const int qrow = row0 + l32;

    bf16x8 qf[D / 16];
    {
        const uint16_t* src = qh + (size_t)min_(qrow, N - 1) * D + 8 * hh;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            qf[kk] = *reinterpret_cast<const bf16x8*>(src + 16 * kk);
    }
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) asm volatile("" : "+v"(qf[kk]));

    f32x16 acc_o[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) acc_o[i] = f32x16{};
    float m_run = -INFINITY, m_ref = -INFINITY, l_part = 0.f;

    const int kv_end = causal ? min_(N, qb * kBr + kBr) : N;
    const int n_tiles = (kv_end + kBc - 1) / kBc;

    // ---- staging: every thread moves kKLoads 16-byte chunks of each K tile and kVKeys keys
    // x 4 columns of each V tile (register-staged buffer loads, issued a tile ahead) ----
    u32x4 kreg[T::kKLoads];
    u32x2 vreg[T::kVKeys];
    const int k_gofs = ((tid / T::kChunks) * D + (tid % T::kChunks) * 8) * 2;
    const int k_lofs = (tid / T::kChunks) * T::kKRow + (tid % T::kChunks) * 16;
    // V: keys v_kg * kVKeys + i of columns 4 v_dq .. 4 v_dq + 3; the key group varies fastest
    // across lanes, so a transposed store of one column by consecutive lanes fills
    // consecutive bytes of one V^T row.
    const int v_kg = tid % T::kVGroups;
    const int v_dq = tid / T::kVGroups;
    const int v_gofs = (v_kg * T::kVKeys * D + v_dq * 4) * 2;
    const int v_lofs = T::kKBytes + (4 * v_dq) * T::kVRow + v_kg * T::kVKeys * 2;
    // Descriptor of tile j of one head's K or V (rows past N read as zero). The row count
    // goes through readfirstlane: the clamp selects to a vector instruction, and a
    // descriptor word in a VGPR would force a per-lane loop around every buffer load.
    auto tile_rsrc = [&](const uint16_t* base, int j) {
        const int kv0 = j * kBc;
        const int rows = __builtin_amdgcn_readfirstlane(max_(0, min_(N - kv0, kBc)));
        return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (size_t)min_(kv0, N) * D),
                                                 (short)0, rows * D * 2, kBufferDword3);
    };
    auto load_k = [&](int j) {
        const __amdgpu_buffer_rsrc_t r = tile_rsrc(kh, j);
#pragma unroll
        for (int i = 0; i < T::kKLoads; ++i)
            kreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    r, k_gofs + i * T::kRowsPerLoad * D * 2, 0, 0));
    };
    auto load_v = [&](int j) {
        const __amdgpu_buffer_rsrc_t r = tile_rsrc(vh, j);
#pragma unroll
        for (int i = 0; i < T::kVKeys; ++i)
            vreg[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, v_gofs + i * D * 2, 0, 0));
    };
    auto store_k_part = [&](int st, int i) {
        *reinterpret_cast<u32x4*>(smem + st * T::kStageBytes + k_lofs + i * T::kRowsPerLoad * T::kKRow) =
            kreg[i];
    };
    // column c of this thread's V keys, transposed: key pairs joined with one v_perm_b32 each
    auto store_v_col = [&](int st, int c) {
        const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
        uint32_t w[T::kVKeys / 2];
#pragma unroll
        for (int i = 0; i < T::kVKeys / 2; ++i)
            w[i] = __builtin_amdgcn_perm(vreg[2 * i + 1][c >> 1], vreg[2 * i][c >> 1], sel);
        unsigned char* dst = smem + st * T::kStageBytes + v_lofs + c * T::kVRow;
        if constexpr (T::kVKeys == 4) *reinterpret_cast<u32x2*>(dst) = u32x2{w[0], w[1]};
        else *reinterpret_cast<uint32_t*>(dst) = w[0];
    };
    // Staging of tile j's end, as kStageOps small operations that the pipelined step spreads
    // over its slots: K of tile j+2 and V of tile j+1 into their stages, then the loads of K
    // of tile j+3 and V of tile j+2 into the freed registers.
    auto stage_op = [&](int j, int op) {
        if (op < T::kKLoads) store_k_part((j + 2) % kStages, op);
        else if (op < T::kKLoads + 4) store_v_col((j + 1) % kStages, op - T::kKLoads);
        else {
            load_k(j + 3);
            load_v(j + 2);
        }
    };

    // Operand addresses: one per-lane base each, the rest immediate.
    const int k_rofs = kappa(l32) * T::kKRow + hh * 16;
    const int v_rofs = T::kKBytes + l32 * T::kVRow + hh * 16;

    // S^T = K Q^T of half tile (stage st, half kb) into s.
    auto compute_s = [&](f32x16& s, int st, int kb) {
        const unsigned char* ks = smem + st * T::kStageBytes + k_rofs + 32 * kb * T::kKRow;
        s = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(ks + 32 * kk);
            s = mfma_32x32x16(a, qf[kk], s);
        }
    };
    // O^T += V^T P^T of half tile (stage st, half kb) with probabilities pk.
    auto compute_pv = [&](const u32x4 (&pk)[2], int st, int kb) {
        const unsigned char* vs = smem + st * T::kStageBytes + v_rofs;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const bf16x8 pb = __builtin_bit_cast(bf16x8, pk[t]);
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                    vs + 32 * db * T::kVRow + (4 * kb + 2 * t) * 16);
                acc_o[db] = mfma_32x32x16(a, pb, acc_o[db]);
            }
        }
    };
    // Lazy O rescale, after the step's MFMAs (which added the previous half tile).
    auto rescale = [&](float alpha) {
        if (__any(alpha != 1.f)) {
#pragma unroll
            for (int i = 0; i < D / 32; ++i) acc_o[i] *= alpha;
        }
    };
    // MFMA operand of slot `sl` of step hi: even slots are the S^T MFMAs of half tile hi+1
    // (K, head dimensions 16 (sl/2) ..), odd slots the O MFMAs of half tile hi-1 (V^T, key
    // group t, head-dimension block db).
    auto frag = [&](int hi, int sl) -> bf16x8 {
        const int i = sl >> 1;
        if ((sl & 1) == 0) {
            const int st = ((hi + 1) >> 1) % kStages, kb = (hi + 1) & 1;
            return *reinterpret_cast<const bf16x8*>(smem + st * T::kStageBytes + k_rofs +
                                                    32 * kb * T::kKRow + 32 * i);
        }
        const int st = ((hi - 1) >> 1) % kStages, kb = (hi - 1) & 1;
        const int t = i / (D / 32), db = i % (D / 32);
        return *reinterpret_cast<const bf16x8*>(smem + st * T::kStageBytes + v_rofs + 4 * kb * 16 +
                                                32 * db * T::kVRow + 2 * t * 16);
    };

    // One pipeline step. Its MFMAs are O^T += V^T P^T of half tile hi-1 (probabilities
    // pk_prev) and S^T of half tile hi+1 (into s_next), taken alternately so consecutive MFMAs
    // are independent; beside them runs the softmax of half tile hi (s_cur -> pk_cur). The
    // step is written as kSlots slots, each one LDS operand read (kAhead slots ahead), one
    // MFMA and a slice of the softmax, with a scheduling barrier after every slot, so the
    // instruction order is the one written here. `fr` holds on entry the operands of this
    // step's first kAhead slots and on exit those of the next step's (read in this step's
    // last slots, so the next step starts without waiting, even across a barrier: its
    // operands were staged before the previous barrier).
    // (with_pv false: half tile 0, whose step has no O update; its odd slots stay empty.)
    // stage_j >= 0: this step also carries the staging of tile stage_j (stage_op 0, 1, ...
    // in its odd slots).
    auto step = [&](int hi, f32x16& s_cur, f32x16& s_next, const u32x4 (&pk_prev)[2],
                    u32x4 (&pk_cur)[2], auto masked, bf16x8 (&fr)[kAhead], auto with_pv,
                    int stage_j) {
        constexpr bool kPV = decltype(with_pv)::value;
        constexpr int kS = D / 16;             // S^T MFMAs (one per 16 head dimensions)
        constexpr int kSlots = 2 * kS;         // as many O MFMAs: 2 key groups x D/32 blocks
        constexpr int kPhasesPerSlot = 16 / kSlots;
        static_assert(kAhead <= kSlots, "read-ahead deeper than a step");

        // softmax state of this half tile
        float m_a = 0.f, m_b = 0.f, mx = 0.f, alpha = 1.f, m_use = 0.f, rs = 0.f;
        auto phase = [&](int ph) {
            if (ph < 2) {
                if constexpr (decltype(masked)::value) {
                    const int kv0 = 32 * hi;
                    const int lim = (causal ? min_(qrow, N - 1) : N - 1) - kv0 - 8 * hh;
#pragma unroll
                    for (int r = 8 * ph; r < 8 * ph + 8; ++r) {
                        const int c = 16 * (r >> 3) + (r & 7);
                        s_cur[r] = c > lim ? -INFINITY : s_cur[r];
                    }
                }
            }
            if (ph == 0) {
                m_a = fmaxf(fmaxf(s_cur[0], s_cur[1]), s_cur[2]);
                m_b = fmaxf(fmaxf(s_cur[3], s_cur[4]), s_cur[5]);
            } else if (ph < 3) {
                const int r = 6 + 4 * (ph - 1);
                m_a = fmaxf(fmaxf(m_a, s_cur[r]), s_cur[r + 1]);
                m_b = fmaxf(fmaxf(m_b, s_cur[r + 2]), s_cur[r + 3]);
            } else if (ph == 3) {
                m_a = fmaxf(fmaxf(m_a, s_cur[14]), s_cur[15]);
                mx = pair32_max(fmaxf(m_a, m_b)) * scale_log2;
            } else if (ph == 4) {
                m_run = fmaxf(m_run, mx);
                const bool move = mx > m_ref + kLazy;
                const float r_new = move ? mx : m_ref;
                alpha = move ? exp2_hw(m_ref - r_new) : 1.f;
                m_ref = r_new;
                m_use = (r_new == -INFINITY) ? 0.f : r_new;
            } else if (ph < 13) {
                const int k2 = ph - 5;  // score pair
                const float p0 = exp2_hw(__builtin_fmaf(s_cur[2 * k2], scale_log2, -m_use));
                const float p1 = exp2_hw(__builtin_fmaf(s_cur[2 * k2 + 1], scale_log2, -m_use));
                const uint32_t w = pack_bf16x2(p0, p1);
                // row sum of the bf16 weights the O MFMA multiplies (one v_dot2 per pair)
                rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                                     __builtin_bit_cast(bf16x2, 0x3f803f80u), rs, false);
                pk_cur[k2 >> 2][k2 & 3] = w;
            } else if (ph == 13) {
                l_part = l_part * alpha + rs;
            }
        };

        bf16x8 cur[kSlots];
#pragma unroll
        for (int sl = 0; sl < kAhead; ++sl) cur[sl] = fr[sl];
        s_next = f32x16{};
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int sl = 0; sl < kSlots; ++sl) {
            if (sl + kAhead < kSlots) {
                if (kPV || ((sl + kAhead) & 1) == 0) cur[sl + kAhead] = frag(hi, sl + kAhead);
            } else {
                fr[sl + kAhead - kSlots] = frag(hi + 1, sl + kAhead - kSlots);
            }
            if ((sl & 1) == 0) {
                s_next = mfma_32x32x16(cur[sl], qf[sl >> 1], s_next);
            } else if (kPV) {
                const int i = sl >> 1;
                const int t = i / (D / 32), db = i % (D / 32);
                acc_o[db] = mfma_32x32x16(cur[sl], __builtin_bit_cast(bf16x8, pk_prev[t]), acc_o[db]);
            }
#pragma unroll
            for (int ph = sl * kPhasesPerSlot; ph < (sl + 1) * kPhasesPerSlot; ++ph) phase(ph);
            // staging op o sits in slot 1 + o (kSlots - 2) / kStageOps
#pragma unroll
            for (int op = 0; op < T::kStageOps; ++op)
                if (sl == 1 + op * (kSlots - 2) / T::kStageOps && stage_j >= 0) stage_op(stage_j, op);
            __builtin_amdgcn_sched_barrier(0);
        }
        // The probabilities are first used by the next step; without this the compiler sinks
        // their exponentials past the rescale branch, away from the MFMAs they overlap.
        asm volatile("" : "+v"(pk_cur[0]), "+v"(pk_cur[1]), "+v"(l_part));
        rescale(alpha);
    };
    using Masked = std::true_type;
    using Plain = std::false_type;
    // Tiles before n_plain need no mask in any wave of the workgroup: all their keys precede
    // the workgroup's first query row (causal) and the end of the sequence. The remaining
    // tiles run the masked step in every wave (a no-op mask where nothing is masked), so each
    // loop below is a single straight path.
    const int n_plain = min_(n_tiles, causal ? (qb * kBr) / kBc : N / kBc);

    f32x16 sa, sb;
    u32x4 pa[2], pb[2];
    bf16x8 fr[kAhead];

    // ---- prologue: K0, K1 and V0 staged; K2 and V1 in registers; scores of half tile 0 ----
    load_k(0);
    load_v(0);
#pragma unroll
    for (int i = 0; i < T::kKLoads; ++i) store_k_part(0, i);
#pragma unroll
    for (int c = 0; c < 4; ++c) store_v_col(0, c);
    load_k(1);
#pragma unroll
    for (int i = 0; i < T::kKLoads; ++i) store_k_part(1, i);
    load_k(2);
    load_v(1);
    barrier_lds();
    compute_s(sa, 0, 0);

    // ---- tile 0: half 0 has no O update yet; its first step stages K2 / V1 ----
#pragma unroll
    for (int sl = 0; sl < kAhead; ++sl) fr[sl] = (sl & 1) ? bf16x8{} : frag(0, sl);
    if (n_plain > 0) {
        step(0, sa, sb, pb, pa, Plain{}, fr, std::false_type{}, 0);
        step(1, sb, sa, pa, pb, Plain{}, fr, std::true_type{}, -1);
    } else {
        step(0, sa, sb, pb, pa, Masked{}, fr, std::false_type{}, 0);
        step(1, sb, sa, pa, pb, Masked{}, fr, std::true_type{}, -1);
    }
    barrier_lds();

    // ---- tiles 1 .. n_tiles-1. Tile j reads K_j (half 1), K_{j+1} (half 0), V_{j-1}
    // (half 1) and V_j (half 0). During its first step it writes K_{j+2} and V_{j+1} to the
    // stages of K_{j-1} and V_{j-2}, both last read during tile j-1, before the previous
    // barrier, and first read after the barrier that ends tile j.
    // (Do-while loops with the exit test at the bottom keep the accumulators in one set of
    // registers.) ----
    auto tile = [&](int j, auto masked) {
        step(2 * j, sa, sb, pb, pa, masked, fr, std::true_type{}, j);
        step(2 * j + 1, sb, sa, pa, pb, masked, fr, std::true_type{}, -1);
        barrier_lds();
    };
    int j = 1;
    if (j < n_plain) {
        do {
            tile(j, Plain{});
        } while (++j < n_plain);
    }
    if (j < n_tiles) {
        do {
            tile(j, Masked{});
        } while (++j < n_tiles);
    }
    // last half tile's O update (its S^T step computed a score block past the end, unused)
    compute_pv(pb, (n_tiles - 1) % kStages, 1);

    // ---- epilogue: O / l, bf16, optional row statistics ----
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

hipError_t launch_fwd_bf16_sp(const void* q, const void* k, const void* v, void* o, float* m_out,
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
        hipLaunchKernelGGL(fwd_bf16_sp_kernel<128>, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                           qp, kp, vp, op, m_out, l_out, B, Hq, Hkv, N, sl2, causal, nqb);
    else
        hipLaunchKernelGGL(fwd_bf16_sp_kernel<64>, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                           qp, kp, vp, op, m_out, l_out, B, Hq, Hkv, N, sl2, causal, nqb);
    return hipGetLastError();
}

}  // namespace fa
