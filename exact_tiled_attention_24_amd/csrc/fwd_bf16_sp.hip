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
// that turns the scores of half tile h into probabilities (about 70 instructions). The two
// streams are independent, so the SIMD runs them side by side; the scheduler is told to
// interleave them (one MFMA, one LDS operand read, a few vector instructions, repeated).
// Two such waves share each SIMD (8 waves, 256 query rows per workgroup).
//
// CDNA4 details:
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: a lane holds the scores of one query row,
//    so row max and sum are in-lane plus one exchange with lane l ^ 32. The S^T
//    accumulator, converted to bf16, is directly the B operand of O^T += V^T P^T: the MFMA
//    reads K rows in an order that swaps bits 2 and 3 of the row index, so the
//    accumulator's register order is the key order the second MFMA needs.
//  * K and V tiles go from global memory straight into LDS (buffer loads with the LDS
//    bit): no staging registers. bf16 rows are stored row-major with their 16-byte chunks
//    XOR-swizzled by row (fp8 K rows padded instead), which makes every operand read conflict
//    free on gfx950's 64 banks; the V^T operand comes out of row-major V through
//    ds_read_b64_tr_b16. Q (dense) comes in and O goes out the same way, in whole 1 KiB
//    pieces through a per-wave LDS block, rather than as 16 or 8 bytes spread over 32 rows.
//  * Four LDS stages per operand: K of tile j+3 and V of tile j+2 are requested while tile
//    j is computed, with one workgroup barrier per 64-key tile. The tile loop is unrolled
//    over the four stages, so every operand address is a loop-invariant base plus an
//    immediate offset.
//  * Scores in the log2 domain; the exponent reference moves only when a row maximum beats
//    it by more than 2^8, so the O rescale (a branch after the MFMAs, out of line) is rare.
//    Without row statistics the reference is fixed per item, and at d = 128 the scale is
//    folded into Q and the reference into the products' initial value (see kPre).
//    The row sum adds the bf16-rounded probabilities (v_dot2 on the packed pairs), i.e.
//    exactly the weights the O MFMA uses.
//  * Every wave runs the half tiles of its workgroup in one schedule; masking is a uniform
//    branch taken only on the diagonal and ragged tiles. Except in the block-sparse
//    instance, a wave leaves out the steps past its own diagonal (they would add zero
//    weights) but still issues its share of the loads and meets every barrier; waves w and
//    w + 4, which share a SIMD, take row blocks w and 7 - w so that those savings are spread
//    over the SIMDs.
//  * Grid: one persistent workgroup per CU; a work item is one (256-row query block, head),
//    and each workgroup walks items of its XCD's contiguous share of the list in snake
//    order (see the kernel).
//
// Block-sparse variant (kSparse): the block-sparse forward of "FlashAttention, explained."
// (vibeengines.com): each work item processes only the key tiles its block list names (64
// keys per tile, 256 query rows per block), in list order; a per-lane window of the list's
// tile offsets feeds the loads as in the paged variant, and a short delay line of the tiles'
// first key positions drives the masking of diagonal, ragged and invalid tiles.
//
// FP8 variant (kFp8, d = 128): e4m3 Q and K. S^T takes two v_mfma_f32_32x32x64_f8f6f4 per half
// tile (a lane holds 32 consecutive head dimensions of its query; it reads the same 32 of
// its K row), in an 8-slot step whose every slot holds one bf16 P V MFMA; softmax, P and O
// as in bf16. K rows are 144 B in LDS (conflict free), a K stage 9 KiB.
//
// Paged variant (kPaged): chunked prefill over a paged KV cache, the paged rows of the
// family table on the same page. The queries are the newest Nq tokens of each sequence, so
// query i sits at position L - Nq + i of its L cached tokens and the causal diagonal is
// aligned to the bottom right. K/V of token t come from physical page
// block_table[b][t / 16], slot t % 16. Each 16-row page of a K stage starts at a 1 KiB
// boundary in LDS (V pages are whole KiB already), so every 1 KiB load lies in one page and
// its lanes add one wave-uniform page offset to fixed per-lane offsets. Pages past the
// sequence end, rows past it in the last page and invalid table entries read as zeros
// through the descriptor's range. Block-table entries come from a per-lane window of 64
// read back with v_readlane.
#include <type_traits>

#include "fa_internal.hpp"
#include "gfx950.hpp"

namespace fa {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBr = 32 * kWaves;  // query rows per workgroup
constexpr int kBc = 64;           // keys per tile (two 32-key half tiles)
// Buffer offset past every descriptor's range: a head's K or V rows span at most 2^30 bytes
// (and a paged cache less than 2^31), and a pad offset plus any tile offset stays below 2^32.
constexpr unsigned kPadOffset = 0x80000000u;
constexpr int kStages = 4;       // LDS stages of K and of V
constexpr int kXcds = 8;
constexpr float kLazy = 8.f;      // the exponent reference moves once a row maximum passes it by 2^8
constexpr float kV8Head = 4.f;    // e4m3 weights: a moved reference sits 2^4 below the maximum
constexpr int kAhead = 4;         // LDS operand reads kept in flight
constexpr int kBufferDword3 = 0x00020000;

// Pointers into LDS (address space 3): 32-bit, so an operand base is one VGPR.
typedef const __attribute__((address_space(3))) unsigned char* lds_cptr;
typedef const __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i32 lds_v2i32;

__device__ __forceinline__ int kappa(int m) {
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Workgroup barrier that orders LDS accesses only: global loads in flight stay in flight.
__device__ __forceinline__ void barrier_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

constexpr int kPageTok = 16;      // tokens per page of the paged cache
constexpr int kModeDense = 0, kModePaged = 1, kModeSparse = 2, kModeFp8 = 3, kModeFp8V = 4;
typedef int v8i32 __attribute__((ext_vector_type(8)));

// Chunk position of a staged row's 16-byte chunk c (bf16): c ^ swz<D>(r). With 64 four-byte
// banks this keeps every read of the kernel conflict-free: the row reads (16 lanes, 16 rows,
// one chunk) and the transposing reads (two 16-lane groups, 4 rows, 4 adjacent chunks) each
// find distinct bank groups, which a row pad gives only at the price of pad bytes in every
// load. d = 128 (a row fills the banks once): row bits 0-1 << 2 | row bits 2-3; d = 64 (two
// rows per bank line): row bit 1 << 2 | row bits 2-3.
// Chunk position of 16-byte chunk c of row r of a wave's 32-row block of Q or O: c ^ osw<D>(r).
// Conflict-free for a 16-lane read or write of one chunk of 16 consecutive rows, and for whole
// rows: d = 128, row bits 0-3; d = 64 (two rows per bank line), row bits 1-3.
template <int D>
__device__ __forceinline__ int osw(int r) {
    return D == 128 ? (r & 15) : ((r >> 1) & 7);
}

template <int D>
__device__ __forceinline__ int swz(int r) {
    return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

template <int D, bool kPaged, bool kFp8 = false, bool kV8 = false>
struct Tile {
    // bf16: unpadded rows with their 16 B chunks swizzled (swz), so that a stage holds only
    // the rows' bytes (d = 64: 16 KiB, two workgroups per CU; d = 128: 32 KiB, 4 loads of
    // 1 KiB per wave and tile)
    static constexpr bool kSwz = !kFp8;
    // K element bytes (fp8 e4m3 K: 1); the 16 B pad keeps a 16 B read of 16 rows in 16
    // distinct bank groups for both row lengths
    static constexpr int kKElem = kFp8 ? 1 : 2;
    static constexpr int kKRow = kSwz ? D * 2 : D * kKElem + 16;      // padded K row, bytes
    // V element bytes (fp8 e4m3 V: 1) and padded V row: bf16, the 64 B pad puts the four
    // rows a transposing read touches per cycle in four different 64 B bank windows; e4m3,
    // an 8-bit transposing read gives two 16-lane groups 32 B of the same eight consecutive
    // rows per cycle, and 160 B rows (5 x 32) put those eight 32 B pieces on eight distinct
    // 32 B bank groups (144 B rows left two of them on the same banks)
    static constexpr int kVElem = kV8 ? 1 : 2;
    static constexpr int kVRow = kV8 ? D + 32 : (kSwz ? D * 2 : D * 2 + 64);
    // paged: a K page (16 padded rows) occupies whole KiB, so no 1 KiB load spans two pages
    static constexpr int kKPage = kPaged ? (kPageTok * kKRow + 1023) / 1024 * 1024 : kPageTok * kKRow;
    static constexpr int kKStage = kPaged ? (kBc / kPageTok) * kKPage : kBc * kKRow;
    static constexpr int kVStage = kBc * kVRow;
    static constexpr int kKChunksPerPage = kKPage / 1024;             // paged only
    static constexpr int kVChunksPerPage = kPageTok * kVRow / 1024;
    static constexpr int kVBase = kStages * kKStage;                  // V stages follow K's
    static constexpr int kKChunks = kKStage / 1024;                   // 1 KiB DMA chunks
    static constexpr int kVChunks = kVStage / 1024;
    static constexpr int kDmaPerWave = (kKChunks + kVChunks + kWaves - 1) / kWaves;
    // Dense bf16 (kLdsQ bytes of LDS): Q comes through LDS too, in whole 1 KiB loads, each
    // wave's 32 rows in a block of kQBlock bytes: waves 0 and 1 in K stage 3, waves 2 .. 7 from
    // V stage 3 on, past the stages' end (stage 3's K and V are first loaded after the item's
    // first barrier)
    static constexpr int kQBlock = 32 * D * 2;
    static constexpr int kLdsQ = kStages * (kKStage + kVStage) + 6 * kQBlock - kVStage;
    static_assert(kPaged || kFp8 || (2 * kQBlock == kKStage && kLdsQ <= 160 * 1024),
                  "two Q blocks fill a K stage; the Q blocks fit");
    static_assert(kKStage % 1024 == 0 && kVStage % 1024 == 0, "stages are whole DMA chunks");
    static_assert(!kPaged || (kPageTok * kVRow) % 1024 == 0, "V pages are whole DMA chunks");
    static_assert(kStages * (kKStage + kVStage) <= 160 * 1024, "fits the LDS of one CU");
};

// Kernel arguments. Dense (and fp8, with e4m3 q and k): k, v are [B, Hkv, N, d]. Paged: k, v
// are the caches [num_pages, Hkv, 16, d], N is the query count Nq, and table / lens name the
// pages and the cached length of each sequence. Block-sparse: blk_off / blk_idx / nnz.
struct FwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* m_out;
    float* l_out;
    const int32_t* table;
    const int32_t* lens;
    const int32_t* q_lens;   // paged: optional query rows per sequence (NULL: N each)
    const int32_t* blk_off;  // block-sparse: compressed rows of key-tile lists
    const int32_t* blk_idx;
    int nnz;                 // entries of blk_idx
    int B, Hq, Hkv, N;
    float scale_log2;
    int causal, nqb;
    int max_pages, num_pages;
};

// One work item: the 256-row query block and head that `item` names in the work list
// (KV group, query block heaviest first, head in group). `smem` is the workgroup's LDS.
// kStats: the caller asked for the row statistics (m needs every tile's row maximum);
// without them the softmax skips the per-tile maximum (see `step`).
// Returns false (and writes nothing) when the softmax without statistics found its exponent
// reference stale; the caller then runs the item again with statistics.
template <int D, int kMode, bool kStats>
__device__ __forceinline__ bool fwd_item(const FwdArgs& a, int item, unsigned char* smem) {
    constexpr bool kPaged = kMode == kModePaged, kSparse = kMode == kModeSparse;
    constexpr bool kV8 = kMode == kModeFp8V;              // e4m3 V, P V on the fp8 matrix cores
    constexpr bool kFp8 = kMode == kModeFp8 || kV8;       // e4m3 Q and K
    constexpr bool kQLds = kMode == kModeDense;            // Q through LDS (see Tile)
    // bf16 without statistics (d = 128): Q is multiplied by the scale (log2 units) once, so
    // that the products give the exponent arguments, and the products of each score block start
    // from minus the row's exponent reference instead of zero: exp2 then takes the product's
    // result as it is (no scale-and-subtract per score)
    constexpr bool kPre = !kStats && !kFp8 && D == 128;
    using T = Tile<D, kPaged, kFp8, kV8>;
    // LDS operand reads kept in flight: fewer for the dense d = 64 instance, whose two
    // workgroups per CU leave a wave 128 registers
    constexpr int kAh = D == 64 && T::kSwz && kMode == kModeDense ? 2 : kAhead;
    constexpr int kKTile = kBc * D * T::kKElem, kVTile = kBc * D * T::kVElem;  // HBM bytes of a tile
    const uint16_t* __restrict__ q = a.q;
    const uint16_t* __restrict__ k = a.k;
    const uint16_t* __restrict__ v = a.v;
    uint16_t* __restrict__ o = a.o;
    float* __restrict__ m_out = a.m_out;
    float* __restrict__ l_out = a.l_out;
    const int Hq = a.Hq, Hkv = a.Hkv, N = a.N, nqb = a.nqb, causal = a.causal;
    const float scale_log2 = a.scale_log2;
    lds_cptr const lds = (lds_cptr)smem;  // generic -> LDS address space
    const unsigned lds_addr = (unsigned)(size_t)lds;  // LDS byte address of smem

    const int G = Hq / Hkv;
    const int per_unit = nqb * G;
    const int kvg = item / per_unit;
    const int rem = item - kvg * per_unit;
    const int qb = causal ? (nqb - 1 - rem / G) : rem / G;
    const int gi = rem - (rem / G) * G;
    const int b = kvg / Hkv;
    const int kvh = kvg - b * Hkv;
    const int h = kvh * G + gi;

    const size_t qoff = ((size_t)(b * Hq + h) * N) * D;
    const size_t koff = kPaged ? 0 : ((size_t)(b * Hkv + kvh) * N) * D;
    const uint16_t* qh = q + qoff;
    // (K addressed in bytes: fp8 K has one byte per element)
    const unsigned char* kh = reinterpret_cast<const unsigned char*>(k) + koff * T::kKElem;
    // Keys of this item's sequence and the position offset of its queries: query row i sits
    // at position i + off (dense: the N keys, off = 0; paged: the cached length L, clamped to
    // the table, and off = L - Nq, the bottom-right alignment).
    // (paged with per-sequence query counts: this sequence's queries are rows 0 .. nq - 1, and
    // a block that starts past them is no work item at all)
    int Nk = N, off = 0, nq = N;
    if constexpr (kPaged) {
        const int L = a.lens[b];
        Nk = __builtin_amdgcn_readfirstlane(L < 0 ? 0 : min_(L, a.max_pages * kPageTok));
        if (a.q_lens) {
            const int n = a.q_lens[b];
            nq = __builtin_amdgcn_readfirstlane(n < 0 ? 0 : min_(n, N));
        }
        off = Nk - nq;
        if (qb * kBr >= nq) return true;
    }
    // Block-sparse: this item's key tiles are blk_idx[list0 .. list0 + n_list) (clamped into
    // the array, so no read leaves it whatever the offsets hold).
    int list0 = 0, n_list = 0;
    if constexpr (kSparse) {
        const int r = (b * Hq + h) * nqb + qb;
        const int e0 = min_(max_(a.blk_off[r], 0), a.nnz);
        const int e1 = min_(max_(a.blk_off[r + 1], e0), a.nnz);
        list0 = __builtin_amdgcn_readfirstlane(e0);
        n_list = __builtin_amdgcn_readfirstlane(e1 - e0);
    }

    // (opaque per item: values derived from the thread index are not hoisted out of the
    // item loop, where two item bodies would hold theirs at once)
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    // (all but block-sparse, whose lists need not be sorted) a wave skips the steps past the
    // last key its rows see (see the tile loop); the waves sharing a SIMD (w and w + 4) take row blocks w and 7 - w, so that on the diagonal
    // tiles every SIMD is left about the same number of steps
    constexpr bool kSkip = kMode != kModeSparse;
    const int row0 = qb * kBr + 32 * (kSkip && wave >= 4 ? 11 - wave : wave);
    const int qrow = row0 + l32;

    // Q as the B operand of S^T = K Q^T: bf16, 8 head dimensions per 16-wide chunk and lane
    // half; fp8, 32 per 64-wide chunk (the same split as the K operand, so every head
    // dimension meets its partner once)
    bf16x8 qf[kFp8 ? 1 : D / 16];
    v8i32 qf8[kFp8 ? D / 64 : 1];
    if constexpr (kFp8) {
        const unsigned char* src = reinterpret_cast<const unsigned char*>(q) + qoff +
                                   (size_t)min_(qrow, N - 1) * D + 32 * hh;
#pragma unroll
        for (int c = 0; c < D / 64; ++c) {
            const u32x4 lo = *reinterpret_cast<const u32x4*>(src + 64 * c);
            const u32x4 hi = *reinterpret_cast<const u32x4*>(src + 64 * c + 16);
            qf8[c] = v8i32{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
    } else if constexpr (!kQLds) {
        const uint16_t* src = qh + (size_t)min_(qrow, N - 1) * D + 8 * hh;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            qf[kk] = *reinterpret_cast<const bf16x8*>(src + 16 * kk);
    }
    // (the Q loads are waited for with the first tiles' below, so the two latencies overlap)

    f32x16 acc_o[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) acc_o[i] = f32x16{};
    // (the exponent reference starts finite: a row whose first tiles are all masked then gets
    // exp2(-inf) = 0 rather than exp2(-inf + inf), and moves to its first finite maximum)
    float m_run = -INFINITY, m_ref = -1e30f, l_part = 0.f;
    f32x16 negm;  // (kPre) minus the exponent reference, the score products' initial value

    const int kv_end = causal ? min_(Nk, qb * kBr + kBr + off) : Nk;
    // (kSkip) the last half tile holding a key some row of the wave sees: the steps of half
    // tiles h_last + 2 on would only add zero weights
    const int h_last = (causal ? min_(row0 + 31 + off, Nk - 1) : Nk - 1) >> 5;
    const int n_tiles = kSparse ? n_list : (kv_end > 0 ? (kv_end + kBc - 1) / kBc : 0);

    // ---- staging: buffer loads straight into LDS (no registers). A tile's K stage (64
    // padded rows) and V stage (64 padded rows, row-major) are cut into 1 KiB chunks; one
    // DMA instruction of a wave fills one chunk, lane i the chunk's bytes 16 i .. 16 i + 15.
    // Wave w issues the chunks w, w + 8, ... of the list (K chunks, then V chunks; the list is
    // padded to a multiple of 8 by repeating its last chunk, which rewrites the same bytes),
    // so every wave issues kDmaPerWave loads per tile and one vmcnt count waits for a tile.
    // A lane that lands on row padding gets an offset past any descriptor's range, so it
    // fetches nothing (and writes zeros that are never read). Rows past N read as zero through
    // the descriptor's range. ----
    // Each wave's operation i targets the same chunk of every tile: its per-lane source
    // offset (relative to the tile, already advanced by the 3 tiles K runs ahead or the 2 of
    // V) and its LDS offset (relative to the stage) are fixed here. The descriptors span the
    // head's rows up to the end of this work item's last tile, so loads issued past the end
    // fetch nothing and fill zeros (as do the negative tile offsets of the prologue).
    // Paged: chunk c of a stage belongs to page c / (chunks per page) of the tile (the same
    // for all lanes: wave-uniform); the lane offset is relative to that page's 16 x d block.
    unsigned dma_src[T::kDmaPerWave];
    unsigned dma_dst[T::kDmaPerWave];
    int dma_pg[T::kDmaPerWave];
#pragma unroll
    for (int i = 0; i < T::kDmaPerWave; ++i) {
        const int c = min_(wave + kWaves * i, T::kKChunks + T::kVChunks - 1);
        const bool is_k = c < T::kKChunks;
        const int row_b = is_k ? T::kKRow : T::kVRow;
        const int cc = is_k ? c : c - T::kKChunks;
        dma_dst[i] = lds_addr + (is_k ? 0u : unsigned(T::kVBase)) + 1024u * cc;
        if constexpr (kPaged) {
            const int cpp = is_k ? T::kKChunksPerPage : T::kVChunksPerPage;
            dma_pg[i] = cc / cpp;
            const int slot = 1024 * (cc - dma_pg[i] * cpp) + 16 * lane;
            const int row = slot / row_b;
            int col = slot - row * row_b;
            if constexpr (T::kSwz) col = 16 * ((col >> 4) ^ swz<D>(row));  // the chunk stored here
            dma_src[i] = row < kPageTok && col < D * 2 ? unsigned(row * D * 2 + col) : kPadOffset;
        } else {
            const int slot = 1024 * cc + 16 * lane;
            const int row = slot / row_b;
            int col = slot - row * row_b;
            if constexpr (T::kSwz) col = 16 * ((col >> 4) ^ swz<D>(row));  // the chunk stored here
            const int rb = is_k ? D * T::kKElem : D * T::kVElem;  // HBM row bytes
            dma_src[i] = (col < rb ? unsigned(row * rb + col) : kPadOffset) +
                         unsigned(kSparse ? 0 : (is_k ? 3 * kKTile : 2 * kVTile));
            dma_pg[i] = 0;
        }
    }
    // Paged: byte offset (from this KV head's block in physical page 0) of every page of a
    // window of 64 pages, one per lane: lane l holds page wb + l, or kPagePad where the page
    // holds no row of the sequence or its table entry lies outside [0, num_pages), which puts
    // every lane of its loads past the descriptor's range (zeros). A load picks its page's
    // offset with one v_readlane. The window moves by 60 pages, so the V tile (one behind the
    // K tile) always lies in it too; the next window's table entries are loaded one tile
    // before they are needed. Rows of the last page past the sequence end are cut per lane
    // in the V loads (K rows there only meet masked scores).
    // (block-sparse: 2^30, past a head's rows and below the pad offset, so pad + 2^30 stays
    // past the range as well; paged: 2^31, past the cache, with pad lanes cut separately)
    constexpr unsigned kPagePad = kSparse ? 0x40000000u : 0x80000000u;
    const int p_last = (Nk - 1) / kPageTok;                          // last page holding a row
    const int last_bytes = (Nk - kPageTok * p_last) * D * 2;         // its rows, in bytes
    const unsigned stride_bytes = (unsigned)Hkv * kPageTok * D * 2;  // one physical page
    const int32_t* trow = nullptr;
    if constexpr (kPaged) trow = a.table + (size_t)b * a.max_pages;
    // Block-sparse: the window holds the byte offsets of list positions wb .. wb + 63 (one
    // tile each; kPagePad past the list or for an index outside the key tiles), and kvq0..3
    // the first key position of tiles j .. j + 3 (1 << 30 for an invalid index: fully masked).
    constexpr int kTileBytes = kBc * D * 2;
    const int n_ktiles = (N + kBc - 1) / kBc;
    int kvq0 = 0, kvq1 = 0, kvq2 = 0, kvq3 = 0;
    int wb = kSparse ? -1 : -4, kidx = 0, vidx = 0;
    int raw_next = -1;
    unsigned win = kPagePad;
    auto list_entries = [&](int first) {  // list entry of position first + lane (clamped)
        return a.blk_idx[list0 + min_(max_(first + lane, 0), n_list - 1)];
    };
    auto tile_offsets = [&](int e, int first) {
        const int pos = first + lane;
        return pos >= 0 && pos < n_list && e >= 0 && e < n_ktiles ? (unsigned)e * kTileBytes : kPagePad;
    };
    auto table_entries = [&](int first) {  // entry of page first + lane (clamped into the row)
        return trow[min_(max_(first + lane, 0), a.max_pages - 1)];
    };
    auto page_offsets = [&](int e, int first) {
        const int p = first + lane;
        return p >= 0 && p <= p_last && e >= 0 && e < a.num_pages ? (unsigned)e * stride_bytes
                                                                 : kPagePad;
    };
    // Before the loads of K tile t and V tile t - 1.
    auto advance = [&](int t) {
        if constexpr (kSparse) {
            if (t >= wb + 64) {
                wb = t - 1;
                win = tile_offsets(raw_next, wb);
            }
            if (t + 1 >= wb + 64) raw_next = list_entries(t);
            kidx = t - wb;
            vidx = kidx - 1;
            const unsigned ot = __builtin_amdgcn_readlane(win, kidx);
            kvq0 = kvq1, kvq1 = kvq2, kvq2 = kvq3;
            kvq3 = ot >= kPagePad ? (1 << 30) : (int)(ot / kTileBytes) * kBc;
        }
        if constexpr (kPaged) {
            if (4 * t + 3 >= wb + 64) {
                wb = 4 * t - 4;
                win = page_offsets(raw_next, wb);
            }
            if (4 * t + 7 >= wb + 64) raw_next = table_entries(4 * t);
            kidx = 4 * t - wb;
            vidx = kidx - 4;
        }
    };
    const int row_end = kSparse ? N : min_(Nk, n_tiles * kBc);
    // (readfirstlane: the clamp selects to a vector instruction, and a descriptor word in a
    // VGPR would force a per-lane loop around every buffer load)
    // Dense: the head's rows up to the end of this item's last tile. Paged: the cache from
    // this KV head's block of page 0 to the end of its block in the last page (under 2 GiB).
    const int head_bytes = __builtin_amdgcn_readfirstlane(
        kPaged ? (a.num_pages > 0 ? (a.num_pages - 1) * (int)stride_bytes + kPageTok * D * 2 : 0)
               : row_end * D * 2);
    const int head_bytes_k = kFp8 ? __builtin_amdgcn_readfirstlane(row_end * D) : head_bytes;
    const int head_bytes_v = kV8 ? head_bytes_k : head_bytes;
    const size_t kv_page = kPaged ? (size_t)kvh * kPageTok * D : 0;  // KV head within a page
    const __amdgpu_buffer_rsrc_t rsrc_k = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kh + kv_page * 2), (short)0, head_bytes_k, kBufferDword3);
    // (V addressed in bytes: e4m3 V has one byte per element)
    const unsigned char* vhb = reinterpret_cast<const unsigned char*>(v) + (koff + kv_page) * T::kVElem;
    const __amdgpu_buffer_rsrc_t rsrc_v =
        __builtin_amdgcn_make_buffer_rsrc((void*)vhb, (short)0, head_bytes_v, kBufferDword3);
    // DMA operation i of tile step j (stage phase P = j mod 4): K of tile j + 3 and V of
    // tile j + 2. Written as assembly: the compiler's own form makes it wait for every
    // outstanding load to LDS before each transposing read (it cannot tell the stages
    // apart); the waits here are explicit. Operations whose chunks are all K (or all V) for
    // every wave need no select.
    auto dma_op = [&](int j, int i, int P, bool k_only = false) {  // P: the stage phase (a constant, or uniform in the e4m3-V steps)
        constexpr int kK = T::kKChunks;
        const bool all_k = kWaves * i + kWaves - 1 < kK, all_v = kWaves * i >= kK;
        const bool is_k = all_k || (!all_v && wave + kWaves * i < kK);
        if (k_only && !is_k) return;  // (uniform per wave)
        const unsigned stage = is_k ? unsigned(((P + 3) & (kStages - 1)) * T::kKStage)
                                    : unsigned(((P + 2) & (kStages - 1)) * T::kVStage);
        if constexpr (kPaged) {
            // page 4 t + pg of the sequence, t = j + 3 (K) or j + 2 (V)
            const int pg = dma_pg[i];
            const unsigned po = __builtin_amdgcn_readlane(win, (is_k ? kidx : vidx) + pg);
            // (pad lanes, and V rows past the end of the last page, take the out-of-range
            // offset: a pad offset plus a page offset could wrap back into the cache)
            const int page = 4 * (j + (is_k ? 3 : 2)) + pg;
            const unsigned lim = !all_k && !is_k && page == p_last ? (unsigned)last_bytes : kPadOffset;
            const unsigned src = dma_src[i] < lim ? dma_src[i] + po : kPagePad;
            const __amdgpu_buffer_rsrc_t r = is_k ? rsrc_k : rsrc_v;
            asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                         :
                         : "v"(src), "s"(r), "{m0}"(dma_dst[i] + stage)
                         : "memory");
        } else if constexpr (kSparse) {
            // list position j + 3 (K) or j + 2 (V)
            const unsigned po = __builtin_amdgcn_readlane(win, is_k ? kidx : vidx);
            const __amdgpu_buffer_rsrc_t r = is_k ? rsrc_k : rsrc_v;
            asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                         :
                         : "v"(dma_src[i] + po), "s"(r), "{m0}"(dma_dst[i] + stage)
                         : "memory");
        } else {
            const __amdgpu_buffer_rsrc_t r = is_k ? rsrc_k : rsrc_v;
            asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                         :
                         : "v"(dma_src[i] + unsigned(j * (is_k ? kKTile : kVTile))), "s"(r),
                           "{m0}"(dma_dst[i] + stage)
                         : "memory");
        }
    };
    auto dma_tile = [&](int j, int P, bool k_only = false) {
#pragma unroll
        for (int i = 0; i < T::kDmaPerWave; ++i) dma_op(j, i, P, k_only);
    };
    // LDS DMA is not tracked by the compiler's waits: wait for all but the newest tile's
    // loads (vmcnt counts this wave's vector loads in issue order), then the barrier.
    auto wait_dma_tile = [&]() {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(T::kDmaPerWave) : "memory");
    };
    auto wait_dma_all = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

    // Operand addresses: a per-lane base plus an immediate. K: lane (l32, hh) reads 16 bytes
    // of row kappa(l32). V: the V^T operand comes from row-major V through
    // ds_read_b64_tr_b16, which transposes within each 16-lane group: when source lane
    // q + 4e (q, e < 4) reads 4 elements at V[k0 + e][d0 + 4q], lane j of the group receives
    // V[k0 .. k0 + 3][d0 + j]. Two such reads give a lane its 8 consecutive keys of one head
    // dimension, as the MFMA's A operand wants (lane l: d = l % 32, keys 8 (l / 32) ..).
    // Stages are compile-time (the tile loop is unrolled over the four stages), so every
    // operand address is one of three loop-invariant bases plus an immediate (the offset
    // field holds 16 bits: the V stages need a second base for stages 2 and 3). The bases
    // go through an empty asm so that the compiler keeps them opaque rather than
    // re-associating the offsets into per-read additions.
    // (paged: row r of a K stage sits in page block r / 16 at row r % 16; kappa keeps bit 4,
    // and the stages need a second base as the V stages do)
    // (fp8: a lane reads 32 bytes of its row per 64 head dimensions, lane half hh the second 32)
    lds_cptr base_k = kPaged ? lds + (l32 >> 4) * T::kKPage + (kappa(l32) & 15) * T::kKRow + hh * 16
                             : lds + kappa(l32) * T::kKRow + hh * (kFp8 ? 32 : 16);
    lds_cptr base_k2 = base_k + 2 * T::kKStage;
    lds_cptr base_v = lds + T::kVBase + (8 * (lane >> 5) + ((lane & 15) >> 2)) * T::kVRow +
                      (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
    lds_cptr base_v2 = base_v + 2 * T::kVStage;
    if constexpr (kPaged) asm volatile("" : "+v"(base_k2));
    asm volatile("" : "+v"(base_k), "+v"(base_v), "+v"(base_v2));
    static_assert(kPaged || 3 * T::kKStage + 32 * T::kKRow + 2 * D < 65536, "K offsets fit the immediate");
    static_assert(!kPaged || T::kKStage + 2 * T::kKPage + 2 * D < 65536, "K offsets fit the immediate");
    static_assert(T::kVStage + 32 * T::kVRow + 20 * T::kVRow + 2 * D < 65536,
                  "V offsets fit the immediate");
    // bf16 (swizzled rows): the lane's column offset differs per 16-byte chunk. Every read
    // takes a per-lane base for its chunk (K: one per 16 head dimensions; V: one per
    // head-dimension block and row half) plus the stage offset as an immediate (the four K
    // stages, and the four V stages, span at most 64 KiB, so one base per read reaches them
    // all). The stage addresses below are then plain offsets from kz0 / vz0.
    const lds_cptr kz0 = lds, vz0 = lds + T::kVBase;
    lds_cptr base_kk[T::kSwz ? D / 16 : 1];
    lds_cptr base_vv[T::kSwz ? D / 32 : 1][2];
    if constexpr (T::kSwz) {
        const int rk = kappa(l32);  // the lane's K row in a stage (paged pages are 16 whole rows)
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            base_kk[kk] = lds + rk * T::kKRow + 16 * ((2 * kk + hh) ^ swz<D>(rk));
            asm volatile("" : "+v"(base_kk[kk]));
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int rv = 8 * (lane >> 5) + ((lane & 15) >> 2) + 4 * h2;
                const int c = 4 * db + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
                base_vv[db][h2] = lds + T::kVBase + rv * T::kVRow + 16 * (c ^ swz<D>(rv)) + 8 * (lane & 1);
                asm volatile("" : "+v"(base_vv[db][h2]));
            }
    }
    // K rows of half kb of stage st; V rows of half kb of stage st.
    auto k_at = [&](int st, int kb) {
        if constexpr (T::kSwz) return kz0 + st * T::kKStage + 32 * kb * T::kKRow;
        else if constexpr (kPaged) return (st < 2 ? base_k : base_k2) + (st & 1) * T::kKStage + 2 * kb * T::kKPage;
        else return base_k + st * T::kKStage + 32 * kb * T::kKRow;
    };
    auto v_at = [&](int st, int kb) {
        if constexpr (T::kSwz) return vz0 + st * T::kVStage + 32 * kb * T::kVRow;
        else return (st < 2 ? base_v : base_v2) + (st & 1) * T::kVStage + 32 * kb * T::kVRow;
    };
    // K operand of head dimensions 16 kk .. of the rows at ks (the lane's row and chunk)
    auto kfrag = [&](lds_cptr ks, int kk) -> bf16x8 {
        if constexpr (T::kSwz) return *reinterpret_cast<const lds_bf16x8*>(base_kk[kk] + (ks - kz0));
        else return *reinterpret_cast<const lds_bf16x8*>(ks + 32 * kk);
    };

    // fp8 K operand of the 64 head dimensions c of the rows at ks (two 16 B reads)
    auto kfrag8 = [&](lds_cptr ks, int c) -> v8i32 {
        typedef const __attribute__((address_space(3))) u32x4 lds_u32x4;
        const u32x4 lo = *reinterpret_cast<lds_u32x4*>(ks + 64 * c);
        const u32x4 hi = *reinterpret_cast<lds_u32x4*>(ks + 64 * c + 16);
        return v8i32{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    };
    // e4m3 x e4m3 -> f32 on the matrix cores (no block scales)
    auto mfma_fp8 = [&](v8i32 a8, v8i32 b8, f32x16 c) {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 0, 0, 0, 0, 0, 0);
    };
    // S^T = K Q^T of half tile (K stage st, half kb) into s.
    auto compute_s = [&](f32x16& s, int st, int kb) {
        const lds_cptr ks = k_at(st, kb);
        s = f32x16{};
        if constexpr (kFp8) {
#pragma unroll
            for (int c = 0; c < D / 64; ++c) s = mfma_fp8(kfrag8(ks, c), qf8[c], s);
        } else {
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) s = mfma_32x32x16(kfrag(ks, kk), qf[kk], s);
        }
    };
    // V^T operand for key group t (16 keys) and head-dimension block db, from the V rows at
    // vb (a stage half).
    auto vfrag = [&](lds_cptr vb, int t, int db) -> bf16x8 {
        v4i16 lo, hi;
        if constexpr (T::kSwz) {
            const int off = (int)(vb - vz0) + 16 * t * T::kVRow;
            lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(base_vv[db][0] + off));
            hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(base_vv[db][1] + off));
        } else {
            const lds_cptr p = vb + 16 * t * T::kVRow + 64 * db;
            lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
            hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 4 * T::kVRow));
        }
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // O^T += V^T P^T of half tile (V stage st, half kb) with probabilities pk.
    auto compute_pv = [&](const u32x4 (&pk)[2], int st, int kb) {
        const lds_cptr vb = v_at(st, kb);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const bf16x8 pb = __builtin_bit_cast(bf16x8, pk[t]);
#pragma unroll
            for (int db = 0; db < D / 32; ++db) acc_o[db] = mfma_32x32x16(vfrag(vb, t, db), pb, acc_o[db]);
        }
    };
    // Lazy O rescale, after the step's MFMAs (which added the previous half tile).
    auto rescale = [&](bool move, float alpha) {
        if (__builtin_expect(__any(move), 0)) {
#pragma unroll
            for (int i = 0; i < D / 32; ++i) acc_o[i] *= alpha;
        }
    };
    // Causal / ragged mask of half tile hi (first key: block-sparse, of the listed tile at
    // key position kv_tile) on scores s: the key of register r is kv0 + 16 (r >> 3) + 8 hh +
    // (r & 7); it is masked when it lies after the query (causal) or at or past the end.
    auto mask_half = [&](f32x16& s, int hi, int kv_tile) {
        const int kv0 = kSparse ? kv_tile + 32 * (hi & 1) : 32 * hi;
        const int lim = (causal ? min_(qrow + off, Nk - 1) : Nk - 1) - kv0 - 8 * hh;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int c = 16 * (r >> 3) + (r & 7);
            s[r] = c > lim ? -INFINITY : s[r];
        }
    };
    // After a step's MFMAs (which added the previous half tile into O): with statistics, the
    // lazy O rescale. Without statistics the exponent reference never moves (see the
    // prologue), so there is nothing to do.
    auto after_step = [&](bool move, float alpha) {
        if constexpr (kStats) rescale(move, alpha);
    };
    // Operand rows of step hi (H8 = hi mod 8, so stages are compile-time): K of half tile
    // hi+1 and V of half tile hi-1.
    struct Bases {
        lds_cptr k, v;
    };
    auto bases = [&](auto h8_c) {
        constexpr int H8 = decltype(h8_c)::value;
        constexpr int hk = (H8 + 1) & 7, hv = (H8 + 7) & 7;
        return Bases{k_at(hk >> 1, hk & 1), v_at(hv >> 1, hv & 1)};
    };
    // Slot order of a step: d = 128 takes the D / 16 S^T MFMAs first (K, head dimensions
    // 16 i ..), then the O MFMAs (V^T, key group t, head-dimension block db); d = 64, whose
    // 128 registers the first order overruns, alternates them (S^T in the even slots).
    constexpr bool kSFirst = D == 128;
    auto slot_is_s = [](int sl) { return kSFirst ? sl < D / 16 : (sl & 1) == 0; };
    auto slot_i = [](int sl) { return kSFirst ? (sl < D / 16 ? sl : sl - D / 16) : sl >> 1; };
    // MFMA operand of slot `sl`
    auto frag = [&](const Bases& b, int sl) -> bf16x8 {
        const int i = slot_i(sl);
        if (slot_is_s(sl)) return kfrag(b.k, i);
        return vfrag(b.v, i / (D / 32), i % (D / 32));
    };
    // One pipeline step. Its MFMAs are S^T of half tile hi+1 (into s_next) and O^T += V^T P^T
    // of half tile hi-1 (probabilities pk_prev); at d = 128 all S^T ones first, so that the
    // next step's first reads of s_next come eight products after its last one (back-to-back
    // dependent products run at full rate); beside them runs the softmax of half tile hi
    // (s_cur -> pk_cur). The
    // step is written as kSlots slots, each one LDS operand read (kAh slots ahead), one
    // MFMA and a slice of the softmax, with a scheduling barrier after every slot, so the
    // instruction order is the one written here. `fr` holds on entry the operands of this
    // step's first kAh slots and on exit those of the next step's (read in this step's
    // last slots, so the next step starts without waiting, even across a barrier: its
    // operands were staged before the previous barrier).
    // (with_pv false: half tile 0, whose step has no O update; its O slots stay empty.)
    // with_dma: this step (the first of tile j = hi / 2) also issues the loads of K of tile
    // j + 3 and V of tile j + 2 (one DMA per odd slot).
    //
    // fp8 scores (kFp8): 8 slots, each one O MFMA (key group sl / 4, head-dimension block
    // sl % 4) and two softmax phases; the two fp8 S^T MFMAs (64 head dimensions each, as long
    // as two bf16 products) sit in slots 0 and 4 with K operands in kq, and the K operands of
    // the next step (half tile hi+2) replace them in slots 2 and 6. V^T operands are read two
    // slots ahead (fr[0..1] carries the next step's first two).
    auto step = [&](int hi, int kv_tile, auto h8_c, f32x16& s_cur, f32x16& s_next, const u32x4 (&pk_prev)[2],
                    u32x4 (&pk_cur)[2], bool masked, bf16x8 (&fr)[kAh], v8i32 (&kq)[2],
                    auto with_pv, auto with_dma) {
        constexpr int H8 = decltype(h8_c)::value;
        constexpr bool kPV = decltype(with_pv)::value;
        constexpr bool kDma = decltype(with_dma)::value;
        constexpr int kS = D / 16;             // S^T MFMAs (one per 16 head dimensions)
        constexpr int kSlots = kFp8 ? D / 16 : 2 * kS;  // bf16: as many O MFMAs as S^T ones
        constexpr int kPhasesPerSlot = 16 / kSlots;
        static_assert(kAh <= kSlots, "read-ahead deeper than a step");

        // Softmax of this half tile, cut into 16 phases (one per slot for d = 128) and
        // software-pipelined so that the instructions of one phase do not wait on each other:
        // the row maximum is a depth-3 tree of max3; the scores go through exp2 one pair per
        // phase, and each pair is packed to bf16 one phase later and added to the row sum one
        // phase after that.
        float t0 = 0.f, t1 = 0.f, t2 = 0.f, t3 = 0.f, t4 = 0.f, mx = 0.f, alpha = 1.f;
        bool move = false;
        float e0[8], e1[8];  // exp2 of score pair k (held until packed)
        uint32_t wk[8];      // packed pair k (held until summed)
        auto mask_scores = [&]() { mask_half(s_cur, hi, kv_tile); };
        // pair k: exp2 in phase ph_e + k, packed one phase later, summed one phase after that
        auto pair_stages = [&](int ph, int ph_e) {
            const int ke = ph - ph_e, kp = ke - 1, ks = ke - 2;
            if (ks >= 0 && ks < 8)
                l_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wk[ks]),
                                                         __builtin_bit_cast(bf16x2, 0x3f803f80u), l_part, false);
            if (kp >= 0 && kp < 8) {
                wk[kp] = pack_bf16x2(e0[kp], e1[kp]);
                pk_cur[kp >> 2][kp & 3] = wk[kp];
            }
            if (ke >= 0 && ke < 8) {
                e0[ke] = exp2_hw(__builtin_fmaf(s_cur[2 * ke], scale_log2, -m_ref));
                e1[ke] = exp2_hw(__builtin_fmaf(s_cur[2 * ke + 1], scale_log2, -m_ref));
            }
        };
        // without statistics: one score per phase from phase 0 (exp2), pair k packed in the
        // phase after its second score and summed one phase later (the last pair at once)
        float es[16];
        auto single_stages = [&](int ph) {
            es[ph] = exp2_hw(kPre ? s_cur[ph] : __builtin_fmaf(s_cur[ph], scale_log2, -m_ref));
            auto pack_pair = [&](int k) {
                wk[k] = pack_bf16x2(es[2 * k], es[2 * k + 1]);
                pk_cur[k >> 2][k & 3] = wk[k];
            };
            auto sum_pair = [&](int k) {
                l_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wk[k]),
                                                         __builtin_bit_cast(bf16x2, 0x3f803f80u), l_part, false);
            };
            if (ph >= 2 && (ph & 1) == 0) pack_pair(ph / 2 - 1);
            if (ph >= 3 && (ph & 1) == 1) sum_pair((ph - 3) / 2);
            if (ph == 15) {
                pack_pair(7);
                sum_pair(7);
            }
        };
        auto phase = [&](int ph) {
            if constexpr (!kStats) {
                // no row maximum: the exponentials start at once against the current reference
                if (ph == 0 && __builtin_expect(masked, 0)) mask_scores();
                single_stages(ph);
                return;
            }
            if (ph == 0) {
                if (__builtin_expect(masked, 0)) mask_scores();
                t0 = vmax(vmax(s_cur[0], s_cur[1]), s_cur[2]);
                t1 = vmax(vmax(s_cur[3], s_cur[4]), s_cur[5]);
                t2 = vmax(vmax(s_cur[6], s_cur[7]), s_cur[8]);
            } else if (ph == 1) {
                t3 = vmax(vmax(s_cur[9], s_cur[10]), s_cur[11]);
                t4 = vmax(vmax(s_cur[12], s_cur[13]), s_cur[14]);
            } else if (ph == 2) {
                t0 = vmax(vmax(t0, t1), t2);
                t3 = vmax(vmax(t3, t4), s_cur[15]);
            } else if (ph == 3) {
                mx = pair32_vmax(vmax(t0, t3)) * scale_log2;
            } else if (ph == 4) {
                // (m_ref starts at -1e30: the first finite row maximum always moves it, with
                // alpha = 0 on a zero O and row sum; a row with no key yet keeps it and gets
                // exp2(-inf) = 0 for its masked scores)
                m_run = vmax(m_run, mx);
                move = mx > m_ref + kLazy;
                const float r_new = move ? mx : m_ref;
                alpha = move ? exp2_hw(m_ref - r_new) : 1.f;
                m_ref = r_new;
                l_part *= alpha;
            }
            pair_stages(ph, 5);
        };

        const Bases b_cur = bases(h8_c), b_next = bases(std::integral_constant<int, (H8 + 1) & 7>{});
        bf16x8 cur[kSlots];
        s_next = f32x16{};
        if constexpr (kFp8) {
            static_assert(D == 128, "fp8 scores: d = 128");
            constexpr int kA8 = 2;  // V^T operand read-ahead, slots
            cur[0] = fr[0];
            cur[1] = fr[1];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int sl = 0; sl < kSlots; ++sl) {
                if (sl + kA8 < kSlots) {
                    if (kPV) cur[sl + kA8] = vfrag(b_cur.v, (sl + kA8) >> 2, (sl + kA8) & 3);
                } else {
                    fr[sl + kA8 - kSlots] = vfrag(b_next.v, (sl + kA8 - kSlots) >> 2, (sl + kA8 - kSlots) & 3);
                }
                if ((sl & 3) == 0) s_next = mfma_fp8(kq[sl >> 2], qf8[sl >> 2], s_next);
                if ((sl & 3) == 2) kq[sl >> 2] = kfrag8(b_next.k, sl >> 2);
                if (kPV)
                    acc_o[sl & 3] = mfma_32x32x16(cur[sl], __builtin_bit_cast(bf16x8, pk_prev[sl >> 2]),
                                                  acc_o[sl & 3]);
#pragma unroll
                for (int ph = sl * kPhasesPerSlot; ph < (sl + 1) * kPhasesPerSlot; ++ph) phase(ph);
#pragma unroll
                for (int i = 0; i < T::kDmaPerWave; ++i)
                    if (sl == 1 + 2 * i && kDma) dma_op(hi >> 1, i, H8 >> 1);
                __builtin_amdgcn_sched_barrier(0);
            }
            asm volatile("" : "+v"(pk_cur[0]), "+v"(pk_cur[1]), "+v"(l_part));
            after_step(move, alpha);
            return;
        }
#pragma unroll
        for (int sl = 0; sl < kAh; ++sl) cur[sl] = fr[sl];
        if constexpr (kPre) s_next = negm;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int sl = 0; sl < kSlots; ++sl) {
            if (sl + kAh < kSlots) {
                if (kPV || slot_is_s(sl + kAh)) cur[sl + kAh] = frag(b_cur, sl + kAh);
            } else {
                fr[sl + kAh - kSlots] = frag(b_next, sl + kAh - kSlots);
            }
            if (slot_is_s(sl)) {
                s_next = mfma_32x32x16(cur[sl], qf[kFp8 ? 0 : slot_i(sl)], s_next);
            } else if (kPV) {
                const int i = slot_i(sl);
                const int t = i / (D / 32), db = i % (D / 32);
                acc_o[db] = mfma_32x32x16(cur[sl], __builtin_bit_cast(bf16x8, pk_prev[t]), acc_o[db]);
            }
#pragma unroll
            for (int ph = sl * kPhasesPerSlot; ph < (sl + 1) * kPhasesPerSlot; ++ph) phase(ph);
            // DMA i sits in slot 1 + 2 i
#pragma unroll
            for (int i = 0; i < T::kDmaPerWave; ++i)
                if (sl == 1 + 2 * i && kDma) dma_op(hi >> 1, i, H8 >> 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        // The probabilities are first used by the next step; without this the compiler sinks
        // their exponentials past the rescale branch, away from the MFMAs they overlap.
        asm volatile("" : "+v"(pk_cur[0]), "+v"(pk_cur[1]), "+v"(l_part));
        after_step(move, alpha);
    };
    // Tiles before n_plain need no mask in any wave of the workgroup: all their keys precede
    // the workgroup's first query row (causal) and the end of the sequence. The others mask
    // in every wave (a no-op where nothing is masked), behind a uniform branch.
    // (block-sparse: a key-tile index below n_plain needs no mask; the other modes compare the
    // tile's position, which is its index)
    const int n_plain = kSparse ? (causal ? (qb * kBr + 1) / kBc : N / kBc)
                                : min_(n_tiles, causal ? max_(0, qb * kBr + off + 1) / kBc : Nk / kBc);

    f32x16 sa, sb;
    u32x4 pa[2], pb[2];
    bf16x8 fr[kAh];
    v8i32 kq[2] = {};  // fp8: K operands of the coming S^T (unused otherwise)

    using Yes = std::true_type;
    using No = std::false_type;

    // (paged: an item none of whose rows sees a key skips to the epilogue)
    if (!(kPaged || kSparse) || n_tiles > 0) {
    if constexpr (kPaged) win = page_offsets(table_entries(wb), wb);
    if constexpr (kSparse) win = tile_offsets(list_entries(wb), wb);

    // ---- prologue: (Q,) K0..K2 and V0, V1 staged; scores of half tile 0 ----
    lds_cptr qblk = lds;
    if constexpr (kQLds) {
        // the wave's 32 Q rows (8 B-operand chunks of 16 bytes a row, stored at chunk
        // c ^ osw(r) of row r): load i fills bytes 1024 i .. 1024 i + 1023 of the block, lane l
        // the 16 at 16 l; rows past N read zero through the descriptor's range
        const unsigned qb_off = wave < 2 ? 3u * T::kKStage + unsigned(wave) * T::kQBlock
                                         : unsigned(T::kVBase + 3 * T::kVStage) + unsigned(wave - 2) * T::kQBlock;
        qblk = lds + qb_off;
        const __amdgpu_buffer_rsrc_t rsrc_q =
            __builtin_amdgcn_make_buffer_rsrc((void*)qh, (short)0, __builtin_amdgcn_readfirstlane(N * D * 2), kBufferDword3);
#pragma unroll
        for (int i = 0; i < T::kQBlock / 1024; ++i) {
            const int slot = 1024 * i + 16 * lane;
            const int r = slot / (2 * D), cs = (slot % (2 * D)) / 16;
            const unsigned src = unsigned((row0 + r) * 2 * D + 16 * (cs ^ osw<D>(r)));
            asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                         :
                         : "v"(src), "s"(rsrc_q), "{m0}"(lds_addr + qb_off + 1024u * i)
                         : "memory");
        }
    }
    advance(0);
    dma_tile(-3, 1, kQLds);  // K0 (and zeros for V of tile -1, in the stage V3 takes later; not
                             // with Q in that stage)
    advance(1);
    dma_tile(-2, 2);  // K1, V0
    advance(2);
    dma_tile(-1, 3);  // K2, V1
    wait_dma_all();
    if constexpr (kQLds) {
        // the wave's own loads have landed: its Q block is readable before the barrier, which
        // also waits for these reads (K3 and V3 overwrite the blocks after it)
        const int rq = l32;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            qf[kk] = *(const lds_bf16x8*)(qblk + rq * 2 * D + 16 * ((2 * kk + hh) ^ osw<D>(rq)));
    }
    barrier_lds();
    if constexpr (kPre) {
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            u32x4 w = __builtin_bit_cast(u32x4, qf[kk]);
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(bf16_lo(w[i]) * scale_log2, bf16_hi(w[i]) * scale_log2);
            qf[kk] = __builtin_bit_cast(bf16x8, w);
        }
    }
    if constexpr (kFp8) {
#pragma unroll
        for (int c = 0; c < D / 64; ++c) asm volatile("" : "+v"(qf8[c]));
    } else {
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) asm volatile("" : "+v"(qf[kk]));
    }
    if constexpr (kV8) {
    // ---- e4m3 V: one step per 64-key tile. Step j computes S^T of tile j + 1 (four fp8
    // MFMAs), the softmax of tile j (both halves against one exponent reference, so that the
    // tile's P shares it) and O^T += V^T P^T of tile j - 1 on the fp8 matrix cores: one
    // v_mfma_f32_32x32x64_f8f6f4 per 32 head dimensions, contracting all 64 keys, plus one
    // against an all-ones operand that adds the tile's row sums of the e4m3 weights to every
    // row of acc_l (so O / l is a convex combination of V rows with exactly the weights used).
    // Over a tile, lane (query q, half hh) holds the scores of 32 keys, registers r of the two
    // halves in order; with K read in kappa order these are keys 16 u + 8 hh + i for byte
    // t = 8 u + i of the B operand, so P^T is the two halves' weights rounded to e4m3 in
    // register order, and V^T takes the same keys: four 8-bit transposing reads per lane, each
    // 8 consecutive V rows (source lane q' + 2 i of a 16-lane group reads row 16 u + 8 hh + i at
    // byte 8 q' of its 16 head dimensions; lane j of the group receives column j of the 8 rows).
    // The exponent reference moves only when a tile's row maximum passes it by more than 2^8,
    // and then to 2^4 below that maximum: every weight stays at most 256, inside e4m3's range
    // (448), and the reference stays at least 2^4 below the row's largest weight, so the
    // weights that fall below e4m3's normal range (2^-6 of the reference) are under 2^-10 of
    // the largest one. ----
    const v8i32 ones8 = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                         0x38383838, 0x38383838, 0x38383838, 0x38383838};  // e4m3 1.0
    lds_cptr base_v8 = lds + T::kVBase + (8 * hh + ((lane & 15) >> 1)) * T::kVRow +
                       16 * ((lane >> 4) & 1) + 8 * (lane & 1);
    asm volatile("" : "+v"(base_v8));
    static_assert(!kV8 || 3 * T::kVStage + 48 * T::kVRow + 96 < 65536, "V offsets fit the immediate");
    auto vfrag8 = [&](lds_cptr vst, int db) -> v8i32 {
        v2i32 r[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            r[u] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32*)(vst + 16 * u * T::kVRow + 32 * db));
        return v8i32{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
    };
    f32x16 acc_l8 = f32x16{};
    // O^T and the row sums += V^T P^T of the V stage at vst with the tile's P in pt
    auto pv_tile8 = [&](lds_cptr vst, const v8i32& pt) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc_o[db] = mfma_fp8(vfrag8(vst, db), pt, acc_o[db]);
        acc_l8 = mfma_fp8(ones8, pt, acc_l8);
    };
    // Step of tile jt (stage phase P = jt mod 4): its scores c0, c1 (four fp8 MFMAs), then its
    // softmax beside the five MFMAs of P V of tile jt - 1 (weights pp). The score MFMAs have
    // no vector work of their own to run beside; the other wave of the SIMD supplies it.
    auto step8 = [&](int jt, f32x16& c0, f32x16& c1, const v8i32& pp, v8i32& pc, bool masked,
                     auto with_pv) {
        constexpr bool kPV = decltype(with_pv)::value;
        const int P = jt & 3;  // stage phase (the stage offsets are added at run time here)
        const lds_cptr kc = base_k + P * T::kKStage;                 // K of tile jt
        const lds_cptr vp = base_v8 + ((P + 3) & 3) * T::kVStage;    // V of tile jt - 1
        float t0 = 0.f, t1 = 0.f, t2 = 0.f, t3 = 0.f, t4 = 0.f, alpha = 1.f;
        bool move = false;
        auto val = [&](int v) -> float { return v < 16 ? c0[v] : c1[v - 16]; };
        auto exps = [&](int k0, int k1) {  // pairs k0 .. k1 - 1: exponentials, rounded to e4m3
#pragma unroll
            for (int k = k0; k < k1; ++k) {
                const int w = k >> 1;
                const float x0 = exp2_hw(__builtin_fmaf(val(2 * k), scale_log2, -m_ref));
                const float x1 = exp2_hw(__builtin_fmaf(val(2 * k + 1), scale_log2, -m_ref));
                if (k & 1)
                    pc[w] = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, pc[w], true);
                else
                    pc[w] = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
            }
        };
        auto phase8 = [&](int ph) {
            if (ph == 0) {
                if (__builtin_expect(masked, 0)) {
                    mask_half(c0, 2 * jt, kvq0);
                    mask_half(c1, 2 * jt + 1, kvq0);
                }
                t0 = vmax(vmax(c0[0], c0[1]), c0[2]);
                t1 = vmax(vmax(c0[3], c0[4]), c0[5]);
                t2 = vmax(vmax(c0[6], c0[7]), c0[8]);
                t3 = vmax(vmax(c0[9], c0[10]), c0[11]);
                t4 = vmax(vmax(c0[12], c0[13]), c0[14]);
                t0 = vmax(vmax(t0, t1), t2);
                t3 = vmax(vmax(t3, t4), c0[15]);
            } else if (ph == 1) {
                t1 = vmax(vmax(c1[0], c1[1]), c1[2]);
                t2 = vmax(vmax(c1[3], c1[4]), c1[5]);
                t4 = vmax(vmax(c1[6], c1[7]), c1[8]);
                t1 = vmax(vmax(t1, t2), t4);
                t2 = vmax(vmax(c1[9], c1[10]), c1[11]);
                t4 = vmax(vmax(c1[12], c1[13]), c1[14]);
                t2 = vmax(vmax(t2, t4), c1[15]);
                const float mx = pair32_vmax(vmax(vmax(t0, t3), vmax(t1, t2))) * scale_log2;
                m_run = vmax(m_run, mx);
                move = mx > m_ref + kLazy;
                const float r_new = move ? mx - kV8Head : m_ref;
                alpha = move ? exp2_hw(m_ref - r_new) : 1.f;
                m_ref = r_new;
            } else if (ph == 2) {
                exps(0, 5);
            } else if (ph == 3) {
                exps(5, 10);
            } else {
                exps(10, 16);
            }
        };
        c0 = f32x16{};
        c1 = f32x16{};
        // slots 0-3: S^T of the tile (half sl / 2, 64 head dimensions sl % 2), K operands read one
        // slot ahead; slots 4-8: P V of the previous tile (32 head dimensions each) and its row
        // sums, V operands one slot ahead, beside the softmax phases
        auto operand = [&](int sl) -> v8i32 {
            if (sl < 4) return kfrag8(kc + 32 * (sl >> 1) * T::kKRow, sl & 1);
            return vfrag8(vp, sl - 4);
        };
        v8i32 op[8];
        op[0] = operand(0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int sl = 0; sl < 9; ++sl) {
            if (sl + 1 < 4 || (kPV && sl + 1 < 8)) op[sl + 1] = operand(sl + 1);
            if (sl < 4) {
                if (sl < 2) c0 = mfma_fp8(op[sl], qf8[sl & 1], c0);
                else c1 = mfma_fp8(op[sl], qf8[sl & 1], c1);
            } else if (kPV) {
                if (sl < 8) acc_o[sl - 4] = mfma_fp8(op[sl], pp, acc_o[sl - 4]);
                else acc_l8 = mfma_fp8(ones8, pp, acc_l8);
            }
            if (sl >= 4) phase8(sl - 4);
#pragma unroll
            for (int i = 0; i < T::kDmaPerWave; ++i)
                if (sl == i) dma_op(jt, i, P);
            __builtin_amdgcn_sched_barrier(0);
        }
        asm volatile("" : "+v"(pc));
        if (__builtin_expect(__any(move), 0)) {
#pragma unroll
            for (int i = 0; i < D / 32; ++i) acc_o[i] *= alpha;
            acc_l8 *= alpha;
        }
    };

    advance(3);
    v8i32 pa8 = {}, pb8 = {};
    step8(0, sa, sb, pb8, pa8, n_plain == 0, No{});
    wait_dma_tile();
    barrier_lds();
    // tiles 1 .. n_tiles - 1, two per iteration (odd tiles write pb8, even ones pa8); the
    // accumulators leave the loop by one exit only
    auto tile8 = [&](int jt, auto odd_c) {
        advance(jt + 3);
        const bool masked = jt >= n_plain;
        if constexpr (decltype(odd_c)::value)
            step8(jt, sa, sb, pa8, pb8, masked, Yes{});
        else
            step8(jt, sa, sb, pb8, pa8, masked, Yes{});
        wait_dma_tile();
        barrier_lds();
    };
    int jt = 1;
    for (; jt + 1 < n_tiles; jt += 2) {
        tile8(jt, Yes{});
        tile8(jt + 1, No{});
    }
    if (jt < n_tiles) {
        tile8(jt, Yes{});
        ++jt;
    }
    // the last tile's O update (tile n_tiles - 1: odd ones wrote pb8)
    pv_tile8(base_v8 + ((n_tiles - 1) & 3) * T::kVStage, ((n_tiles - 1) & 1) ? pb8 : pa8);
    l_part = acc_l8[0];  // every row of acc_l holds the query's row sum (both lane halves)
    } else {
    compute_s(sa, 0, 0);

    // ---- tile 0: half 0 has no O update yet; its first step issues K3 / V2 ----
    {
        const Bases b0 = bases(std::integral_constant<int, 0>{});
        if constexpr (kFp8) {
            // step 0 has no O update; its S^T (half tile 1) takes K from the first stage
#pragma unroll
            for (int sl = 0; sl < kAh; ++sl) fr[sl] = bf16x8{};
#pragma unroll
            for (int c = 0; c < D / 64; ++c) kq[c] = kfrag8(b0.k, c);
        } else {
#pragma unroll
            for (int sl = 0; sl < kAh; ++sl) fr[sl] = slot_is_s(sl) ? frag(b0, sl) : bf16x8{};
        }
    }
    advance(3);
    if constexpr (!kStats && !kV8) {
        // Without statistics the exponent reference is fixed for the whole item at the row
        // maximum of the first half tile's admissible scores (a row with none there starts at
        // -1e30). It is a maximum of real scores, so the row's largest weight stays at least 1
        // and a weight that underflows is negligible next to it; a score far above it makes
        // the row sum overflow, which the end of the item detects.
        const bool masked0 = kSparse ? kvq0 >= n_plain * kBc : n_plain == 0;
        f32x16 t = sa;
        if (masked0) mask_half(t, 0, kvq0);
        float u = t[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) u = vmax(u, t[r]);
        u = pair32_vmax(u) * (kPre ? 1.f : scale_log2);
        m_ref = u > -1e30f ? u : -1e30f;
        if constexpr (kPre) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                negm[r] = -m_ref;
                sa[r] -= m_ref;  // (the first half tile's products started from zero)
            }
        }
    }
    {
        const bool masked0 = kSparse ? kvq0 >= n_plain * kBc : n_plain == 0;
        step(0, kvq0, std::integral_constant<int, 0>{}, sa, sb, pb, pa, masked0, fr, kq, No{}, Yes{});
        step(1, kvq0, std::integral_constant<int, 1>{}, sb, sa, pa, pb, masked0, fr, kq, Yes{}, No{});
    }
    wait_dma_tile();
    barrier_lds();

    // ---- tiles 1 .. n_tiles-1. Tile j reads K_j (half 1), K_{j+1} (half 0), V_{j-1}
    // (half 1) and V_j (half 0). Its first step issues the loads of K_{j+3} and V_{j+2}
    // into the stages of K_{j-1} and V_{j-2}, both last read during tile j-1, before the
    // previous barrier; they have until the barrier that ends tile j+1 to land (the wait
    // before each barrier leaves only the newest tile's loads in flight). The loop is
    // unrolled over the four stage phases (it starts at j = 1). ----
    auto tile = [&](int j, auto phase_c) {
        constexpr int P = decltype(phase_c)::value;
        advance(j + 3);
        const bool masked = kSparse ? kvq0 >= n_plain * kBc : j >= n_plain;
        step(2 * j, kvq0, std::integral_constant<int, 2 * P>{}, sa, sb, pb, pa, masked, fr, kq, Yes{}, Yes{});
        step(2 * j + 1, kvq0, std::integral_constant<int, 2 * P + 1>{}, sb, sa, pa, pb, masked, fr, kq, Yes{}, No{});
        wait_dma_tile();
        barrier_lds();
    };
    // (kSkip) the wave's steps end with tile j_stop - 1: from there on the half tiles are past
    // its last visible key (the last step run, half tile 2 j_stop - 1, is too, so its weights
    // are zero and nothing is left for the O update that would follow)
    const int j_stop = kSkip ? min_(n_tiles, max_(1, (h_last + 3) >> 1)) : n_tiles;
    int j = 1;
    while (j < j_stop) {
        tile(j, std::integral_constant<int, 1>{});
        if (++j >= j_stop) break;
        tile(j, std::integral_constant<int, 2>{});
        if (++j >= j_stop) break;
        tile(j, std::integral_constant<int, 3>{});
        if (++j >= j_stop) break;
        tile(j, std::integral_constant<int, 0>{});
        ++j;
    }
    if constexpr (kSkip) {
        // the item's remaining tiles: the wave's share of their loads and the barriers only
        auto idle_tile = [&](int jj, auto phase_c) {
            constexpr int P = decltype(phase_c)::value;
            advance(jj + 3);
#pragma unroll
            for (int i = 0; i < T::kDmaPerWave; ++i) dma_op(jj, i, P);
            wait_dma_tile();
            barrier_lds();
        };
        for (; j < n_tiles; ++j) {
            switch (j & 3) {
                case 0: idle_tile(j, std::integral_constant<int, 0>{}); break;
                case 1: idle_tile(j, std::integral_constant<int, 1>{}); break;
                case 2: idle_tile(j, std::integral_constant<int, 2>{}); break;
                default: idle_tile(j, std::integral_constant<int, 3>{}); break;
            }
        }
    }
    // last half tile's O update (its S^T step computed a score block past the end, unused)
    if (j_stop >= n_tiles) switch ((n_tiles - 1) & 3) {
        case 0: compute_pv(pb, 0, 1); break;
        case 1: compute_pv(pb, 1, 1); break;
        case 2: compute_pv(pb, 2, 1); break;
        default: compute_pv(pb, 3, 1); break;
    }
    }
    wait_dma_all();  // no load may still be writing LDS when the item ends
    barrier_lds();   // and no wave still reads it when the next item's loads start
    }
    // ---- epilogue: O / l, bf16, optional row statistics ----
    float l_tot = kV8 ? l_part : pair32_sum(l_part);
    if constexpr (kPaged) {
        // a query before the sequence's first key (causal, L < Nq) or an empty sequence:
        // O = 0, m = -inf, l = 0 (its lanes ran on scores that were all masked)
        if (Nk <= 0 || (causal && qrow + off < 0)) {
            l_tot = 0.f;
#pragma unroll
            for (int i = 0; i < D / 32; ++i) acc_o[i] = f32x16{};
        }
    }
    {
        // O / l in bf16, through LDS: the wave writes its 32 rows row-major into a block of its
        // own in the stage area (idle now: no load in flight, no wave reading it), then stores
        // whole rows, 16 bytes a lane, so that one store instruction fills 1 KiB of O (the
        // accumulator layout alone gives a lane 8 bytes in each of 16 places). Chunk c of row r
        // sits at c ^ osw(r).
        constexpr int kRowB = 2 * D, kCh = kRowB / 16, kRowsPer = 1024 / kRowB;
        typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
        typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
        typedef __attribute__((address_space(3))) unsigned char* lds_ptr;
        lds_ptr const ob = (lds_ptr)smem + wave * 32 * kRowB;
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        const int sw_w = osw<D>(l32);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w = {pack_bf16x2(acc_o[db][4 * g] * inv, acc_o[db][4 * g + 1] * inv),
                           pack_bf16x2(acc_o[db][4 * g + 2] * inv, acc_o[db][4 * g + 3] * inv)};
                *(lds_u32x2*)(ob + l32 * kRowB + 16 * ((4 * db + g) ^ sw_w) + 8 * hh) = w;
            }
        // (a wave's LDS accesses complete in order: its reads below see all its lanes' writes)
        __builtin_amdgcn_wave_barrier();
        const int rr = lane / kCh, ch = lane % kCh;
#pragma unroll
        for (int i = 0; i < 32 / kRowsPer; ++i) {
            const int r = kRowsPer * i + rr;
            const u32x4 val = *(const lds_u32x4*)(ob + r * kRowB + 16 * (ch ^ osw<D>(r)));
            if (row0 + r < nq) *reinterpret_cast<u32x4*>(o + qoff + (size_t)(row0 + r) * D + 8 * ch) = val;
        }
    }
    if (qrow < nq) {
        if (hh == 0) {
            const size_t ridx = (size_t)(b * Hq + h) * N + qrow;
            if (m_out) m_out[ridx] = (l_tot > 0.f) ? m_run * kLn2 : -INFINITY;
            if (l_out) l_out[ridx] = (l_tot > 0.f) ? l_tot * exp2_hw(m_ref - m_run) : 0.f;
        }
    }
    if constexpr (!kStats && !kV8) {
        // Every weight stayed at most 2^100 (and finite) iff the row sums did: then no
        // product overflowed. Otherwise the whole workgroup runs the item again with
        // statistics, which rewrites every output row the garbage above went to (the decision
        // must be uniform: the item's loads and barriers are shared).
        // Each wave reports in one word of the tile area past the O blocks, idle at this point
        // (no load in flight, no wave reading it); the second barrier keeps the next item's
        // loads from overwriting the words (and the O blocks) before every wave is done with
        // them.
        int* flags = reinterpret_cast<int*>(smem + kWaves * 32 * 2 * D);
        const bool bad = __any(!(l_part <= 0x1p100f));
        if ((threadIdx.x & 63) == 0) flags[wave] = bad ? 1 : 0;
        barrier_lds();
        int any = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) any |= flags[w];
        barrier_lds();
        if (any) return false;
    } else {
        barrier_lds();  // the next item's loads wait until every wave has read its O block
    }

    return true;
}

// Persistent grid: one workgroup per CU (two for dense d = 64), a multiple of the 8
// XCDs. Workgroup w runs on XCD w mod 8 and walks the x-th contiguous eighth of the work
// list (so one KV group's tiles are re-read from one XCD's L2), taking its items in snake
// order over the XCD's workgroups: round r gives the workgroup of local index j the item
// r * W + j (r even) or r * W + W - 1 - j (r odd). The list runs heaviest query block first,
// so the snake pairs heavy with light items and the workgroups finish together; and a
// workgroup moves to its next item without a new launch.
// Workgroups per CU: two for the dense d = 64 instance (its swizzled stages take 64 KiB of
// LDS and it fits 128 registers a wave); one otherwise (the paged and block-sparse d = 64
// instances would spill at 128 registers).
template <int D, int kMode>
constexpr int kWgPerCu = D == 64 && Tile<D, false>::kSwz && kMode == kModeDense ? 2 : 1;

// (the second bound is the waves per SIMD the register budget must allow)
template <int D, int kMode, bool kStats>
__global__ __launch_bounds__(kThreads, (kWgPerCu<D, kMode> * kWaves / 4)) void fwd_bf16_sp_kernel(FwdArgs a) {
    using T = Tile<D, kMode == kModePaged, kMode == kModeFp8 || kMode == kModeFp8V, kMode == kModeFp8V>;
    __shared__ __attribute__((aligned(16)))
    unsigned char smem[kMode == kModeDense ? T::kLdsQ : kStages * (T::kKStage + T::kVStage)];

    const int per_unit = a.nqb * (a.Hq / a.Hkv);  // items of one KV group
    const int n_kvg = a.B * a.Hkv;
    const int total = n_kvg * per_unit;
    const int xcd = (int)(blockIdx.x % kXcds), j = (int)(blockIdx.x / kXcds);
    const int W = (int)(gridDim.x / kXcds);
    // Dense: XCD x takes the x-th contiguous eighth of the list. Paged and block-sparse: XCD x
    // takes the KV groups g = x, x + 8, ..., so every XCD gets a share of every sequence (or
    // head) whatever their lengths or block lists (a KV group's items stay on one XCD).
    int seg0 = 0, seg_n;
    if constexpr (kMode != kModeDense) {
        seg_n = (n_kvg > xcd ? (n_kvg - xcd + kXcds - 1) / kXcds : 0) * per_unit;
    } else {
        const int per_xcd = (total + kXcds - 1) / kXcds;
        seg0 = xcd * per_xcd;
        seg_n = min_(per_xcd, total - seg0);
    }
    // Two workgroups per CU: local ids j and j + W / 2 are taken to share a CU, so the snake
    // runs over W / 2 units whose rounds alternate between the two (a heavy item on one of
    // them, the matching light one on the other). The first of the two to start (the lower
    // id) takes the heavy item: the waves that started first win the CU's instruction issue,
    // so the heavy item runs at the pace of a workgroup alone and the light one in the gaps.
    // For that the XCD's share, when it is whole KV groups, is walked by query block first
    // (all its groups' heaviest blocks, then the next), so that the first W / 2 items are the
    // heavy half.
    constexpr int kPer = kWgPerCu<D, kMode>;
    const int Wu = W / kPer, u = j % Wu, sub = j / Wu;
    const int G = a.Hq / a.Hkv;
    const bool by_block = kPer == 2 && seg0 % per_unit == 0 && seg_n % per_unit == 0;
    const int seg_units = seg_n / per_unit;
    for (int r = 0; r * W < seg_n; ++r) {
        const int rr = kPer * r + sub;  // the unit's round
        const int local = rr * Wu + ((rr & 1) ? Wu - 1 - u : u);
        if (local >= seg_n) continue;
        int item;
        if constexpr (kMode != kModeDense) {
            const int g = local / per_unit;
            item = (xcd + kXcds * g) * per_unit + (local - g * per_unit);
        } else if (by_block) {
            // local = (t * units + k) * G + hg: block rank t of unit k, head hg of the group
            const int t = local / (seg_units * G), rem = local - t * seg_units * G;
            const int k = rem / G, hg = rem - k * G;
            item = seg0 + k * per_unit + t * G + hg;
        } else {
            item = seg0 + local;
        }
        if (!fwd_item<D, kMode, kStats>(a, item, smem)) fwd_item<D, kMode, true>(a, item, smem);
    }
}

}  // namespace

namespace {
template <int kMode>
hipError_t launch_sp(const FwdArgs& a, int d, hipStream_t stream) {
    const long long items = (long long)a.nqb * a.B * a.Hq;
    // (dense d = 64: two workgroups per CU; the grid is a multiple of 8 x that count, so that
    // every XCD's workgroups pair up)
    const int per_cu = d == 64 ? kWgPerCu<64, kMode> : 1;
    const long long unit = (long long)kXcds * per_cu;
    const long long slots = (long long)(device_cus() / kXcds) * unit;
    long long grid = (items + unit - 1) / unit * unit;
    if (grid > slots) grid = slots;
    const bool stats = a.m_out != nullptr || a.l_out != nullptr;
    const dim3 g((unsigned)grid), blk(kThreads);
    if (d == 128) {
        if (stats)
            hipLaunchKernelGGL((fwd_bf16_sp_kernel<128, kMode, true>), g, blk, 0, stream, a);
        else
            hipLaunchKernelGGL((fwd_bf16_sp_kernel<128, kMode, false>), g, blk, 0, stream, a);
    } else if constexpr (kMode != kModeFp8 && kMode != kModeFp8V) {
        if (stats)
            hipLaunchKernelGGL((fwd_bf16_sp_kernel<64, kMode, true>), g, blk, 0, stream, a);
        else
            hipLaunchKernelGGL((fwd_bf16_sp_kernel<64, kMode, false>), g, blk, 0, stream, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
}  // namespace

hipError_t launch_fwd_bf16_sp(const void* q, const void* k, const void* v, void* o, float* m_out,
                              float* l_out, int B, int Hq, int Hkv, int N, int d, float scale,
                              int causal, hipStream_t stream) {
    FwdArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.o = static_cast<uint16_t*>(o);
    a.m_out = m_out;
    a.l_out = l_out;
    a.B = B, a.Hq = Hq, a.Hkv = Hkv, a.N = N;
    a.scale_log2 = scale * kLog2e;
    a.causal = causal;
    a.nqb = (N + kBr - 1) / kBr;
    return launch_sp<kModeDense>(a, d, stream);
}

hipError_t launch_fwd_bf16_sp_paged(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    const int32_t* q_lens, void* o,
                                    float* m_out, float* l_out, int B, int Hq, int Hkv, int Nq,
                                    int d, int num_pages, int max_pages_per_seq, float scale,
                                    int causal, hipStream_t stream) {
    FwdArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k_cache);
    a.v = static_cast<const uint16_t*>(v_cache);
    a.o = static_cast<uint16_t*>(o);
    a.m_out = m_out;
    a.l_out = l_out;
    a.table = block_table;
    a.lens = seq_lens;
    a.q_lens = q_lens;
    a.B = B, a.Hq = Hq, a.Hkv = Hkv, a.N = Nq;
    a.scale_log2 = scale * kLog2e;
    a.causal = causal;
    a.nqb = (Nq + kBr - 1) / kBr;
    a.max_pages = max_pages_per_seq;
    a.num_pages = num_pages;
    return launch_sp<kModePaged>(a, d, stream);
}

hipError_t launch_fwd_fp8qk_sp(const void* q, const void* k, const void* v, int v_fp8, void* o,
                               float* m_out, float* l_out, int B, int Hq, int Hkv, int N, int d,
                               float scale, int causal, hipStream_t stream) {
    FwdArgs a{};
    a.q = static_cast<const uint16_t*>(q);  // e4m3 bytes, addressed as such in the kernel
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.o = static_cast<uint16_t*>(o);
    a.m_out = m_out;
    a.l_out = l_out;
    a.B = B, a.Hq = Hq, a.Hkv = Hkv, a.N = N;
    a.scale_log2 = scale * kLog2e;
    a.causal = causal;
    a.nqb = (N + kBr - 1) / kBr;
    return v_fp8 ? launch_sp<kModeFp8V>(a, d, stream) : launch_sp<kModeFp8>(a, d, stream);
}

hipError_t launch_fwd_bf16_sp_block_sparse(const void* q, const void* k, const void* v, void* o,
                                           float* m_out, float* l_out, const int32_t* block_offsets,
                                           const int32_t* block_indices, int nnz, int B, int Hq,
                                           int Hkv, int N, int d, float scale, int causal,
                                           hipStream_t stream) {
    FwdArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.o = static_cast<uint16_t*>(o);
    a.m_out = m_out;
    a.l_out = l_out;
    a.blk_off = block_offsets;
    a.blk_idx = block_indices;
    a.nnz = nnz;
    a.B = B, a.Hq = Hq, a.Hkv = Hkv, a.N = N;
    a.scale_log2 = scale * kLog2e;
    a.causal = causal;
    a.nqb = (N + kBr - 1) / kBr;
    return launch_sp<kModeSparse>(a, d, stream);
}

}  // namespace fa
