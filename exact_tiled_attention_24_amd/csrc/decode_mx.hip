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
//  * At the end the waves' states are merged through LDS. A sequence of one chunk writes its
//    output directly. Otherwise each chunk writes a normalised float32 partial (m in log2
//    units, l, O) per query head to the workspace and counts itself done on the completion
//    word of its (sequence, KV head); the last chunk to arrive merges the partials with the
//    same rule, in chunk order (so the result does not depend on which chunk is last), and
//    writes the output. No second launch.
//  * The completion word holds a tag of the call in its high bits and the arrivals in the low
//    bits: an arrival that finds another tag counts as the first, so the words need no
//    clearing between calls and the workspace contents on entry do not matter. The last
//    arrival leaves the word at zero, so that a call replayed with the same tag (a captured
//    graph's launch) also starts from a clean count.
#include <atomic>
#include <mutex>
#include <random>

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
constexpr int kWaves = 4;                       // waves per workgroup
constexpr int kSlots = 2;                       // page slots per wave (one page in flight)
constexpr int kThreads = 64 * kWaves;
constexpr int kCountBits = 24;                  // completion word: tag << 24 | arrivals
constexpr unsigned long long kCountMask = (1ull << kCountBits) - 1;

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

struct DecodeArgs {
    const uint16_t* q;
    const uint16_t* kc;
    const uint16_t* vc;
    const int32_t* table;
    const int32_t* lens;
    uint16_t* o;
    float* ws_o;                // partial O [S][B * Hq][d], normalised
    float* ws_m;                // partial m [S][B * Hq], log2 units
    float* ws_l;                // partial l [S][B * Hq]
    unsigned long long* done;   // completion words [B * Hkv]
    unsigned long long tag;     // this call's tag, < 2^40
    int B, Hq, Hkv, G, num_pages, max_pages, len_cap, chunk_pages;
    float scale_log2;
};

// Counts one arrival on a completion word and reports whether it was the n-th of this call
// (the n-th clears the word: zero counts as no arrival for any tag).
// Vector (global) atomics at device scope, relaxed. The caller orders the partials around it
// without fences: every wave waits for its partial stores to complete (s_waitcnt vmcnt(0))
// before the barrier behind which one thread arrives, and the last arriver's loads of the
// other partials are issued only after its exchange has returned. The loop ends because every
// failed exchange means another workgroup's arrival succeeded.
__device__ bool arrive(unsigned long long* word, unsigned long long tag, int n) {
    unsigned long long old = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (;;) {
        const unsigned long long cnt = (old >> kCountBits) == tag ? (old & kCountMask) : 0;
        const unsigned long long next = cnt + 1 == (unsigned long long)n ? 0ull : (tag << kCountBits) | (cnt + 1);
        if (__hip_atomic_compare_exchange_strong(word, &old, next, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            return cnt + 1 == (unsigned long long)n;
    }
}

// Partial values go through device-scope stores and loads: coherent across the XCDs' L2s
// on their own, without a cache write-back or invalidate.
__device__ __forceinline__ void publish(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float collect(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(kThreads) void decode_mx_kernel(DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[kWaves * kSlots * kSlot];
    __shared__ int last_flag;
    lds_cptr const lds = (lds_cptr)smem;
    const unsigned lds_addr = (unsigned)(size_t)lds;
    const int Hq = a.Hq, Hkv = a.Hkv, G = a.G, num_pages = a.num_pages;
    const float scale_log2 = a.scale_log2;

    // x = sequence x KV head, y = chunk. Workgroups are dealt to the XCDs by linear id, so
    // XCD x streams KV head x (mod 8) of every page: measured faster than spreading each
    // XCD over all KV heads (150 against 158 us on the decode workload).
    const int split = blockIdx.y;
    const int bk = blockIdx.x;
    const int b = bk / Hkv;
    const int kvh = bk - b * Hkv;
    const int R = a.B * Hq;
    const int row0 = b * Hq + kvh * G;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
    const int lane = tid & 63;
    const int l16 = lane & 15;  // query column (S^T, P) / head dimension in a block (O)
    const int g4 = lane >> 4;   // token group: tokens 4 g4 .. 4 g4 + 3

    // Q as the B operand of S^T = K Q^T: lane l holds query l16, dims 32 m + 8 g4 .. +7,
    // requested before the length is known. Columns l16 >= G repeat query G - 1: they yield
    // finite duplicates of its scores and output rows, which are never written.
    bf16x8 qb[kD / 32];
    {
        const uint16_t* qrow = a.q + (size_t)(row0 + min_(l16, G - 1)) * kD + 8 * g4;
#pragma unroll
        for (int m = 0; m < kD / 32; ++m) qb[m] = *reinterpret_cast<const bf16x8*>(qrow + 32 * m);
    }

    int L = a.lens[b];
    L = L < 0 ? 0 : (L > a.len_cap ? a.len_cap : L);
    const int npages = (L + kPage - 1) / kPage;
    // This sequence gets ceil(npages / chunk_pages) chunks of near-equal size (they differ by
    // at most one page). Workgroups past its chunk count have nothing to do; an empty
    // sequence keeps chunk 0, which writes O = 0.
    const int n_chunks = (npages + a.chunk_pages - 1) / a.chunk_pages;
    if (split >= max_(n_chunks, 1)) return;
    const int p_begin = n_chunks > 0 ? (int)((long long)split * npages / n_chunks) : 0;
    const int p_end = n_chunks > 0 ? (int)((long long)(split + 1) * npages / n_chunks) : 0;

    f32x4 acc[kD / 16];  // O: lane holds queries 4 g4 + r, dims 16 blk + l16
#pragma unroll
    for (int i = 0; i < kD / 16; ++i) acc[i] = f32x4{};
    float m_ref = -INFINITY;  // exponent reference of query l16 (equal in its four lanes)
    float lsum = 0.f;         // this lane's part of query l16's sum

    const int n_mine = p_end - p_begin > wave ? (p_end - p_begin - wave + kWaves - 1) / kWaves : 0;
    if (n_mine > 0 && num_pages > 0) {
        // Q as the B operand of S^T = K Q^T: lane l holds query l16 (zero past G), dims
        // 32 m + 8 g4 .. +7.

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
        const int32_t* trow = a.table + (size_t)b * a.max_pages;
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
                __builtin_amdgcn_make_buffer_rsrc((void*)(a.kc + off), (short)0, bytes, kBufferDword3);
            const __amdgpu_buffer_rsrc_t rv =
                __builtin_amdgcn_make_buffer_rsrc((void*)(a.vc + off), (short)0, bytes, kBufferDword3);
            const unsigned dst = wave_lds + s * kSlot;
            // Non-temporal loads: each page of the call is read once, so its lines need not
            // stay in the caches, and streaming them does not evict what other work left there
            // (with a forward's output still dirty in the Infinity Cache, the decode otherwise
            // pays for its write-back: measured 157.6 against 136.4 us after a long-prefill
            // forward, and 151.5 against 135.4 us alone).
#pragma unroll
            for (int c = 0; c < kPiece / 1024; ++c)
                asm volatile("buffer_load_dwordx4 %0, %1, 0 offen nt lds"
                             :
                             : "v"(ksrc[c]), "s"(rk), "{m0}"(dst + 1024 * c)
                             : "memory");
#pragma unroll
            for (int c = 0; c < kPiece / 1024; ++c)
                asm volatile("buffer_load_dwordx4 %0, %1, 0 offen nt lds"
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
                    const float f = __shfl(alpha, 4 * g4 + r);
#pragma unroll
                    for (int blk = 0; blk < kD / 16; ++blk) acc[blk][r] *= f;
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

    // ---- merge the waves (lanes of a query: l16 = g, all g4) ----
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
    // This chunk's (m, l, O) per query head: thread idx handles (g, d) = divmod(idx, kD).
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
        const float od = lt > 0.f ? ot / lt : 0.f;
        if (n_chunks <= 1) {
            // the sequence's only chunk: this is the output
            a.o[(size_t)(row0 + g) * kD + d] = (uint16_t)(pack_bf16x2(od, 0.f) & 0xffffu);
        } else {
            const size_t prow = (size_t)split * R + row0 + g;
            publish(a.ws_o + prow * kD + d, od);
            if (d == 0) {
                publish(a.ws_m + prow, lt > 0.f ? m : -INFINITY);
                publish(a.ws_l + prow, lt);
            }
        }
    }
    if (n_chunks <= 1) return;

    // ---- count this chunk done; the last of the (sequence, KV head) merges ----
    // The partials were written with device-scope stores, which complete only once they are
    // visible to every XCD; each wave waits for its own, so after the barrier the whole
    // partial is visible before the arrival is counted. The merging workgroup reads the
    // partials with device-scope loads, which do not hit stale lines of its XCD's L2. (A
    // device-scope release / acquire pair would write back and invalidate whole L2s, which
    // stalls the XCDs while other workgroups still stream.)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) last_flag = arrive(a.done + bk, a.tag, n_chunks) ? 1 : 0;
    __syncthreads();
    if (!last_flag) return;

    // m = max_s m_s over the partials that hold weight; w_s = l_s 2^(m_s - m);
    // O = sum_s w_s O_s / sum_s w_s, taken in chunk order (the result does not depend on
    // which chunk arrived last). Chunks go in groups of 8 whose loads are issued together; a
    // group that raises the maximum rescales the running sums.
    constexpr int kGroup = 8;
    for (int idx = tid; idx < G * kD; idx += kThreads) {
        const int g = idx / kD, d = idx - g * kD;
        const size_t row = (size_t)row0 + g;
        float M = -INFINITY, lt = 0.f, ot = 0.f;
        for (int s0 = 0; s0 < n_chunks; s0 += kGroup) {
            float ms[kGroup], ls[kGroup], os[kGroup];
#pragma unroll
            for (int j = 0; j < kGroup; ++j) {
                const size_t prow = (size_t)min_(s0 + j, n_chunks - 1) * R + row;  // (clamped)
                ms[j] = collect(a.ws_m + prow);
                ls[j] = collect(a.ws_l + prow);
                os[j] = collect(a.ws_o + prow * kD + d);
            }
            float mb = M;
#pragma unroll
            for (int j = 0; j < kGroup; ++j)
                if (s0 + j < n_chunks && ls[j] > 0.f) mb = fmaxf(mb, ms[j]);
            if (mb == -INFINITY) continue;
            const float f = M == -INFINITY ? 0.f : exp2_hw(M - mb);
            lt *= f;
            ot *= f;
#pragma unroll
            for (int j = 0; j < kGroup; ++j) {
                if (s0 + j < n_chunks && ls[j] > 0.f) {
                    const float w = ls[j] * exp2_hw(ms[j] - mb);
                    lt += w;
                    ot = __builtin_fmaf(w, os[j], ot);
                }
            }
            M = mb;
        }
        const float od = lt > 0.f ? ot / lt : 0.f;
        a.o[row * kD + d] = (uint16_t)(pack_bf16x2(od, 0.f) & 0xffffu);
    }
}

// Scratch of the allocation-free entry point: the completion words and partials of one call
// (the same layout as a caller's workspace), resident on every device the library runs on
// until the process ends. Host code never uses this name as an address: the device address
// comes from hipGetSymbolAddress, once per device (see decode_scratch).
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// A tag no earlier call of this process used: a per-process random start plus a call count,
// kept to 40 bits (the completion word's high bits).
unsigned long long next_tag() {
    static std::atomic<unsigned long long> count{0};
    static const unsigned long long start = [] {
        std::random_device rd;
        return ((unsigned long long)rd() << 32) ^ rd();
    }();
    return (start + count.fetch_add(1, std::memory_order_relaxed)) & ((1ull << 40) - 1);
}

}  // namespace

size_t decode_scratch_bytes() { return kScratchBytes; }

hipError_t decode_scratch(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with `dev` current
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_decode_bf16_mx(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_table, const int32_t* seq_lens, void* o,
                                 int B, int Hq, int Hkv, int d, int num_pages,
                                 int max_pages_per_seq, int len_cap, float scale, int splits,
                                 int chunk_pages, const DecodeWorkspace& ws, hipStream_t stream) {
    (void)d;
    DecodeArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.kc = static_cast<const uint16_t*>(k_cache);
    a.vc = static_cast<const uint16_t*>(v_cache);
    a.table = block_table;
    a.lens = seq_lens;
    a.o = static_cast<uint16_t*>(o);
    a.ws_o = ws.o;
    a.ws_m = ws.m;
    a.ws_l = ws.l;
    a.done = ws.done;
    a.tag = next_tag();
    a.Hq = Hq, a.Hkv = Hkv, a.G = Hq / Hkv;
    a.num_pages = num_pages, a.max_pages = max_pages_per_seq, a.len_cap = len_cap;
    a.chunk_pages = chunk_pages;
    a.B = B;
    a.scale_log2 = scale * kLog2e;
    hipLaunchKernelGGL(decode_mx_kernel, dim3((unsigned)(B * Hkv), (unsigned)splits),
                       dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace fa
