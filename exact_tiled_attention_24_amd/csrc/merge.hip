// merge.hip - merge partial (m, l, O) results over disjoint key sets.
//
// Method: "FlashAttention" (shubhamtatvamasi.com), "Decode is a different problem": each KV
// chunk produces a partial (m, l, O), merged with the same rule as the running update of
// "The trick: tiles and an online softmax": with m = max_s m_s and w_s = l_s e^(m_s - m),
// l = sum_s w_s and O = sum_s w_s O_s / l, where O_s is the chunk's normalised output.
//
// The partials of a row are combined in a fixed order, so the result is deterministic.
#include "fa_internal.hpp"
#include "gfx950.hpp"

namespace fa {
namespace {

constexpr int kLanes = 64;

// One 64-lane workgroup per row, columns c = lane + 64 k. The partials are combined with the
// online rule in batches of 8: all loads of a batch are issued first, then
//   M' = max(M, m_s), Lsum' = Lsum e^(M - M') + l_s e^(m_s - M'), acc' likewise with l_s O_s,
// so a row costs one memory round trip per batch. Empty partials (l_s = 0) are skipped.
template <int CPL>
__global__ __launch_bounds__(kLanes) void merge_kernel(
    const float* __restrict__ o_parts, const float* __restrict__ m_parts,
    const float* __restrict__ l_parts, void* __restrict__ o, int out_bf16,
    float* __restrict__ m_out, float* __restrict__ l_out, int S, int R, int d, int log2_units) {
    constexpr int kBatch = 8;
    const int row = blockIdx.x;
    const int lane = threadIdx.x;
    auto ex = [&](float x) { return log2_units ? exp2_hw(x) : expf(x); };

    float M = -INFINITY, lsum = 0.f;
    float acc[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) acc[k] = 0.f;

    for (int s0 = 0; s0 < S; s0 += kBatch) {
        float ls[kBatch], ms[kBatch], ov[kBatch][CPL];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int s = min_(s0 + u, S - 1);  // clamped reads; extra ones are skipped below
            const size_t i = (size_t)s * R + row;
            ls[u] = l_parts[i];
            ms[u] = m_parts[i];
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                const int c = min_(lane + kLanes * k, d - 1);
                ov[u][k] = o_parts[i * d + c];
            }
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (s0 + u < S && ls[u] > 0.f) {
                const float mn = fmaxf(M, ms[u]);
                const float a = M == -INFINITY ? 0.f : ex(M - mn);
                const float w = ls[u] * ex(ms[u] - mn);
                lsum = lsum * a + w;
#pragma unroll
                for (int k = 0; k < CPL; ++k) acc[k] = __builtin_fmaf(w, ov[u][k], acc[k] * a);
                M = mn;
            }
        }
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const int c = lane + kLanes * k;
        if (c < d) {
            const float out = acc[k] * inv;
            if (out_bf16)
                static_cast<uint16_t*>(o)[(size_t)row * d + c] = (uint16_t)(pack_bf16x2(out, 0.f) & 0xffffu);
            else
                static_cast<float*>(o)[(size_t)row * d + c] = out;
        }
    }
    if (lane == 0) {
        const float m_nat = lsum > 0.f ? (log2_units ? M * kLn2 : M) : -INFINITY;
        if (m_out) m_out[row] = m_nat;
        if (l_out) l_out[row] = lsum;
    }
}

}  // namespace

hipError_t launch_merge(const float* o_parts, const float* m_parts, const float* l_parts, void* o,
                        int out_bf16, float* m_out, float* l_out, int S, int R, int d,
                        int log2_units, hipStream_t stream) {
    if (R == 0) return hipSuccess;
    const int cpl = (d + kLanes - 1) / kLanes;  // columns per lane, d <= 1024
#define FA_MERGE_LAUNCH(C)                                                                       \
    hipLaunchKernelGGL(merge_kernel<C>, dim3((unsigned)R), dim3(kLanes), 0, stream, o_parts,     \
                       m_parts, l_parts, o, out_bf16, m_out, l_out, S, R, d, log2_units)
    if (cpl <= 1) FA_MERGE_LAUNCH(1);
    else if (cpl <= 2) FA_MERGE_LAUNCH(2);
    else if (cpl <= 4) FA_MERGE_LAUNCH(4);
    else if (cpl <= 8) FA_MERGE_LAUNCH(8);
    else FA_MERGE_LAUNCH(16);
#undef FA_MERGE_LAUNCH
    return hipGetLastError();
}

}  // namespace fa
