// merge.hip - merge partial (m, l, O) results over disjoint key sets.
//
// Method: "FlashAttention" (shubhamtatvamasi.com), "Decode is a different problem": each KV
// chunk produces a partial (m, l, O), merged with the same rule as the running update of
// "The trick: tiles and an online softmax": with m = max_s m_s and w_s = l_s e^(m_s - m),
// l = sum_s w_s and O = sum_s w_s O_s / l, where O_s is the chunk's normalised output.
//
// One 64-lane workgroup per row: the lanes first reduce max and sum over the partials of
// the row, then each lane accumulates its columns over all partials in a fixed order, so
// the result is deterministic. Partial weights are cached in LDS when S fits.
#include "fa_internal.hpp"
#include "gfx950.hpp"

namespace fa {
namespace {

constexpr int kLanes = 64;
constexpr int kCachedWeights = 2048;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

__global__ __launch_bounds__(kLanes) void merge_kernel(
    const float* __restrict__ o_parts, const float* __restrict__ m_parts,
    const float* __restrict__ l_parts, void* __restrict__ o, int out_bf16,
    float* __restrict__ m_out, float* __restrict__ l_out, int S, int R, int d, int log2_units) {
    __shared__ float wts[kCachedWeights];
    const int row = blockIdx.x;
    const int lane = threadIdx.x;

    auto ex = [&](float x) { return log2_units ? exp2_hw(x) : expf(x); };

    float mx = -INFINITY;
    for (int s = lane; s < S; s += kLanes) {
        const size_t i = (size_t)s * R + row;
        if (l_parts[i] > 0.f) mx = fmaxf(mx, m_parts[i]);
    }
    mx = wave_max(mx);

    float lt = 0.f;
    if (mx != -INFINITY) {
        for (int s = lane; s < S; s += kLanes) {
            const size_t i = (size_t)s * R + row;
            const float w = l_parts[i] > 0.f ? l_parts[i] * ex(m_parts[i] - mx) : 0.f;
            if (s < kCachedWeights) wts[s] = w;
            lt += w;
        }
    }
    lt = wave_sum(lt);
    __syncthreads();
    const float inv = lt > 0.f ? 1.f / lt : 0.f;

    for (int c = lane; c < d; c += kLanes) {
        float acc = 0.f;
        if (lt > 0.f) {
            for (int s = 0; s < S; ++s) {
                float w;
                if (s < kCachedWeights) {
                    w = wts[s];
                } else {
                    const size_t i = (size_t)s * R + row;
                    w = l_parts[i] > 0.f ? l_parts[i] * ex(m_parts[i] - mx) : 0.f;
                }
                if (w != 0.f) acc = __builtin_fmaf(w, o_parts[((size_t)s * R + row) * d + c], acc);
            }
        }
        const float out = acc * inv;
        if (out_bf16) {
            const uint32_t packed = pack_bf16x2(out, 0.f);
            static_cast<uint16_t*>(o)[(size_t)row * d + c] = (uint16_t)(packed & 0xffffu);
        } else {
            static_cast<float*>(o)[(size_t)row * d + c] = out;
        }
    }
    if (lane == 0) {
        const float m_nat = lt > 0.f ? (log2_units ? mx * kLn2 : mx) : -INFINITY;
        if (m_out) m_out[row] = m_nat;
        if (l_out) l_out[row] = lt;
    }
}

}  // namespace

hipError_t launch_merge(const float* o_parts, const float* m_parts, const float* l_parts, void* o,
                        int out_bf16, float* m_out, float* l_out, int S, int R, int d,
                        int log2_units, hipStream_t stream) {
    if (R == 0) return hipSuccess;
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)R), dim3(kLanes), 0, stream, o_parts, m_parts,
                       l_parts, o, out_bf16, m_out, l_out, S, R, d, log2_units);
    return hipGetLastError();
}

}  // namespace fa
