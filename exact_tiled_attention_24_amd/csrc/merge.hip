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


// Vectorised form for d % 4 == 0: TPR = d / 4 threads per row, each owning four columns;
// several rows per workgroup. The loop over partials is unrolled so that several partial
// loads are in flight at once (the scalar form above waits for one load per partial).
__global__ __launch_bounds__(256) void merge_vec4_kernel(
    const float* __restrict__ o_parts, const float* __restrict__ m_parts,
    const float* __restrict__ l_parts, void* __restrict__ o, int out_bf16,
    float* __restrict__ m_out, float* __restrict__ l_out, int S, int R, int d, int log2_units,
    int tpr) {
    const int rows_per_block = blockDim.x / tpr;
    const int row = blockIdx.x * rows_per_block + threadIdx.x / tpr;
    const int c4 = threadIdx.x % tpr;
    if (row >= R || threadIdx.x >= rows_per_block * tpr) return;
    auto ex = [&](float x) { return log2_units ? exp2_hw(x) : expf(x); };

    float mx = -INFINITY;
#pragma unroll 8
    for (int s = 0; s < S; ++s) {
        const size_t i = (size_t)s * R + row;
        const float l = l_parts[i], m = m_parts[i];
        mx = l > 0.f ? fmaxf(mx, m) : mx;
    }
    float lt = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (mx != -INFINITY) {
        const f32x4* o4 = reinterpret_cast<const f32x4*>(o_parts);
#pragma unroll 8
        for (int s = 0; s < S; ++s) {
            const size_t i = (size_t)s * R + row;
            const float l = l_parts[i], m = m_parts[i];
            const f32x4 ov = o4[i * (size_t)tpr + c4];
            const bool live = l > 0.f;
            const float w = live ? l * ex(m - mx) : 0.f;
            lt += w;
            // an empty partial's O is never used, whatever it holds
            acc[0] = live ? __builtin_fmaf(w, ov[0], acc[0]) : acc[0];
            acc[1] = live ? __builtin_fmaf(w, ov[1], acc[1]) : acc[1];
            acc[2] = live ? __builtin_fmaf(w, ov[2], acc[2]) : acc[2];
            acc[3] = live ? __builtin_fmaf(w, ov[3], acc[3]) : acc[3];
        }
    }
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const size_t oi = (size_t)row * d + 4 * c4;
    if (out_bf16) {
        u32x2 w = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(o) + oi) = w;
    } else {
        f32x4 w = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
        *reinterpret_cast<f32x4*>(static_cast<float*>(o) + oi) = w;
    }
    if (c4 == 0) {
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
    const bool aligned = ((reinterpret_cast<uintptr_t>(o_parts) | reinterpret_cast<uintptr_t>(o)) &
                          (out_bf16 ? 7u : 15u)) == 0 && (reinterpret_cast<uintptr_t>(o_parts) & 15u) == 0;
    if (d % 4 == 0 && aligned) {
        const int tpr = d / 4;
        const int rows_per_block = tpr >= 256 ? 1 : 256 / tpr;
        const int threads = rows_per_block * tpr;
        const unsigned blocks = (unsigned)((R + rows_per_block - 1) / rows_per_block);
        hipLaunchKernelGGL(merge_vec4_kernel, dim3(blocks), dim3(threads), 0, stream, o_parts,
                           m_parts, l_parts, o, out_bf16, m_out, l_out, S, R, d, log2_units, tpr);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)R), dim3(kLanes), 0, stream, o_parts, m_parts,
                       l_parts, o, out_bf16, m_out, l_out, S, R, d, log2_units);
    return hipGetLastError();
}

}  // namespace fa
