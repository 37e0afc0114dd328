// fwd_f32.hip - tiled attention forward in float32 throughout.
//
// The same tiled online softmax as the bf16 kernel ("FlashAttention", "The trick: tiles and
// an online softmax"), kept in float32 with natural-base exponentials for inputs whose
// accuracy target is float32 rounding. This path is for small problems (a single-head
// N = 256 case); it uses plain FMAs, not the matrix cores.
//
// Workgroup: 64 query rows x 4 lanes per row (each lane owns d/4 columns of q and of the
// accumulator); K/V tiles of 64 keys are staged in LDS and broadcast to all rows.
#include "fa_internal.hpp"
#include "gfx950.hpp"

namespace fa {
namespace {

constexpr int kRows = 64;
constexpr int kKeys = 64;
constexpr int kParts = 4;
constexpr int kThreads = kRows * kParts;

template <int D>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ m_out, float* __restrict__ l_out, int B, int Hq,
    int Hkv, int N, float scale, int causal) {
    constexpr int DP = D / kParts;
    __shared__ float ks[kKeys][D];
    __shared__ float vs[kKeys][D];

    const int BH = B * Hq;
    const int bh = blockIdx.x % BH;
    const int qb = blockIdx.x / BH;
    const int b = bh / Hq;
    const int h = bh - b * Hq;
    const int kvh = h / (Hq / Hkv);
    const float* qh = q + (size_t)bh * N * D;
    const float* kh = k + (size_t)(b * Hkv + kvh) * N * D;
    const float* vh = v + (size_t)(b * Hkv + kvh) * N * D;

    const int tid = threadIdx.x;
    const int row = qb * kRows + tid / kParts;
    const int part = tid % kParts;
    const int col0 = part * DP;

    float qr[DP], acc[DP];
    {
        const float* src = qh + (size_t)min_(row, N - 1) * D + col0;
#pragma unroll
        for (int i = 0; i < DP; ++i) {
            qr[i] = src[i];
            acc[i] = 0.f;
        }
    }
    float m = -INFINITY, l = 0.f;

    const int kv_end = causal ? min_(N, qb * kRows + kRows) : N;
    for (int kv0 = 0; kv0 < kv_end; kv0 += kKeys) {
        __syncthreads();
        for (int idx = tid; idx < kKeys * D; idx += kThreads) {
            const int r = idx / D;
            const int c = idx - r * D;
            const size_t g = (size_t)min_(kv0 + r, N - 1) * D + c;
            ks[r][c] = kh[g];
            vs[r][c] = vh[g];
        }
        __syncthreads();

        float s[kKeys];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < kKeys; ++j) {
            float dot = 0.f;
#pragma unroll
            for (int i = 0; i < DP; ++i) dot = __builtin_fmaf(qr[i], ks[j][col0 + i], dot);
            dot += __shfl_xor(dot, 1);
            dot += __shfl_xor(dot, 2);
            const int key = kv0 + j;
            const bool bad = key >= N || (causal && key > row);
            s[j] = bad ? -INFINITY : dot * scale;
            mx = fmaxf(mx, s[j]);
        }
        const float m_new = fmaxf(m, mx);
        if (m_new == -INFINITY) continue;
        const float alpha = (m == -INFINITY) ? 0.f : expf(m - m_new);
        l *= alpha;
#pragma unroll
        for (int i = 0; i < DP; ++i) acc[i] *= alpha;
#pragma unroll
        for (int j = 0; j < kKeys; ++j) {
            const float pj = (s[j] == -INFINITY) ? 0.f : expf(s[j] - m_new);
            l += pj;
#pragma unroll
            for (int i = 0; i < DP; ++i) acc[i] = __builtin_fmaf(pj, vs[j][col0 + i], acc[i]);
        }
        m = m_new;
    }

    if (row < N) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        float* dst = o + (size_t)bh * N * D + (size_t)row * D + col0;
#pragma unroll
        for (int i = 0; i < DP; ++i) dst[i] = acc[i] * inv;
        if (part == 0) {
            const size_t ridx = (size_t)bh * N + row;
            if (m_out) m_out[ridx] = m;
            if (l_out) l_out[ridx] = l;
        }
    }
}

}  // namespace

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* m_out,
                          float* l_out, int B, int Hq, int Hkv, int N, int d, float scale,
                          int causal, hipStream_t stream) {
    const int nqb = (N + kRows - 1) / kRows;
    const dim3 grid((unsigned)((long long)nqb * B * Hq));
    if (d == 128)
        hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, dim3(kThreads), 0, stream, q, k, v, o, m_out,
                           l_out, B, Hq, Hkv, N, scale, causal);
    else
        hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, dim3(kThreads), 0, stream, q, k, v, o, m_out,
                           l_out, B, Hq, Hkv, N, scale, causal);
    return hipGetLastError();
}

}  // namespace fa
