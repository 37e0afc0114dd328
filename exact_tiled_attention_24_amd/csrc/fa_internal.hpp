// fa_internal.hpp - launchers shared between the C ABI layer and the kernel files.
// Every launcher assumes arguments were validated by the caller (fa_api.hip) and only
// enqueues kernels on `stream`; it returns hipGetLastError() after the launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Compute units assumed when the device cannot be queried (MI355X: 256 CUs in 8 XCDs).
constexpr int kDefaultCUs = 256;

// Compute units of the current device, queried once per device and cached.
int device_cus();

// Software-pipelined: 8 waves, 256 query rows; MFMAs of neighbouring half tiles overlap
// each half tile's softmax within every wave.
hipError_t launch_fwd_bf16_sp(const void* q, const void* k, const void* v, void* o, float* m_out,
                              float* l_out, int B, int Hq, int Hkv, int N, int d, float scale,
                              int causal, hipStream_t stream);

// Chunked prefill over a paged KV cache with the same kernel: the Nq (or q_lens[b]) queries of
// sequence b are its newest tokens (bottom-right causal alignment); K/V through the table.
hipError_t launch_fwd_bf16_sp_paged(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    const int32_t* q_lens, void* o,
                                    float* m_out, float* l_out, int B, int Hq, int Hkv, int Nq,
                                    int d, int num_pages, int max_pages_per_seq, float scale,
                                    int causal, hipStream_t stream);

// Block-sparse forward with the same kernel: query block qb (256 rows) of head (b, h) visits
// only the 64-key tiles blk_idx[blk_off[r] .. blk_off[r + 1]), r = (b * Hq + h) * nqb + qb.
hipError_t launch_fwd_bf16_sp_block_sparse(const void* q, const void* k, const void* v, void* o,
                                           float* m_out, float* l_out, const int32_t* block_offsets,
                                           const int32_t* block_indices, int nnz, int B, int Hq,
                                           int Hkv, int N, int d, float scale, int causal,
                                           hipStream_t stream);

// Backward by recomputation: D and the log2 normaliser of every query row into `ld` (caller
// workspace of bwd_ld_bytes(B, Hq, N) bytes), then dK/dV and dQ (bf16 outputs, float32
// accumulation).
hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* m, const float* l, void* dq, void* dk,
                           void* dv, int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                           float* ld, hipStream_t stream);
// Bytes of that workspace: two float32 values per query row, a head's rows padded to 32.
inline size_t bwd_ld_bytes(int B, int Hq, int N) {
    return (size_t)B * (size_t)Hq * (((size_t)N + 31) / 32 * 32) * 2 * sizeof(float);
}

// Forward with fp8 (OCP e4m3) Q and K: S^T on the fp8 matrix cores. v_fp8 == 0: V bf16, P
// rounded to bf16, P V as in the bf16 kernel; v_fp8 != 0: V e4m3, P rounded to e4m3, P V on the
// fp8 matrix cores too. O bf16; d = 128.
hipError_t launch_fwd_fp8qk_sp(const void* q, const void* k, const void* v, int v_fp8, void* o,
                               float* m_out, float* l_out, int B, int Hq, int Hkv, int N, int d,
                               float scale, int causal, hipStream_t stream);

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* m_out,
                          float* l_out, int B, int Hq, int Hkv, int N, int d, float scale,
                          int causal, hipStream_t stream);

// Caller workspace of the split-K decode: completion words [B * Hkv] (any contents), then
// float32 partials O [S][B * Hq][d], m [S][B * Hq] (log2 units), l [S][B * Hq].
struct DecodeWorkspace {
    unsigned long long* done;
    float* o;
    float* m;
    float* l;
};

// Split-K paged decode with both products on the matrix cores (query heads per KV head
// <= 16): each chunk of `chunk_pages` pages of a (sequence, KV head) yields a partial, and
// the last chunk to finish merges them into o, in the same launch.
hipError_t launch_decode_bf16_mx(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_table, const int32_t* seq_lens, void* o,
                                 int B, int Hq, int Hkv, int d, int num_pages,
                                 int max_pages_per_seq, int len_cap, float scale, int splits,
                                 int chunk_pages, const DecodeWorkspace& ws, hipStream_t stream);

// The decode scratch of the allocation-free entry point: its size, and its device address on
// the current device (looked up once per device; no allocation).
size_t decode_scratch_bytes();
hipError_t decode_scratch(void** ptr);

// Row-wise merge of S partials. log2_units != 0: m is in log2 units (internal workspace);
// otherwise natural-log units (public fa_merge). out_bf16 selects the output type.
hipError_t launch_merge(const float* o_parts, const float* m_parts, const float* l_parts, void* o,
                        int out_bf16, float* m_out, float* l_out, int S, int R, int d,
                        int log2_units, hipStream_t stream);

}  // namespace fa
