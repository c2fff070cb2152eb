// Internal launch interface between the C ABI (mla_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

struct FwdArgs {
  const uint16_t *q;
  int64_t q_stride_token, q_stride_head;  // elements
  const uint8_t *records;
  int64_t num_records;
  const void *indptr;
  const void *indices;
  int64_t num_indices;
  bool index_i64;
  float scale_log2;  // softmax_scale * log2(e)
  int32_t num_tokens;
  int32_t num_heads;
  uint16_t *out;
  int64_t out_stride_token, out_stride_head;  // elements
  float *lse;                                 // [T, H] or nullptr
  int32_t splits;
  float *ws_out;  // [T, splits, H, 512] float32 when splits > 1
  float *ws_lse;  // [T, splits, H] float32 (base-2 log-sum-exp) when splits > 1
};

hipError_t launch_sparse_fwd(const FwdArgs &a, hipStream_t stream);

struct InsertArgs {
  const uint16_t *kv_c;
  int64_t kv_c_stride;
  const uint16_t *k_pe;
  int64_t k_pe_stride;
  const int64_t *slots;
  int64_t num_tokens;
  uint8_t *records;
  int64_t num_records;
};

hipError_t launch_cache_insert(const InsertArgs &a, hipStream_t stream);

// Bytes of split partials for a call (0 when splits <= 1), 256-byte aligned parts.
inline size_t split_workspace_bytes(int64_t tokens, int32_t heads, int32_t splits) {
  if (splits <= 1 || tokens <= 0) return 0;
  const size_t rows = (size_t)tokens * (size_t)splits * (size_t)heads;
  const size_t out_bytes = (rows * 512 * sizeof(float) + 255) & ~(size_t)255;
  const size_t lse_bytes = (rows * sizeof(float) + 255) & ~(size_t)255;
  return out_bytes + lse_bytes;
}
inline size_t split_workspace_lse_offset(int64_t tokens, int32_t heads, int32_t splits) {
  const size_t rows = (size_t)tokens * (size_t)splits * (size_t)heads;
  return (rows * 512 * sizeof(float) + 255) & ~(size_t)255;
}

}  // namespace mla
