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
  // Split-KV: chunk_bound == 0 = one workgroup per row.  Otherwise rows are
  // cut into chunks of chunk_forced entries if > 0, else of a size the
  // partial pass picks on the device so the chunks fit chunk_bound, its grid
  // (an upper bound on the number of chunks).  At most 512 rows.
  int32_t chunk_forced;
  int64_t chunk_bound;
  // one workgroup per row: rows most likely start at t * row_len_guess
  // (checked against indptr by each workgroup; 0 = no guess)
  int64_t row_len_guess = 0;
  float *ws_out;       // [chunk_bound, H, 512] float32 partials
  float *ws_lse;       // [chunk_bound, H] float32 base-2 log-sum-exp
  int32_t *ws_prefix;  // [T + 1] first chunk of each row
  // Optional second segment (extra_indptr != nullptr): a second pool whose
  // CSR list joins each row's softmax.  Optional per-head sink logits.
  const uint8_t *extra_records = nullptr;
  int64_t extra_num_records = 0;
  const void *extra_indptr = nullptr;
  const void *extra_indices = nullptr;
  int64_t extra_num_indices = 0;
  const float *sink = nullptr;
  // Optional up-projection fused into the merge of a split call (prepared
  // W_UV, no sink, no second segment); a call that does not split leaves
  // the projection to the caller.
  const uint16_t *vp_w = nullptr;
  const uint16_t *vp_gate = nullptr;
  int64_t vp_gate_st = 0;
  uint16_t *vp_out = nullptr;
  int64_t vp_st = 0, vp_sh = 0;
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

struct DecodeEpilogueArgs {
  const uint16_t *ql_nope;
  int64_t ql_stride_token, ql_stride_head;  // elements
  const uint16_t *q_pe;
  int64_t qpe_stride_token, qpe_stride_head;
  const uint16_t *kv_c;
  int64_t kv_c_stride;
  const uint16_t *k_pe;
  int64_t k_pe_stride;
  const int64_t *slots;
  int64_t num_tokens;
  int32_t num_heads;
  const int64_t *positions;  // nullptr: no RoPE
  const float *cos_sin;      // [max_position, 64]: cos of pair i at i, sin at 32 + i
  int64_t max_position;
  uint16_t *mqa_q;
  int64_t mq_stride_token, mq_stride_head;
  uint8_t *records;
  int64_t num_records;
};

hipError_t launch_decode_epilogue(const DecodeEpilogueArgs &a, hipStream_t stream);

struct PrefillEpilogueArgs {
  uint16_t *q;  // [Tp, H, nope + 64]: RoPE in place on columns nope .. nope+63
  int64_t q_stride_token, q_stride_head;
  int32_t nope;  // qk_nope_head_dim, a multiple of 8
  const uint16_t *k_nope;  // [Tp, H, nope]
  int64_t kn_stride_token, kn_stride_head;
  const uint16_t *kv_c;
  int64_t kv_c_stride;
  const uint16_t *k_pe;
  int64_t k_pe_stride;
  const int64_t *slots;
  int64_t num_tokens;
  int32_t num_heads;
  const int64_t *positions;  // nullptr: no RoPE
  const float *cos_sin;
  int64_t max_position;
  uint16_t *k_out;  // [Tp, H, nope + 64]
  int64_t ko_stride_token, ko_stride_head;
  uint8_t *records;
  int64_t num_records;
};

hipError_t launch_prefill_epilogue(const PrefillEpilogueArgs &a, hipStream_t stream);

struct GatherArgs {
  const uint8_t *records;
  int64_t num_records;
  int64_t block_size;
  const int32_t *block_table;
  int64_t bt_stride;  // elements between requests' rows
  int64_t bt_width;   // blocks per row
  const int32_t *cu;  // [batch + 1] workspace row of each request's first token
  const int32_t *starts;  // [batch] first context position of each request, or nullptr (0)
  int32_t batch;
  int64_t num_tokens;
  uint16_t *dst;
  int64_t dst_stride;  // elements
};

hipError_t launch_gather_upconvert(const GatherArgs &a, hipStream_t stream);

struct VUpProjArgs {
  const uint16_t *latent;  // bf16, element (t, h, l) at t*lat_st + h*lat_sh + l
  int64_t lat_st, lat_sh;
  const uint16_t *w;       // bf16 [H, 512, 128] contiguous
  const uint16_t *gate;    // bf16, element (t, h*128 + v) at t*gate_st + h*128 + v, or nullptr
  int64_t gate_st;
  int64_t num_tokens;
  int32_t num_heads;
  uint16_t *out;           // bf16, element (t, h, v) at t*out_st + h*out_sh + v
  int64_t out_st, out_sh;
  bool w_prepared = false;  // w holds launch_prepare_w_uv's fragment order
  int32_t parts = 0;        // row-tile workgroups per head (set by launch_v_up_proj)
};

hipError_t launch_v_up_proj(const VUpProjArgs &a, int num_cus, hipStream_t stream);

// The split-KV merge fused with the up-projection on prepared weights: each
// row's chunk partials are merged exactly as merge_kernel merges them with
// `lanes` chunk lanes (bit for bit), the merged latent row is written to
// `out` as bf16 (and the LSE), and the same bf16 row goes straight into the
// projection, which computes what v_up_proj_kernel<gate, prepared> computes
// (bit for bit).
struct MergeVUpProjArgs {
  const float *ws_out;       // [chunks, H, 512] float32 partials
  const float *ws_lse;       // [chunks, H] base-2 LSEs
  const int32_t *ws_prefix;  // [T + 1] first chunk of each row
  int32_t num_tokens;
  int32_t num_heads;
  uint16_t *out;  // merged latent, element (t, h, l) at t*out_st + h*out_sh + l
  int64_t out_st, out_sh;
  float *lse;                 // [T, H] natural log, or nullptr
  const uint16_t *w_prepared;  // W_UV in launch_prepare_w_uv's order
  const uint16_t *gate;        // element (t, 128h + v) at t*gate_st + 128h + v, or nullptr
  int64_t gate_st;
  uint16_t *v_out;  // element (t, h, v) at t*v_st + h*v_sh + v
  int64_t v_st, v_sh;
};
hipError_t launch_merge_v_up_proj(const MergeVUpProjArgs &a, int lanes, hipStream_t stream);
// W_UV [H, 512, 128] bf16 -> the same bytes in the up-projection's fragment order
hipError_t launch_prepare_w_uv(const uint16_t *w, uint16_t *w_prepared, int32_t num_heads, hipStream_t stream);

// Workspace of a chunked (split-KV) call, in 256-byte aligned parts:
// partials, partial LSEs, row prefix.
struct SplitLayout {
  size_t out_off, lse_off, prefix_off, bytes;
};
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline SplitLayout split_layout(int64_t tokens, int32_t heads, int64_t chunk_bound) {
  SplitLayout l;
  const size_t rows = (size_t)chunk_bound * (size_t)heads;
  l.out_off = 0;
  l.lse_off = align256(rows * 512 * sizeof(float));
  l.prefix_off = l.lse_off + align256(rows * sizeof(float));
  l.bytes = l.prefix_off + align256(((size_t)tokens + 1) * sizeof(int32_t));
  return l;
}
// Upper bound on the number of chunks of a forced chunk size: every row adds
// at most one partial chunk.
inline int64_t forced_chunk_bound(int64_t tokens, int64_t nnz, int32_t chunk_entries) {
  return (nnz + chunk_entries - 1) / chunk_entries + tokens;
}

constexpr int64_t kMaxSplitRows = 512;  // rows the split pass serves

}  // namespace mla
