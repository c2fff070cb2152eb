// fp8_ds_mla cache insert for gfx950: quantize [kv_c_normed | k_pe] into
// 656-byte records.
//
// The record is the one written by fused_mla_key_concat_ds_mla_insert and by
// fused_mla_decode_q_concat_kv_cache_insert(ds_mla=True) (vLLM API page
// vllm.models.kimi_k3.nvidia.ops.fused_mla_key_concat_kv_cache): the latent
// in 4 tiles of 128 with a per-tile dynamic scale (amax / 448), stored as
// E4M3 with the writer's saturating quant, then the rope as bf16.
//
// One wave per token (write_record_wave).
#include "mla_internal.h"
#include "record_writer.h"

namespace mla {
namespace {

constexpr int kTokensPerBlock = 4;

__global__ __launch_bounds__(256) void cache_insert_kernel(InsertArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * kTokensPerBlock + (threadIdx.x >> 6);
  if (i >= a.num_tokens) return;
  const int64_t slot = a.slots[i];
  if (slot < 0 || slot >= a.num_records) return;  // skipped token (whole wave)
  const uint32_t *pe = reinterpret_cast<const uint32_t *>(a.k_pe + i * a.k_pe_stride);
  const uint32_t rope_word = lane < 32 ? pe[lane] : 0u;
  write_record_wave(lane, a.kv_c + i * a.kv_c_stride, rope_word, a.records + slot * kRecordBytes);
}

}  // namespace

hipError_t launch_cache_insert(const InsertArgs &a, hipStream_t stream) {
  const int64_t blocks = (a.num_tokens + kTokensPerBlock - 1) / kTokensPerBlock;
  cache_insert_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace mla
