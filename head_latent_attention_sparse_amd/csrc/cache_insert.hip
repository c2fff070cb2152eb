// fp8_ds_mla cache insert for gfx950: quantize [kv_c_normed | k_pe] into
// 656-byte records.
//
// The record is the one written by fused_mla_key_concat_ds_mla_insert and by
// fused_mla_decode_q_concat_kv_cache_insert(ds_mla=True) (vLLM API page
// vllm.models.kimi_k3.nvidia.ops.fused_mla_key_concat_kv_cache): the latent
// in 4 tiles of 128 with a per-tile dynamic scale (amax / 448), stored as
// E4M3 with the writer's saturating quant, then the rope as bf16.
//
// Each wave takes kTokensPerWave consecutive tokens and issues every load
// (slots, latent, rope) before the first encode: the slot gates only the
// store, so no load waits on another and a wave keeps several tokens of
// reads in flight.
#include "mla_internal.h"
#include "record_writer.h"

namespace mla {
namespace {

constexpr int kWaves = 4;
constexpr int kTokensPerWave = 2;

__global__ __launch_bounds__(64 * kWaves) void cache_insert_kernel(InsertArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t first = ((int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6)) * kTokensPerWave;
  if (first >= a.num_tokens) return;
  int64_t slot[kTokensPerWave];
  u32x4_t lat[kTokensPerWave];
  uint32_t rope[kTokensPerWave];
#pragma unroll
  for (int k = 0; k < kTokensPerWave; ++k) {
    const bool live = first + k < a.num_tokens;
    const int64_t i = live ? first + k : first;  // past the end: reload token `first`, store nothing
    slot[k] = live ? a.slots[i] : -1;
    lat[k] = load_latent_lane(lane, a.kv_c + i * a.kv_c_stride);
    rope[k] = lane < 32 ? reinterpret_cast<const uint32_t *>(a.k_pe + i * a.k_pe_stride)[lane] : 0u;
  }
#pragma unroll
  for (int k = 0; k < kTokensPerWave; ++k) {
    if (slot[k] < 0 || slot[k] >= a.num_records) continue;  // skipped token (whole wave)
    encode_store_record(lane, lat[k], rope[k], a.records + slot[k] * kRecordBytes);
  }
}

}  // namespace

hipError_t launch_cache_insert(const InsertArgs &a, hipStream_t stream) {
  constexpr int64_t per_block = kWaves * kTokensPerWave;
  const int64_t blocks = (a.num_tokens + per_block - 1) / per_block;
  cache_insert_kernel<<<dim3((unsigned)blocks), dim3(64 * kWaves), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace mla
