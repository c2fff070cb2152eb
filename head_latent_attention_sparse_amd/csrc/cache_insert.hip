// fp8_ds_mla cache insert for gfx950: quantize [kv_c_normed | k_pe] into
// 656-byte records.
//
// The record is the one written by fused_mla_key_concat_ds_mla_insert and by
// fused_mla_decode_q_concat_kv_cache_insert(ds_mla=True) (vLLM API page
// vllm.models.kimi_k3.nvidia.ops.fused_mla_key_concat_kv_cache): the latent
// in 4 tiles of 128 with a per-tile dynamic scale (amax / 448), stored as
// E4M3 with the writer's saturating quant, then the rope as bf16.
//
// One wave per token; lane l owns latent columns 8l .. 8l+7, so the 16 lanes
// of a k-group own exactly one 128-wide tile and the tile maximum is a
// 4-step butterfly.  Codes leave as one 8-byte store per lane (512
// contiguous bytes per wave).
#include "device_utils.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kTokensPerBlock = 4;

// Saturating E4M3 ("e4m3fn") encode, round to nearest even, from the format
// definition: 4 exponent bits (bias 7), 3 mantissa bits, subnormals m*2^-9,
// largest finite 448.  Finite inputs.
__device__ __forceinline__ uint32_t e4m3_encode_sat(float y) {
  const uint32_t sign = (as_u32(y) >> 24) & 0x80u;
  const float a = fminf(fabsf(y), 448.0f);
  if (a < 0x1p-6f) {
    // m * 2^-9 with m = rne(a * 2^9); the scaling is exact and m = 8 is the
    // smallest normal (code 0x08), so both ranges meet without a seam.
    return sign | (uint32_t)__builtin_rintf(a * 512.0f);
  }
  const uint32_t bits = as_u32(a);
  const uint32_t mant = bits & 0x7FFFFFu;
  // exponent field of E4M3 = (float exponent - 127) + 7 = biased - 120
  uint32_t code = (((bits >> 23) - 120u) << 3) | (mant >> 20);
  const uint32_t rem = mant & 0xFFFFFu;  // the 20 dropped mantissa bits
  code += (rem > 0x80000u || (rem == 0x80000u && (code & 1u))) ? 1u : 0u;
  return sign | code;
}

__global__ __launch_bounds__(256) void cache_insert_kernel(InsertArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * kTokensPerBlock + (threadIdx.x >> 6);
  if (i >= a.num_tokens) return;
  const int64_t slot = a.slots[i];
  if (slot < 0 || slot >= a.num_records) return;  // skipped token (whole wave)
  uint8_t *rec = a.records + slot * kRecordBytes;

  // 8 latent values of this lane (bf16 -> f32 is exact)
  const uint32_t *src = reinterpret_cast<const uint32_t *>(a.kv_c + i * a.kv_c_stride + 8 * lane);
  float x[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w = src[j];
    x[2 * j] = as_float(w << 16);
    x[2 * j + 1] = as_float(w & 0xFFFF0000u);
  }
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[j]));
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, xor_shuffle(amax, m));

  const float scale = amax / 448.0f;  // IEEE division (HIP default: correctly rounded)
  uint32_t lo = 0u, hi = 0u;
  if (scale > 0.f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) lo |= e4m3_encode_sat(x[j] / scale) << (8 * j);
#pragma unroll
    for (int j = 0; j < 4; ++j) hi |= e4m3_encode_sat(x[4 + j] / scale) << (8 * j);
  }
  u32x2_t codes;
  codes.x = lo;
  codes.y = hi;
  *reinterpret_cast<u32x2_t *>(rec + 8 * lane) = codes;
  if ((lane & 15) == 0) *reinterpret_cast<float *>(rec + kScaleOffset + 4 * (lane >> 4)) = scale;
  if (lane < 32) {
    const uint32_t *pe = reinterpret_cast<const uint32_t *>(a.k_pe + i * a.k_pe_stride);
    *reinterpret_cast<uint32_t *>(rec + kRopeOffset + 4 * lane) = pe[lane];
  }
}

}  // namespace

hipError_t launch_cache_insert(const InsertArgs &a, hipStream_t stream) {
  const int64_t blocks = (a.num_tokens + kTokensPerBlock - 1) / kTokensPerBlock;
  cache_insert_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace mla
