// The fp8_ds_mla record writer shared by the insert kernels: one wave writes
// one token's 656-byte record.
//
// The record is the one written by fused_mla_key_concat_ds_mla_insert and by
// fused_mla_decode_q_concat_kv_cache_insert(ds_mla=True) (vLLM API page
// vllm.models.kimi_k3.nvidia.ops.fused_mla_key_concat_kv_cache): the latent
// in 4 tiles of 128 with a per-tile dynamic scale (amax / 448), stored as
// E4M3 with the writer's saturating quant, then the rope as bf16.
#pragma once

#include "device_utils.h"

namespace mla {

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

// Write one record with the 64 lanes of a wave.  Lane l owns latent columns
// 8l .. 8l+7 of `latent` (bf16, 4-byte aligned), so the 16 lanes of a k-group
// own exactly one 128-wide tile and the tile maximum is a 4-step butterfly;
// codes leave as one 8-byte store per lane.  Lanes 0..31 pass rope word l
// (bf16 values 2l and 2l+1, low half first) in `rope_word`; it is stored as
// is.  The scale is amax / 448 with IEEE division (HIP's default: correctly
// rounded), and so is x / scale.
__device__ __forceinline__ void write_record_wave(int lane, const uint16_t *latent, uint32_t rope_word, uint8_t *rec) {
  const uint32_t *src = reinterpret_cast<const uint32_t *>(latent + 8 * lane);
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

  const float scale = amax / 448.0f;
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
  if (lane < 32) *reinterpret_cast<uint32_t *>(rec + kRopeOffset + 4 * lane) = rope_word;
}

}  // namespace mla
