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

// Saturating E4M3 ("e4m3fn") encode of four floats, round to nearest even:
// clamp to [-448, 448] (448 is the format's largest finite value), then the
// gfx950 packed fp32 -> fp8 convert, whose rounding is RNE with the format's
// subnormals (m * 2^-9) and which keeps the sign of zero.  Clamped, it agrees
// bit for bit with the encode written out from the format definition (4
// exponent bits of bias 7, 3 mantissa bits) on every non-NaN fp32 input.
// Bytes of the result: y0, y1, y2, y3 from low to high.  Finite inputs.
__device__ __forceinline__ uint32_t e4m3x4_encode_sat(float y0, float y1, float y2, float y3) {
  const float a0 = __builtin_amdgcn_fmed3f(y0, -448.0f, 448.0f);
  const float a1 = __builtin_amdgcn_fmed3f(y1, -448.0f, 448.0f);
  const float a2 = __builtin_amdgcn_fmed3f(y2, -448.0f, 448.0f);
  const float a3 = __builtin_amdgcn_fmed3f(y3, -448.0f, 448.0f);
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, lo, true);
}

// x / s for the encoder, given r = 1 / s rounded to nearest even and
// s >= 2^-92.  The product |x| r is within about an ulp of |x| / s; one fused
// multiply-add gives the residual |x| - q s, exact while |x| >= 2^-103 (it
// then stays clear of float32's subnormal range), and a second adds the
// residual times r back (Markstein's correction step), which rounds the
// quotient correctly.  Below that |x|, |x| / s < 2^-11 and every candidate
// rounds to a zero code.  The sign of x goes back on last, so -0 gives -0.
// Exhaustively, over every bf16 tile maximum and every bf16 x of magnitude
// at most it, the codes equal those of the IEEE division.
__device__ __forceinline__ float quotient_by_reciprocal(float x, float s, float r) {
  const float ax = fabsf(x);
  const float q = ax * r;
  const float corrected = __builtin_fmaf(__builtin_fmaf(-q, s, ax), r, q);
  return as_float((as_u32(corrected) & 0x7FFFFFFFu) | (as_u32(x) & 0x80000000u));
}

// One record is written by the 64 lanes of a wave.  Lane l owns latent
// columns 8l .. 8l+7 (bf16, 4-byte aligned), so the 16 lanes of a k-group own
// exactly one 128-wide tile and the tile maximum is a 4-step butterfly; codes
// leave as one 8-byte store per lane.  Lanes 0..31 pass rope word l (bf16
// values 2l and 2l+1, low half first), stored as is.  The scale is
// amax / 448 with IEEE division (HIP's default: correctly rounded), and x /
// scale is the correctly rounded quotient (quotient_by_reciprocal).
//
// The load and the encode are separate so that a caller can keep several
// tokens' loads in flight before the first encode waits for them.
__device__ __forceinline__ u32x4_t load_latent_lane(int lane, const uint16_t *latent) {
  const uint32_t *src = reinterpret_cast<const uint32_t *>(latent + 8 * lane);
  return u32x4_t{src[0], src[1], src[2], src[3]};
}

__device__ __forceinline__ void encode_store_record(int lane, u32x4_t w, uint32_t rope_word, uint8_t *rec) {
  float x[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = as_float(w[j] << 16);
    x[2 * j + 1] = as_float(w[j] & 0xFFFF0000u);
  }
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[j]));
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, xor_shuffle(amax, m));

  const float scale = amax / 448.0f;
  uint32_t lo = 0u, hi = 0u;
  if (scale > 0.f) {
    float q[8];
    if (scale < 0x1p-92f) {  // residuals that matter could underflow: divide
#pragma unroll
      for (int j = 0; j < 8; ++j) q[j] = x[j] / scale;
    } else {
      const float r = 1.0f / scale;
#pragma unroll
      for (int j = 0; j < 8; ++j) q[j] = quotient_by_reciprocal(x[j], scale, r);
    }
    lo = e4m3x4_encode_sat(q[0], q[1], q[2], q[3]);
    hi = e4m3x4_encode_sat(q[4], q[5], q[6], q[7]);
  }
  u32x2_t codes;
  codes.x = lo;
  codes.y = hi;
  *reinterpret_cast<u32x2_t *>(rec + 8 * lane) = codes;
  if ((lane & 15) == 0) *reinterpret_cast<float *>(rec + kScaleOffset + 4 * (lane >> 4)) = scale;
  if (lane < 32) *reinterpret_cast<uint32_t *>(rec + kRopeOffset + 4 * lane) = rope_word;
}

__device__ __forceinline__ void write_record_wave(int lane, const uint16_t *latent, uint32_t rope_word, uint8_t *rec) {
  encode_store_record(lane, load_latent_lane(lane, latent), rope_word, rec);
}

}  // namespace mla
