// Device helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef int intx2_t __attribute__((ext_vector_type(2)));
typedef int intx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef int intx8_t __attribute__((ext_vector_type(8)));

constexpr int kRecordBytes = 656;
constexpr int kLatent = 512;
constexpr int kRope = 64;
constexpr int kQkDim = 576;
constexpr int kScaleOffset = 512;
constexpr int kRopeOffset = 528;
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.44269504088896341f;

__device__ __forceinline__ float as_float(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u32(float f) { return __builtin_bit_cast(uint32_t, f); }

// Two E4M3 codes (the low or the high 16 bits of w) -> two bf16 packed in a
// u32, low code in the low half.  The gfx950 scaled convert with scale 1.0
// is exact here: every E4M3 value (subnormals included) is a bf16 value.
__device__ __forceinline__ uint32_t e4m3x2_lo_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
}
__device__ __forceinline__ uint32_t e4m3x2_hi_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}

// Eight E4M3 codes (bytes of w0 then w1) -> an MFMA bf16x8 operand.
__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  u32x4_t r;
  r.x = e4m3x2_lo_to_bf16x2(w0);
  r.y = e4m3x2_hi_to_bf16x2(w0);
  r.z = e4m3x2_lo_to_bf16x2(w1);
  r.w = e4m3x2_hi_to_bf16x2(w1);
  return __builtin_bit_cast(bf16x8_t, r);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

typedef float floatx2_t __attribute__((ext_vector_type(2)));

// Two floats -> two bf16 (low half = lo), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const floatx2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ floatx4_t mfma_16x16x32_bf16(bf16x8_t a, bf16x8_t b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Butterfly over lanes that differ in bit `mask` of the lane id (wave64).
__device__ __forceinline__ float xor_shuffle(float v, int mask) {
  const int lane = __lane_id();
  const int src = (lane ^ mask) << 2;
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, v)));
}

// Job of workgroup `id` in a grid of 8 * ceil(jobs / 8) workgroups: the
// dispatcher hands workgroups to the 8 XCDs round-robin (XCD id % 8), so
// this gives each XCD a contiguous run of jobs; neighbouring jobs (the same
// head's rows, say) then share that XCD's L2.  A result >= jobs means no job.
__device__ __forceinline__ int64_t xcd_job(int64_t id, int64_t jobs) {
  return (id % 8) * ((jobs + 7) / 8) + id / 8;
}
inline int64_t xcd_grid(int64_t jobs) { return 8 * ((jobs + 7) / 8); }

}  // namespace mla
