// The split-KV merge accumulator shared by the merge kernels: one (row,
// head, column quad)'s running combination of chunk partials (o_s, lse_s)
// in the base-2 log domain, lse = log2 sum_s 2^lse_s and
// out = sum_s 2^(lse_s - lse) o_s (the merge named by merge_attn_states on
// the kimi_k3 nvidia mla page).
#pragma once

#include "device_utils.h"

namespace mla {

struct MergeAcc {
  float m, l;   // running max (log2 domain) and sum of 2^(lse - m)
  floatx4_t o;  // running sum of 2^(lse - m) o
};

__device__ __forceinline__ MergeAcc merge_acc_empty() { return MergeAcc{-INFINITY, 0.f, floatx4_t{0.f, 0.f, 0.f, 0.f}}; }

// The updates are written as explicit fused multiply-adds, so every kernel
// that merges computes the same roundings (left to the compiler, a*x + b*y
// may be fused either way).

// Add one partial; an empty partial (lse = -inf) weighs 0.
__device__ __forceinline__ void merge_add(MergeAcc &a, float lse, const floatx4_t &o) {
  if (lse == -INFINITY) return;
  const float m = fmaxf(a.m, lse);
  const float sa = a.m == -INFINITY ? 0.f : fast_exp2(a.m - m);
  const float w = fast_exp2(lse - m);
  a.l = __builtin_fmaf(a.l, sa, w);
#pragma unroll
  for (int i = 0; i < 4; ++i) a.o[i] = __builtin_fmaf(o[i], w, a.o[i] * sa);
  a.m = m;
}

// Fold accumulator b into a.
__device__ __forceinline__ void merge_combine(MergeAcc &a, const MergeAcc &b) {
  if (b.m == -INFINITY) return;
  const float m = fmaxf(a.m, b.m);
  const float sa = a.m == -INFINITY ? 0.f : fast_exp2(a.m - m);
  const float sb = fast_exp2(b.m - m);
  a.l = __builtin_fmaf(b.l, sb, a.l * sa);
#pragma unroll
  for (int i = 0; i < 4; ++i) a.o[i] = __builtin_fmaf(b.o[i], sb, a.o[i] * sa);
  a.m = m;
}

}  // namespace mla
