// MLA decode and prefill epilogues for gfx950, each one launch.
//
// Decode: the latent decode query mqa_q = [ql_nope | RoPE(q_pe)] and the
// fp8_ds_mla insert of [kv_c_normed | RoPE(k_pe)].
//
// Prefill (fused_mla_key_concat_ds_mla_insert on the same page): RoPE on the
// rope part of q in place, the bf16 full key k_out = [k_nope | RoPE(k_pe)]
// for every head, and the same insert.
//
// What it computes is fused_mla_decode_q_concat_kv_cache_insert with
// ds_mla=True (vLLM API page
// vllm.models.kimi_k3.nvidia.ops.fused_mla_key_concat_kv_cache, function
// docstring and its dispatch by cache format: bf16 mqa_q, 656-byte
// block-scaled cache).  The optional positions / cos_sin_cache pair selects
// GPT-J-style RoPE (the module docstring), read from an fp32 table and
// computed in fp32 (vllm.models.kimi_k3.nvidia.mla page,
// MultiHeadLatentAttention: a float32 table, is_neox_style=False, passed
// straight to the fused epilogues): for pair i of the
// 64 rope values, (x0, x1) = (x[2i], x[2i+1]), c = cos_sin[pos][i],
// s = cos_sin[pos][32 + i],
//     y[2i]   = x0 * c - x1 * s,    y[2i+1] = x1 * c + x0 * s,
// each product and the sum rounded to float32 (no fused multiply-add), then
// to bf16 round-to-nearest-even.
//
// One workgroup per token: wave 0 loads the record's inputs, every thread
// loads its first batch of query (or key) chunks, then wave 0 writes the
// record and every thread its chunks, 16 bytes per thread per chunk.
#include "mla_internal.h"
#include "record_writer.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kChunksPerHead = kQkDim / 8;  // 72 x 8 bf16
// chunks whose loads a thread keeps in flight together
constexpr int kBatchDecode = 4;
constexpr int kBatchPrefill = 2;

#pragma clang fp contract(off)
// GPT-J rotation of one pair, float32 with a rounding after every operation.
__device__ __forceinline__ void rope_pair(float x0, float x1, float c, float s, float &y0, float &y1) {
  y0 = x0 * c - x1 * s;
  y1 = x1 * c + x0 * s;
}
#pragma clang fp contract(on)

__device__ __forceinline__ uint32_t rope_word(uint32_t w, float c, float s) {
  float y0, y1;
  rope_pair(as_float(w << 16), as_float(w & 0xFFFF0000u), c, s, y0, y1);
  return pack_bf16x2(y0, y1);
}

// The record's inputs, loaded by wave 0 (tid < 64) of the token's workgroup.
struct RecordLoads {
  int64_t slot;
  u32x4_t latent;
  uint32_t pe;  // rope word tid (tid < 32), before RoPE
};

__device__ __forceinline__ RecordLoads load_record_inputs(int tid, int64_t b, const int64_t *slots, const uint16_t *kv_c,
                                                          int64_t kv_c_stride, const uint16_t *k_pe, int64_t k_pe_stride) {
  RecordLoads r{-1, u32x4_t{0u, 0u, 0u, 0u}, 0u};
  if (tid < 64) {
    r.slot = slots[b];
    r.latent = load_latent_lane(tid, kv_c + b * kv_c_stride);
    if (tid < 32) r.pe = reinterpret_cast<const uint32_t *>(k_pe + b * k_pe_stride)[tid];
  }
  return r;
}

// Wave 0 rotates the rope words (when cs is set) and writes the record,
// unless the slot is -1 or out of range.
__device__ __forceinline__ void store_record(int tid, const RecordLoads &r, const float *cs, int64_t num_records,
                                             uint8_t *records) {
  if (tid >= 64 || r.slot < 0 || r.slot >= num_records) return;
  uint32_t w = r.pe;
  if (cs && tid < 32) w = rope_word(w, cs[tid], cs[32 + tid]);
  encode_store_record(tid, r.latent, w, records + r.slot * kRecordBytes);
}

__global__ __launch_bounds__(kThreads) void decode_epilogue_kernel(DecodeEpilogueArgs a) {
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.x;
  const float *cs = nullptr;  // this token's cos/sin row, or none
  if (a.positions) {
    int64_t pos = a.positions[b];
    pos = pos < 0 ? 0 : (pos >= a.max_position ? a.max_position - 1 : pos);
    cs = a.cos_sin + pos * kRope;
  }

  // ---- the record's loads (wave 0), issued before the query's so that no
  // load waits on a store; the record is encoded after the first batch.
  RecordLoads rl = load_record_inputs(tid, b, a.slots, a.kv_c, a.kv_c_stride, a.k_pe, a.k_pe_stride);
  bool record_pending = true;

  // ---- the query: chunk j of head h holds columns 8j .. 8j+7 of the 576.
  // Batches of kBatchDecode chunks per thread: all loads first, then the stores
  // (the output may alias the inputs as far as the compiler knows, so loads
  // after a store would wait for it).
  const int chunks = a.num_heads * kChunksPerHead;
  for (int base = 0; base < chunks; base += kThreads * kBatchDecode) {
    u32x4_t w[kBatchDecode];
#pragma unroll
    for (int k = 0; k < kBatchDecode; ++k) {
      const int c = base + tid + kThreads * k;
      if (c >= chunks) break;
      const int h = c / kChunksPerHead;
      const int j = c - h * kChunksPerHead;
      const uint32_t *src = j < kLatent / 8
                                ? reinterpret_cast<const uint32_t *>(a.ql_nope + b * a.ql_stride_token +
                                                                     (int64_t)h * a.ql_stride_head + 8 * j)
                                : reinterpret_cast<const uint32_t *>(a.q_pe + b * a.qpe_stride_token +
                                                                     (int64_t)h * a.qpe_stride_head + 8 * (j - kLatent / 8));
      w[k] = u32x4_t{src[0], src[1], src[2], src[3]};
    }
    if (record_pending) {
      record_pending = false;
      store_record(tid, rl, cs, a.num_records, a.records);
    }
#pragma unroll
    for (int k = 0; k < kBatchDecode; ++k) {
      const int c = base + tid + kThreads * k;
      if (c >= chunks) break;
      const int h = c / kChunksPerHead;
      const int j = c - h * kChunksPerHead;
      if (cs && j >= kLatent / 8) {
        const int jr = j - kLatent / 8;  // rope pairs 4jr .. 4jr+3
#pragma unroll
        for (int i = 0; i < 4; ++i) w[k][i] = rope_word(w[k][i], cs[4 * jr + i], cs[32 + 4 * jr + i]);
      }
      uint32_t *dst =
          reinterpret_cast<uint32_t *>(a.mqa_q + b * a.mq_stride_token + (int64_t)h * a.mq_stride_head + 8 * j);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = w[k][i];
    }
  }
  if (record_pending) store_record(tid, rl, cs, a.num_records, a.records);
}

__global__ __launch_bounds__(kThreads) void prefill_epilogue_kernel(PrefillEpilogueArgs a) {
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.x;
  const float *cs = nullptr;
  if (a.positions) {
    int64_t pos = a.positions[b];
    pos = pos < 0 ? 0 : (pos >= a.max_position ? a.max_position - 1 : pos);
    cs = a.cos_sin + pos * kRope;
  }

  // ---- the record's loads (wave 0) first; encoded after the first batch
  RecordLoads rl = load_record_inputs(tid, b, a.slots, a.kv_c, a.kv_c_stride, a.k_pe, a.k_pe_stride);
  bool record_pending = true;

  // ---- k_out = [k_nope | RoPE(k_pe)] and, with RoPE, q's rope part in
  // place: per head, nope / 8 key chunks from k_nope, 8 rotated k_pe chunks
  // (the same for every head) and 8 q chunks.
  const int nk = a.nope / 8;
  const int per_head = nk + 8 + (cs ? 8 : 0);
  const int chunks = a.num_heads * per_head;
  const uint32_t *pe = reinterpret_cast<const uint32_t *>(a.k_pe + b * a.k_pe_stride);
  // kind of chunk j of a head: 0 = k_nope -> k_out, 1 = RoPE(k_pe) -> k_out,
  // 2 = q's rope part in place.  Batches of kBatchPrefill chunks per thread: all
  // loads first, then the stores (see the decode kernel).
  for (int base = 0; base < chunks; base += kThreads * kBatchPrefill) {
    u32x4_t w[kBatchPrefill];
#pragma unroll
    for (int k = 0; k < kBatchPrefill; ++k) {
      const int c = base + tid + kThreads * k;
      if (c >= chunks) break;
      const int h = c / per_head;
      const int j = c - h * per_head;
      const uint32_t *src;
      if (j < nk)
        src = reinterpret_cast<const uint32_t *>(a.k_nope + b * a.kn_stride_token + (int64_t)h * a.kn_stride_head + 8 * j);
      else if (j < nk + 8)
        src = pe + 4 * (j - nk);
      else
        src = reinterpret_cast<const uint32_t *>(a.q + b * a.q_stride_token + (int64_t)h * a.q_stride_head + a.nope +
                                                 8 * (j - nk - 8));
      w[k] = u32x4_t{src[0], src[1], src[2], src[3]};
    }
    if (record_pending) {
      record_pending = false;
      store_record(tid, rl, cs, a.num_records, a.records);
    }
#pragma unroll
    for (int k = 0; k < kBatchPrefill; ++k) {
      const int c = base + tid + kThreads * k;
      if (c >= chunks) break;
      const int h = c / per_head;
      const int j = c - h * per_head;
      uint32_t *dst;
      if (j < nk) {
        dst = reinterpret_cast<uint32_t *>(a.k_out + b * a.ko_stride_token + (int64_t)h * a.ko_stride_head + 8 * j);
      } else {
        const int jr = j < nk + 8 ? j - nk : j - nk - 8;  // rope pairs 4jr .. 4jr+3
        if (cs) {
#pragma unroll
          for (int i = 0; i < 4; ++i) w[k][i] = rope_word(w[k][i], cs[4 * jr + i], cs[32 + 4 * jr + i]);
        }
        dst = j < nk + 8 ? reinterpret_cast<uint32_t *>(a.k_out + b * a.ko_stride_token +
                                                        (int64_t)h * a.ko_stride_head + a.nope + 8 * jr)
                         : reinterpret_cast<uint32_t *>(a.q + b * a.q_stride_token + (int64_t)h * a.q_stride_head +
                                                        a.nope + 8 * jr);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = w[k][i];
    }
  }
  if (record_pending) store_record(tid, rl, cs, a.num_records, a.records);
}

}  // namespace

hipError_t launch_prefill_epilogue(const PrefillEpilogueArgs &a, hipStream_t stream) {
  prefill_epilogue_kernel<<<dim3((unsigned)a.num_tokens), dim3(kThreads), 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_decode_epilogue(const DecodeEpilogueArgs &a, hipStream_t stream) {
  decode_epilogue_kernel<<<dim3((unsigned)a.num_tokens), dim3(kThreads), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace mla
