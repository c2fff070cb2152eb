// Gather + upconvert for gfx950: a context chunk's fp8_ds_mla records,
// addressed through the block table, into a bf16 [tokens, 576] workspace.
//
// What it computes is cp_gather_and_upconvert_fp8_kv_cache as the kimi_k3
// nvidia mla page calls it in _gather_context_latent (src_cache, dst =
// workspace[:toks], block_table, workspace_starts = cu_seq_lens, batch_size,
// seq_starts): workspace row cu[r] + j holds context position
// p = seq_starts[r] + j of request r, for j < cu[r+1] - cu[r]; the record of
// p is block_table[r][p / block_size] * block_size + p % block_size; the row
// is [latent | rope] in the model dtype (bf16), latent[d] =
// bf16(f32(E4M3(code[d])) * scale[d / 128]) (float32 product, then round to
// nearest even) and the rope copied as stored.  A row with no valid source
// (block id outside the pool, position past the table's width, row outside
// every request) is written as zeros: it reads a zero record instead.
//
// Each wave moves 8 consecutive rows: lanes 0..7 resolve one row's record
// each (binary search of cu, one block-table read) and every lane then loads
// its 8 codes and its tile scale of all 8 records before converting, so a
// wave keeps 8 records in flight.  Lane l owns latent columns 8l .. 8l+7
// (one 16-byte store per row) and, for l < 32, rope word l.
#include "device_utils.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerWave = 8;
constexpr int kRowsPerBlock = kRowsPerWave * (kThreads / 64);

// Read in place of a record for a row with no source: all fields zero.
__device__ __attribute__((aligned(16))) uint8_t g_zero_record[kRecordBytes];

__global__ __launch_bounds__(kThreads) void gather_upconvert_kernel(GatherArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row0 = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6) * kRowsPerWave;

  // ---- lanes 0..7: the record of row row0 + lane (-1: none)
  int64_t src = -1;
  if (lane < kRowsPerWave) {
    const int64_t row = row0 + lane;
    if (row < a.num_tokens && a.batch > 0 && row >= a.cu[0] && row < a.cu[a.batch]) {
      // the request r with cu[r] <= row < cu[r + 1]
      int lo = 0, hi = a.batch - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.cu[mid] <= row) lo = mid; else hi = mid - 1;
      }
      const int64_t pos = (a.starts ? (int64_t)a.starts[lo] : 0) + (row - a.cu[lo]);
      const int64_t bi = pos >= 0 ? pos / a.block_size : -1;
      if (bi >= 0 && bi < a.bt_width) {
        const int64_t blk = a.block_table[lo * a.bt_stride + bi];
        const int64_t slot = blk * a.block_size + pos % a.block_size;
        if (blk >= 0 && slot < a.num_records) src = slot;
      }
    }
  }

  // ---- every lane: its codes and tile scale of the 8 records, and rope word
  u32x2_t codes[kRowsPerWave];
  float scale[kRowsPerWave];
  uint32_t rope[kRowsPerWave];
  int64_t srcs[kRowsPerWave];
#pragma unroll
  for (int k = 0; k < kRowsPerWave; ++k) {
    srcs[k] = __shfl(src, k, 64);
    const uint8_t *rec = srcs[k] >= 0 ? a.records + srcs[k] * kRecordBytes : g_zero_record;
    codes[k] = *reinterpret_cast<const u32x2_t *>(rec + 8 * lane);
    scale[k] = *reinterpret_cast<const float *>(rec + kScaleOffset + 4 * (lane >> 4));
    rope[k] = *reinterpret_cast<const uint32_t *>(rec + kRopeOffset + 4 * (lane & 31));
  }

#pragma unroll
  for (int k = 0; k < kRowsPerWave; ++k) {
    const int64_t row = row0 + k;
    if (row >= a.num_tokens) break;
    u32x4_t v;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const floatx2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(codes[k][i], false);  // exact
      const floatx2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(codes[k][i], true);
      v[2 * i] = pack_bf16x2(lo.x * scale[k], lo.y * scale[k]);
      v[2 * i + 1] = pack_bf16x2(hi.x * scale[k], hi.y * scale[k]);
    }
    uint16_t *drow = a.dst + row * a.dst_stride;
    *reinterpret_cast<u32x4_t *>(drow + 8 * lane) = v;
    if (lane < 32) reinterpret_cast<uint32_t *>(drow + kLatent)[lane] = rope[k];
  }
}

}  // namespace

hipError_t launch_gather_upconvert(const GatherArgs &a, hipStream_t stream) {
  const int64_t blocks = (a.num_tokens + kRowsPerBlock - 1) / kRowsPerBlock;
  gather_upconvert_kernel<<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace mla
