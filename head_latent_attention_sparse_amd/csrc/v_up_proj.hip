// W_UV up-projection of the latent attention output, with the optional
// sigmoid gate, for gfx950.
//
// What it computes is _v_up_proj on the vllm.models.kimi_k3.nvidia.mla page
// (per head h: [T, 512] latent rows times W_UV[h], the (N, L, V) = [H, 512,
// 128] weight that process_weights_after_loading splits out of kv_b_proj),
// followed by the gate of the layer's forward (attn_out times the sigmoid of
// the g_proj output, [T, H * 128]):
//     out[t, h, v] = bf16( (sum_l latent[t, h, l] * W_UV[h, l, v]) * sigmoid(gate[t, 128h + v]) )
// with float32 accumulation on the matrix cores, the gate applied in
// float32, and one round to nearest even.
//
// Memory-bound (about 86 FLOP per byte at H = 16), so the design keeps the
// latent read exactly once and keeps HBM busy: a workgroup takes one head,
// holds that head's whole W_UV (128 KB) in registers as MFMA B fragments
// (wave w owns output columns 32w .. 32w+31; the weight is brought in with
// coalesced loads and transposed through LDS), and streams 32-row latent
// tiles and their gate rows with a two-tile register pipeline (loads are
// unconditional, so each wait covers exactly the tile it needs).  With one
// wave per SIMD nothing hides LDS latency, so each tile's A fragments are
// read from LDS four k-steps ahead of their MFMAs.  A tile's 32 x 128
// float32 result is staged in LDS, so the gate is applied and the output
// written in coalesced 16-byte pieces.
#include "device_utils.h"
#include "merge_acc.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;           // wave w owns output columns 32w .. 32w+31
constexpr int kV = 128;                          // v_head_dim
constexpr int kTileRows = 32;
constexpr int kKSteps = kLatent / 32;            // 16 MFMA k-steps of 32
constexpr int kAPitch = kLatent + 8;             // bf16 per LDS latent row (1040 B: conflict-free 16-B reads)
constexpr int kOPitch = kV + 4;                  // floats per LDS output row
constexpr int kWRows = 128;                      // W_UV rows per transposition pass
constexpr int kWPitch = kV + 4;                  // bf16 per LDS weight row (264 B)
constexpr int kABytes = kTileRows * kAPitch * 2;
constexpr int kOBytes = kTileRows * kOPitch * 4;
constexpr int kWBytes = kWRows * kWPitch * 2;
constexpr int kSmem = (kABytes + kOBytes) > kWBytes ? (kABytes + kOBytes) : kWBytes;
constexpr int kLatChunks = kTileRows * kLatent / 8 / kThreads;  // 8 x 16 B of latent per thread and tile
constexpr int kOutChunks = kTileRows * kV / 8 / kThreads;       // 2 x 8 outputs per thread and tile
static_assert(kWRows * kV / 8 / kThreads == 8, "weight pass: 8 chunks per thread");

struct TileRegs {
  u32x4_t lat[kLatChunks];
  u32x4_t gate[kOutChunks];
};

template <bool kGate, bool kPrepared>
__global__ __launch_bounds__(kThreads, 1) void v_up_proj_kernel(VUpProjArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmem];
  uint16_t *s_a = reinterpret_cast<uint16_t *>(smem);
  float *s_o = reinterpret_cast<float *>(smem + kABytes);
  uint16_t *s_w = reinterpret_cast<uint16_t *>(smem);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  // job = (head, part): a head's parts share an XCD and its copy of W_UV[h]
  const int64_t jobs = (int64_t)a.parts * a.num_heads;
  const int64_t job = xcd_job(blockIdx.x, jobs);
  if (job >= jobs) return;  // whole workgroup
  const int h = (int)(job / a.parts);
  const int64_t part = job - (int64_t)h * a.parts;
  const int64_t tiles = (a.num_tokens + kTileRows - 1) / kTileRows;

  // ---- tile loads.  Latent chunk q = tid + 256k of the tile's 32 x 64
  // 16-byte chunks: row q / 64, chunk q % 64 (a wave reads a whole row).
  // Output / gate chunk q = tid + 256k of 32 x 16: row q / 16, chunk q % 16.
  // A tile index past the end reloads the last tile, and rows past the end
  // repeat the last row, so every load is unconditional and in bounds.
  auto load_tile = [&](int64_t tile, TileRegs &r) {
    tile = tile < tiles ? tile : tiles - 1;
#pragma unroll
    for (int k = 0; k < kLatChunks; ++k) {
      const int q = tid + kThreads * k;
      int64_t row = tile * kTileRows + (q >> 6);
      row = row < a.num_tokens ? row : a.num_tokens - 1;
      r.lat[k] = *reinterpret_cast<const u32x4_t *>(a.latent + row * a.lat_st + (int64_t)h * a.lat_sh + 8 * (q & 63));
    }
    if (kGate) {
#pragma unroll
      for (int k = 0; k < kOutChunks; ++k) {
        const int q = tid + kThreads * k;
        int64_t row = tile * kTileRows + (q >> 4);
        row = row < a.num_tokens ? row : a.num_tokens - 1;
        const uint32_t *gp = reinterpret_cast<const uint32_t *>(a.gate + row * a.gate_st + (int64_t)h * kV + 8 * (q & 15));
        r.gate[k] = u32x4_t{gp[0], gp[1], gp[2], gp[3]};
      }
    }
  };

  // the first two tiles load while the weights are set up
  const int64_t step = a.parts;
  TileRegs r0, r1;
  int64_t tile = part;
  load_tile(tile, r0);
  load_tile(tile + step, r1);

  // ---- W_UV[h] as B fragments: bw[s][j] holds, for lane (c, g), rows
  // 32s + 8g .. +7 of column 32 * wave + 16j + c.  Four passes of 128 rows:
  // coalesced 16-byte loads into LDS (pitch 264 B: the 4 row groups of a
  // read land 16 banks apart), then 2-byte reads down the columns.
  bf16x8_t bw[kKSteps][2];
  if (kPrepared) {
    // the fragments in the order prepare_w_uv_kernel wrote them: one
    // 16-byte load each, no staging
    const u32x4_t *wp = reinterpret_cast<const u32x4_t *>(a.w) + ((int64_t)h * kWaves + wave) * (kKSteps * 2 * 64);
#pragma unroll
    for (int s = 0; s < kKSteps; ++s)
#pragma unroll
      for (int j = 0; j < 2; ++j) bw[s][j] = as_bf16x8(wp[(s * 2 + j) * 64 + lane]);
  } else {
    const uint16_t *w = a.w + (int64_t)h * kLatent * kV;
    u32x4_t wr[kLatent / kWRows][8];  // every pass's loads in flight at once
#pragma unroll
    for (int pass = 0; pass < kLatent / kWRows; ++pass)
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int q = tid + kThreads * k;  // row q / 16, chunk q % 16 of the pass
        wr[pass][k] = *reinterpret_cast<const u32x4_t *>(w + (int64_t)(kWRows * pass + (q >> 4)) * kV + 8 * (q & 15));
      }
#pragma unroll
    for (int pass = 0; pass < kLatent / kWRows; ++pass) {
      if (pass > 0) __syncthreads();  // the previous pass's reads are done
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int q = tid + kThreads * k;
        uint32_t *d = reinterpret_cast<uint32_t *>(s_w + (q >> 4) * kWPitch + 8 * (q & 15));
        *reinterpret_cast<u32x2_t *>(d) = u32x2_t{wr[pass][k].x, wr[pass][k].y};
        *reinterpret_cast<u32x2_t *>(d + 2) = u32x2_t{wr[pass][k].z, wr[pass][k].w};
      }
      __syncthreads();
#pragma unroll
      for (int sl = 0; sl < kWRows / 32; ++sl) {
        const int s = pass * (kWRows / 32) + sl;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const uint16_t *col = s_w + (32 * sl + 8 * g) * kWPitch + 32 * wave + 16 * j + c;
          uint32_t v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (uint32_t)col[(2 * e) * kWPitch] | ((uint32_t)col[(2 * e + 1) * kWPitch] << 16);
          bw[s][j] = as_bf16x8(u32x4_t{v[0], v[1], v[2], v[3]});
        }
      }
    }
    __syncthreads();  // the weight staging area becomes the tile buffers
  }

  auto compute_tile = [&](int64_t tile, const TileRegs &r) {
    __syncthreads();  // the previous tile's LDS reads are done
#pragma unroll
    for (int k = 0; k < kLatChunks; ++k) {
      const int q = tid + kThreads * k;
      *reinterpret_cast<u32x4_t *>(s_a + (q >> 6) * kAPitch + 8 * (q & 63)) = r.lat[k];
    }
    __syncthreads();
    floatx4_t acc[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m) acc[m][0] = acc[m][1] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    // A fragments in blocks of kBlk k-steps, the next block's LDS reads
    // issued before the current block's MFMAs (one wave per SIMD: nothing
    // else would hide the LDS latency)
    constexpr int kBlk = 4;
    bf16x8_t af[2][2][kBlk];  // [buffer][m][k-step in block]
    auto read_block = [&](int blk, bf16x8_t (&dst)[2][kBlk]) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int i = 0; i < kBlk; ++i)
          dst[m][i] = as_bf16x8(*reinterpret_cast<const u32x4_t *>(s_a + (16 * m + c) * kAPitch + 32 * (kBlk * blk + i) + 8 * g));
    };
    read_block(0, af[0]);
#pragma unroll
    for (int blk = 0; blk < kKSteps / kBlk; ++blk) {
      if (blk + 1 < kKSteps / kBlk) read_block(blk + 1, af[(blk + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < kBlk; ++i)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          acc[m][0] = mfma_16x16x32_bf16(af[blk & 1][m][i], bw[kBlk * blk + i][0], acc[m][0]);
          acc[m][1] = mfma_16x16x32_bf16(af[blk & 1][m][i], bw[kBlk * blk + i][1], acc[m][1]);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
    // D of m-tile m, n-tile j: lane (c, g) holds rows 16m + 4g + r, column 32 * wave + 16j + c
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_o[(16 * m + 4 * g + i) * kOPitch + 32 * wave + 16 * j + c] = acc[m][j][i];
    __syncthreads();
    // All results first, then unconditional stores: a store counts in the
    // same counter as the loads, and a conditional one would make every later
    // wait assume it was not issued (so waits would cover the prefetched
    // tiles too).  A row past the end was computed from the last row's
    // latent and gate (the loads clamp), so it holds exactly the last row's
    // bits and is stored there, rewriting the same value.
    uint32_t res[kOutChunks][4];
#pragma unroll
    for (int k = 0; k < kOutChunks; ++k) {
      const int q = tid + kThreads * k;
      const int rr = q >> 4, ch = q & 15;
      const floatx4_t y0 = *reinterpret_cast<const floatx4_t *>(s_o + rr * kOPitch + 8 * ch);
      const floatx4_t y1 = *reinterpret_cast<const floatx4_t *>(s_o + rr * kOPitch + 8 * ch + 4);
      float y[8] = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
      if (kGate) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t gw = r.gate[k][i];
          y[2 * i] *= __builtin_amdgcn_rcpf(1.0f + __expf(-as_float(gw << 16)));
          y[2 * i + 1] *= __builtin_amdgcn_rcpf(1.0f + __expf(-as_float(gw & 0xFFFF0000u)));
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) res[k][i] = pack_bf16x2(y[2 * i], y[2 * i + 1]);
    }
#pragma unroll
    for (int k = 0; k < kOutChunks; ++k) {
      const int q = tid + kThreads * k;
      int64_t row = tile * kTileRows + (q >> 4);
      row = row < a.num_tokens ? row : a.num_tokens - 1;
      uint32_t *dst = reinterpret_cast<uint32_t *>(a.out + row * a.out_st + (int64_t)h * a.out_sh + 8 * (q & 15));
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = res[k][i];
    }
  };

  // ---- two tiles in flight: while tile i is computed, tiles i+1 and i+2
  // are loading (into the register set tile i used, once it is in LDS).
  // The steady loop runs while both tiles it prefetches exist, so its loads
  // are unconditional; the last (up to three) tiles follow with only the
  // loads that exist.
  for (; tile + 3 * step < tiles; tile += 2 * step) {
    compute_tile(tile, r0);
    load_tile(tile + 2 * step, r0);
    compute_tile(tile + step, r1);
    load_tile(tile + 3 * step, r1);
  }
  if (tile < tiles) {
    compute_tile(tile, r0);
    if (tile + 2 * step < tiles) load_tile(tile + 2 * step, r0);
    if (tile + step < tiles) compute_tile(tile + step, r1);
    if (tile + 2 * step < tiles) compute_tile(tile + 2 * step, r0);
  }
}

// ---- The split-KV merge fused with the up-projection on prepared weights.
// A workgroup of eight waves takes kFRows = 4 rows of one head.  Merge:
// thread (row tid / 128, column quad tid % 128) merges its chunk partials
// into kLanes accumulators, chunk s into accumulator s % kLanes in
// increasing s, then folds accumulators 1.. into 0: the order
// merge_kernel<kLanes> uses (with the same fused multiply-adds), so the
// merged bf16 row is that kernel's.  The row goes to `out` and, as the same
// bf16 values, into the LDS A tile (rows 4..15 zero); wave w' then
// multiplies by the 16 columns 16w' .. 16w'+15 of W_UV[h] (its B fragments
// in registers: fragment j = w' % 2 of v_up_proj_kernel's wave w' / 2,
// k-steps in that kernel's order) and applies the gate as that kernel does.
// Rows past the end load nothing and store nothing.
constexpr int kFThreads = 512;
constexpr int kFWaves = kFThreads / 64;
constexpr int kFRows = kFThreads / 128;  // one (row, column quad) per thread
constexpr int kFBatch = 8;               // chunks with their loads in flight together
static_assert(kFRows <= 16 && kFWaves * 16 == kV, "one MFMA row tile, 16 columns per wave");

template <bool kGate, bool kLse, int kLanes>
__global__ __launch_bounds__(kFThreads, 1) void merge_v_up_proj_kernel(MergeVUpProjArgs a) {
  static_assert(kFBatch % kLanes == 0, "a batch starts at chunk lane 0");
  __shared__ __attribute__((aligned(16))) uint16_t s_a[16 * kAPitch];
  __shared__ __attribute__((aligned(16))) float s_o[kFRows * kOPitch];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  // job = (head, row block): a head's row blocks share an XCD and its copy of W_UV[h]
  const int64_t blocks = (a.num_tokens + kFRows - 1) / kFRows;
  const int64_t jobs = blocks * a.num_heads;
  const int64_t job = xcd_job(blockIdx.x, jobs);
  if (job >= jobs) return;  // whole workgroup
  const int h = (int)(job / blocks);
  const int64_t row0 = (job - (int64_t)h * blocks) * kFRows;

  // this wave's 16 columns of W_UV[h] as B fragments (requested first, used last)
  bf16x8_t bw[kKSteps];
  {
    const u32x4_t *wp = reinterpret_cast<const u32x4_t *>(a.w_prepared) +
                        ((int64_t)h * kWaves + (wave >> 1)) * (kKSteps * 2 * 64) + (wave & 1) * 64 + lane;
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) bw[s] = as_bf16x8(wp[s * 2 * 64]);
  }
  // the storing threads' gate words, requested now rather than after the projection
  uint32_t gate_w[4] = {0u, 0u, 0u, 0u};
  if (kGate && tid < kFRows * 16 && row0 + (tid >> 4) < a.num_tokens) {
    const uint32_t *gp =
        reinterpret_cast<const uint32_t *>(a.gate + (row0 + (tid >> 4)) * a.gate_st + (int64_t)h * kV + 8 * (tid & 15));
#pragma unroll
    for (int i = 0; i < 4; ++i) gate_w[i] = gp[i];
  }
  for (int i = tid; i < (16 - kFRows) * kAPitch / 8; i += kFThreads)
    reinterpret_cast<u32x4_t *>(s_a + kFRows * kAPitch)[i] = u32x4_t{0u, 0u, 0u, 0u};

  // ---- merge
  {
    const int r = tid >> 7, cq = tid & 127;
    const int64_t t = row0 + r;
    int32_t c0 = 0, nc = 0;
    if (t < a.num_tokens) {
      c0 = a.ws_prefix[t];
      nc = a.ws_prefix[t + 1] - c0;
    }
    const float *lp = a.ws_lse + (int64_t)c0 * a.num_heads + h;                     // chunk s at lp[s * H]
    const float *op = a.ws_out + ((int64_t)c0 * a.num_heads + h) * kLatent + 4 * cq;  // at op[s * H * 512]
    MergeAcc acc[kLanes];
#pragma unroll
    for (int l = 0; l < kLanes; ++l) acc[l] = merge_acc_empty();
    for (int base = 0; base < nc; base += kFBatch) {
      float ls[kFBatch];
      floatx4_t os[kFBatch];
#pragma unroll
      for (int j = 0; j < kFBatch; ++j) {
        const int s = base + j;
        const int sc = s < nc ? s : base;  // in range: base < nc
        ls[j] = lp[(int64_t)sc * a.num_heads];
        os[j] = *reinterpret_cast<const floatx4_t *>(op + (int64_t)sc * a.num_heads * kLatent);
        if (s >= nc) ls[j] = -INFINITY;
      }
#pragma unroll
      for (int j = 0; j < kFBatch; ++j) merge_add(acc[j % kLanes], ls[j], os[j]);
    }
#pragma unroll
    for (int l = 1; l < kLanes; ++l) merge_combine(acc[0], acc[l]);
    const float inv = acc[0].l > 0.f ? 1.f / acc[0].l : 0.f;
    const uint32_t lo = pack_bf16x2(acc[0].o[0] * inv, acc[0].o[1] * inv);
    const uint32_t hi = pack_bf16x2(acc[0].o[2] * inv, acc[0].o[3] * inv);
    *reinterpret_cast<u32x2_t *>(s_a + r * kAPitch + 4 * cq) = u32x2_t{lo, hi};
    if (t < a.num_tokens) {
      uint32_t *dst = reinterpret_cast<uint32_t *>(a.out + t * a.out_st + (int64_t)h * a.out_sh + 4 * cq);
      dst[0] = lo;
      dst[1] = hi;
      if (kLse && cq == 0)
        a.lse[t * a.num_heads + h] = acc[0].m == -INFINITY ? -INFINITY : (acc[0].m + fast_log2(acc[0].l)) * kLn2;
    }
  }
  __syncthreads();

  // ---- projection: rows 16 (kFRows real) x columns 16 * wave + c
  floatx4_t acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kKSteps; ++s) {
    const bf16x8_t af = as_bf16x8(*reinterpret_cast<const u32x4_t *>(s_a + c * kAPitch + 32 * s + 8 * g));
    acc2 = mfma_16x16x32_bf16(af, bw[s], acc2);
  }
  // D: lane (c, g) holds rows 4g + i, column 16 * wave + c
  if (4 * g < kFRows) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * g + i < kFRows) s_o[(4 * g + i) * kOPitch + 16 * wave + c] = acc2[i];
  }
  __syncthreads();
  if (tid < kFRows * 16) {
    const int rr = tid >> 4, ch = tid & 15;
    const int64_t t = row0 + rr;
    if (t < a.num_tokens) {
      const floatx4_t y0 = *reinterpret_cast<const floatx4_t *>(s_o + rr * kOPitch + 8 * ch);
      const floatx4_t y1 = *reinterpret_cast<const floatx4_t *>(s_o + rr * kOPitch + 8 * ch + 4);
      float y[8] = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
      if (kGate) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t gw = gate_w[i];
          y[2 * i] *= __builtin_amdgcn_rcpf(1.0f + __expf(-as_float(gw << 16)));
          y[2 * i + 1] *= __builtin_amdgcn_rcpf(1.0f + __expf(-as_float(gw & 0xFFFF0000u)));
        }
      }
      uint32_t *dst = reinterpret_cast<uint32_t *>(a.v_out + t * a.v_st + (int64_t)h * a.v_sh + 8 * ch);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = pack_bf16x2(y[2 * i], y[2 * i + 1]);
    }
  }
}

// W_UV in the kernel's B-fragment order: fragment (h, w, s, j) of lane
// (c, g) = rows 32s + 8g .. +7 of column 32w + 16j + c of W_UV[h], 8 bf16
// values (row order, the first in the low half), stored as 16 bytes at
// index ((((h * 4 + w) * 16 + s) * 2 + j) * 64 + lane).  One thread per
// fragment.
__global__ __launch_bounds__(256) void prepare_w_uv_kernel(const uint16_t *w, uint16_t *wp, int64_t fragments) {
  const int64_t f = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (f >= fragments) return;
  const int lane = (int)(f & 63), c = lane & 15, g = lane >> 4;
  const int j = (int)((f >> 6) & 1);
  const int s = (int)((f >> 7) & (kKSteps - 1));
  const int64_t hw = f >> 11;  // h * 4 + wave
  const int wave = (int)(hw & 3);
  const int64_t h = hw >> 2;
  const uint16_t *col = w + h * kLatent * kV + (int64_t)(32 * s + 8 * g) * kV + 32 * wave + 16 * j + c;
  uint32_t v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = (uint32_t)col[(2 * e) * kV] | ((uint32_t)col[(2 * e + 1) * kV] << 16);
  *reinterpret_cast<u32x4_t *>(wp + f * 8) = u32x4_t{v[0], v[1], v[2], v[3]};
}
static_assert(kKSteps == 16 && kWaves == 4, "fragment index layout");

}  // namespace

hipError_t launch_v_up_proj(const VUpProjArgs &a, int num_cus, hipStream_t stream) {
  const int64_t tiles = (a.num_tokens + kTileRows - 1) / kTileRows;
  // one workgroup per CU in all (each holds a head's weights in registers)
  int64_t per_head = (num_cus > 0 ? num_cus : 256) / a.num_heads;
  per_head = per_head < 1 ? 1 : (per_head > tiles ? tiles : per_head);
  VUpProjArgs k = a;
  k.parts = (int32_t)per_head;
  const dim3 grid((unsigned)xcd_grid(per_head * a.num_heads));
  if (a.w_prepared) {
    if (a.gate)
      v_up_proj_kernel<true, true><<<grid, dim3(kThreads), 0, stream>>>(k);
    else
      v_up_proj_kernel<false, true><<<grid, dim3(kThreads), 0, stream>>>(k);
  } else {
    if (a.gate)
      v_up_proj_kernel<true, false><<<grid, dim3(kThreads), 0, stream>>>(k);
    else
      v_up_proj_kernel<false, false><<<grid, dim3(kThreads), 0, stream>>>(k);
  }
  return hipGetLastError();
}

template <bool kGate, bool kLse>
void launch_merge_v_up_proj_lanes(const MergeVUpProjArgs &a, int lanes, hipStream_t stream) {
  const dim3 grid((unsigned)xcd_grid((int64_t)((a.num_tokens + kFRows - 1) / kFRows) * a.num_heads));
  if (lanes == 2)
    merge_v_up_proj_kernel<kGate, kLse, 2><<<grid, dim3(kFThreads), 0, stream>>>(a);
  else if (lanes == 4)
    merge_v_up_proj_kernel<kGate, kLse, 4><<<grid, dim3(kFThreads), 0, stream>>>(a);
  else
    merge_v_up_proj_kernel<kGate, kLse, 8><<<grid, dim3(kFThreads), 0, stream>>>(a);
}

hipError_t launch_merge_v_up_proj(const MergeVUpProjArgs &a, int lanes, hipStream_t stream) {
  if (lanes != 2 && lanes != 4 && lanes != 8) return hipErrorInvalidValue;
  if (a.gate) {
    if (a.lse)
      launch_merge_v_up_proj_lanes<true, true>(a, lanes, stream);
    else
      launch_merge_v_up_proj_lanes<true, false>(a, lanes, stream);
  } else {
    if (a.lse)
      launch_merge_v_up_proj_lanes<false, true>(a, lanes, stream);
    else
      launch_merge_v_up_proj_lanes<false, false>(a, lanes, stream);
  }
  return hipGetLastError();
}

hipError_t launch_prepare_w_uv(const uint16_t *w, uint16_t *w_prepared, int32_t num_heads, hipStream_t stream) {
  const int64_t fragments = (int64_t)num_heads * kLatent * kV / 8;
  prepare_w_uv_kernel<<<dim3((unsigned)((fragments + 255) / 256)), dim3(256), 0, stream>>>(w, w_prepared, fragments);
  return hipGetLastError();
}

}  // namespace mla
