// Sparse absorbed-MLA forward over fp8_ds_mla records, for gfx950.
//
// What it computes is the sparse_mla_fwd semantics of
// flydsl_sparse_mla_fp8ds_fwd (vLLM API page
// vllm.models.kimi_k3.amd.ops.flydsl_sparse_mla, function docstring): for
// each query row t and head h, softmax(scale * q . k) . v over the row's CSR
// slot list, keys k = [latent | rope] (576), values v = latent (512),
// negative slots masked, an empty row giving out 0 and lse -inf.
//
// Design (one workgroup of 4 waves per row, or per chunk of a row in the
// split-KV pass; 64-key tiles):
//  * the row's query (H x 576 bf16) is read from memory once per workgroup
//    and handed to the waves through LDS, since each wave needs all of it;
//  * the 64 records of a tile (64 x 656 B) are gathered with 16-byte loads
//    into registers one tile ahead (4 threads per record), then stored to
//    LDS as 64 consecutive records; the slot ids of the tile after that are
//    loaded a tile earlier still;
//  * QK^T: wave w scores keys 16w..16w+15 of the tile for all 16 head rows
//    with bf16 dot products (v_mfma_f32_16x16x32_bf16: exact products,
//    float32 accumulation).  The records' E4M3 codes are converted to bf16
//    exactly (every E4M3 value is a bf16 value) and each key's per-128 tile
//    scale multiplies that tile's float32 partial, so the logits carry no
//    rounding of code * scale; the rope part is a plain bf16 product;
//  * the 16x64 logits go through LDS; every wave computes the online-softmax
//    weights of the whole tile in the exp2 domain (scale * log2 e, as the
//    FlyDSL launcher passes it) and keeps identical running max / sum; the
//    running reference only moves when a logit passes it by 2^8;
//  * PV: wave w owns latent tile w (128 columns) and computes
//    O^T[d, h] += V^T[d, key] P^T[key, h] with v_mfma_f32_16x16x32_bf16;
//    P is multiplied by the key's scale of tile w before its bf16 rounding,
//    and V^T comes straight from the record bytes in LDS with the gfx950
//    transposing LDS read (ds_read_b64_tr_b8) and an exact E4M3 -> bf16
//    conversion, so each lane ends up owning one head;
//  * when there are too few rows to fill the GPU, rows are cut into chunks
//    planned on the device (split_plan), each chunk's float32 partial and
//    base-2 LSE go to a workspace, and merge_kernel combines them;
//  * with one workgroup per row and rows of equal length laid out back to
//    back (a top-k selection), each workgroup fetches its first slot ids at
//    the guessed row start while its indptr pair is still in flight.
#include "device_utils.h"
#include "merge_acc.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kTileKeys = 64;
constexpr int kThreads = 256;
constexpr int kChunks = kRecordBytes / 16;                                // 41 x 16 B per record
constexpr int kChunksPerThread = (kChunks + 3) / 4;                       // 11 (4 threads per record)
static_assert(kThreads == 4 * kTileKeys, "gather mapping: 4 threads per record");
static_assert(4 * (kChunksPerThread - 1) + 1 == kChunks, "the last chunk belongs to sub 0 alone");
// Softmax weights may grow to 2^kLazyRescale before the running reference
// (and with it O and the sum) is moved up.
constexpr float kLazyRescale = 8.0f;
constexpr int kLogitPitch = kTileKeys + 4;                                 // floats per head row
// The row's query in LDS: bf16 per head row (576 + 8, so the 16 head rows
// start 4 banks apart) and 16-byte pieces per head.
constexpr int kQPitch = kQkDim + 8;
constexpr int kQPieces = kQkDim / 8;
constexpr int kQStage = (16 * kQPieces + kThreads - 1) / kThreads;  // pieces per thread

typedef __attribute__((address_space(3))) intx2_t lds_intx2_t;

struct FwdKernelArgs {
  const uint16_t *q;
  int64_t q_st, q_sh;
  const uint8_t *rec;
  int64_t num_records;
  const void *indptr;
  const void *indices;
  int64_t nnz;
  float scale_log2;
  int32_t heads;
  uint16_t *out;
  int64_t o_st, o_sh;
  float *lse;
  float *ws_out;
  float *ws_lse;
  int32_t *ws_prefix;
  int32_t tokens;
  int32_t forced_chunk;  // split pass: chunk size if > 0, else chosen by split_plan
  int64_t bound;         // split pass: its workgroups, an upper bound on the chunks
  // second segment (kExtra): its pool and CSR list
  const uint8_t *erec;
  int64_t enum_records;
  const void *eindptr;
  const void *eindices;
  int64_t ennz;
  const float *sink;  // [heads] sink logits (natural-log units of the scaled logits), or nullptr
  int64_t guess_len;  // one workgroup per row: rows most likely start at t * guess_len (0: no guess)
  int32_t direct_single;  // split pass: a row of one chunk writes out / lse itself (the merge skips it)
};

// A workgroup's share of a row.  Entry v of the row (0 <= v < lenp + lene)
// is primary entry beg + v for v < lenp, else extra entry ebeg + v - lenp;
// the workgroup takes entries [vb, ve).
struct RowRange {
  int64_t t, beg, lenp, ebeg, vb, ve;
  int64_t chunk;  // split pass: the chunk's index in row order (its partial's slot)
  bool single;    // split pass: the chunk is its row's only one
};

// Clamp a CSR pair to [0, nnz] (a decreasing pair gives an empty range).
__device__ __forceinline__ void clamp_range(int64_t b, int64_t e, int64_t nnz, int64_t &beg, int64_t &len) {
  b = b < 0 ? 0 : (b > nnz ? nnz : b);
  e = e < b ? b : (e > nnz ? nnz : e);
  beg = b;
  len = e - b;
}

// ---- Split-KV plan, computed by every wave of the partial pass ----
// Each wave computes the same plan on its own (no LDS, no barrier): row
// lengths with the forward's clamping of indptr; a chunk size; each row's
// first chunk (an exclusive prefix); then this workgroup's chunk.  The chunk
// size is `forced` if given, otherwise the smallest C of kPlanCandidates
// multiples of 64 (at least kMinChunk) whose chunk total fits the `bound`
// workgroups, so the partial pass is one round of the shortest chunks; then
// sizes alternating C + kSkewEntries, C - kSkewEntries along the chunk
// order, if that fits too (the longer ones go to the first half of the
// workgroups).  The candidates run from ceil(n / bound) to
// ceil(n / (bound - rows)) (n = sum of lengths, rows = the non-empty ones);
// the last always fits, since sum ceil(len / C) <= n / C + rows.
// Prefix values are capped at `bound`:
// a non-monotone indptr (overlapping rows) loses chunks instead of indexing
// out of range.  Lane l owns rows l, l + 64, ... (at most kPlanRowsPerLane).
constexpr int kMaxSplitRows = 512;
constexpr int kPlanRowsPerLane = kMaxSplitRows / 64;
constexpr uint32_t kMinChunk = 512;
constexpr uint32_t kMaxChunk = 1u << 29;
constexpr int kPlanCandidates = 4;

// ceil(len / c) for 0 <= len <= 2^30 and 64 <= c <= 2^30 (rcp = 1 / c): a
// float estimate (off by at most 2: len / c < 2^24 and the estimate's
// relative error is below 2^-23) and an exact integer correction.
__device__ __forceinline__ int32_t ceil_div_rcp(int32_t len, int32_t c, float rcp) {
  int32_t q = (int32_t)((float)len * rcp);
  int32_t r = len - q * c;
#pragma unroll
  for (int i = 0; i < 3; ++i)
    if (r < 0) {
      q -= 1;
      r += c;
    }
#pragma unroll
  for (int i = 0; i < 3; ++i)
    if (r >= c) {
      q += 1;
      r -= c;
    }
  return q + (r > 0 ? 1 : 0);
}

// Sum and inclusive prefix sum over the 64 lanes of a wave (all lanes
// active): DPP row shifts within each 16-lane row, then row broadcasts of
// lanes 15 and 31 into the rows above.  A lane without a source adds 0.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ int32_t dpp_i32(int32_t v) {
  return __builtin_amdgcn_update_dpp(0, v, kCtrl, kRowMask, 0xf, false);
}
__device__ __forceinline__ int32_t wave_incl_scan(int32_t v) {
  v += dpp_i32<0x111, 0xf>(v);  // row_shr:1
  v += dpp_i32<0x112, 0xf>(v);  // row_shr:2
  v += dpp_i32<0x114, 0xf>(v);  // row_shr:4
  v += dpp_i32<0x118, 0xf>(v);  // row_shr:8
  v += dpp_i32<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_i32<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}
__device__ __forceinline__ int32_t wave_sum(int32_t v) { return __builtin_amdgcn_readlane(wave_incl_scan(v), 63); }

constexpr int32_t kSkewEntries = 128;  // two tiles

// Chunks of one row of len entries when chunk sizes alternate along the
// chunk order: even chunks hold `big` entries, odd ones `small`
// (big + small = c2, rcp2 = 1 / c2).  k0 / k1: the chunks it needs when its
// first chunk is even / odd.  With big == small this is ceil(len / big).
__device__ __forceinline__ void row_chunk_counts(int32_t len, int32_t big, int32_t small, float rcp2, int32_t &k0,
                                                 int32_t &k1) {
  const int32_t c2 = big + small;
  const int32_t q = ceil_div_rcp(len + 1, c2, rcp2) - 1;  // floor(len / c2)
  const int32_t rem = len - q * c2;
  k0 = 2 * q + (rem == 0 ? 0 : (rem <= big ? 1 : 2));
  k1 = 2 * q + (rem == 0 ? 0 : (rem <= small ? 1 : 2));
}

// Inclusive scan over the lanes (rows in order) of the maps "first chunk's
// parity p -> chunks of the rows so far": a lane holds (a0, a1) = its row's
// (k0, k1) and ends with the composition of lanes 0..lane, which is
// associative: (left then self)(p) = left(p) + self((p + left(p)) & 1).
// The same DPP network as wave_incl_scan; a lane without a source reads
// (0, 0), the identity map.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ void parity_step(int32_t &a0, int32_t &a1) {
  const int32_t l0 = dpp_i32<kCtrl, kRowMask>(a0), l1 = dpp_i32<kCtrl, kRowMask>(a1);
  const int32_t n0 = l0 + ((l0 & 1) ? a1 : a0);
  const int32_t n1 = l1 + ((l1 & 1) ? a0 : a1);
  a0 = n0;
  a1 = n1;
}
__device__ __forceinline__ void wave_scan_parity(int32_t &a0, int32_t &a1) {
  parity_step<0x111, 0xf>(a0, a1);  // row_shr:1
  parity_step<0x112, 0xf>(a0, a1);  // row_shr:2
  parity_step<0x114, 0xf>(a0, a1);  // row_shr:4
  parity_step<0x118, 0xf>(a0, a1);  // row_shr:8
  parity_step<0x142, 0xa>(a0, a1);  // row_bcast:15 into rows 1 and 3
  parity_step<0x143, 0xc>(a0, a1);  // row_bcast:31 into rows 2 and 3
}
// The value of the lane below (0 for lane 0): DPP wave_shr:1.
__device__ __forceinline__ int32_t lane_below(int32_t v) { return dpp_i32<0x138, 0xf>(v); }

template <typename IdxT, bool kExtra>
__device__ bool split_plan(const FwdKernelArgs &p, RowRange &rr) {
  const int lane = threadIdx.x & 63;
  const IdxT *indptr = static_cast<const IdxT *>(p.indptr);
  const int32_t tokens = p.tokens;  // <= kMaxSplitRows
  const int nj = (tokens + 63) >> 6;  // row slots in use per lane (uniform)

  // this lane's rows: both segments' offsets, all requested at once and
  // unconditionally (a slot past the last row reads indptr[T] twice: an
  // empty row), so no load waits on another
  IdxT x0[kPlanRowsPerLane], x1[kPlanRowsPerLane], y0[kPlanRowsPerLane], y1[kPlanRowsPerLane];
#pragma unroll
  for (int j = 0; j < kPlanRowsPerLane; ++j) {
    const int r = lane + 64 * j < tokens ? lane + 64 * j : tokens;
    const int r1 = r < tokens ? r + 1 : tokens;
    x0[j] = indptr[r];
    x1[j] = indptr[r1];
    y0[j] = y1[j] = 0;
    if (kExtra) {
      const IdxT *eindptr = static_cast<const IdxT *>(p.eindptr);
      y0[j] = eindptr[r];
      y1[j] = eindptr[r1];
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // all loads in flight before any use
  // len = the row's entries over both segments (< 2^30)
  int32_t len[kPlanRowsPerLane], rb[kPlanRowsPerLane], lp[kPlanRowsPerLane], eb[kPlanRowsPerLane];
#pragma unroll
  for (int j = 0; j < kPlanRowsPerLane; ++j) {
    int64_t b, l;
    clamp_range((int64_t)x0[j], (int64_t)x1[j], p.nnz, b, l);
    rb[j] = (int32_t)b;  // nnz < 2^29
    lp[j] = (int32_t)l;
    len[j] = (int32_t)l;
    eb[j] = 0;
    if (kExtra) {
      clamp_range((int64_t)y0[j], (int64_t)y1[j], p.ennz, b, l);
      eb[j] = (int32_t)b;
      len[j] += (int32_t)l;
    }
  }

  // Chunk sizes: even chunks (in row order) hold `big` entries, odd ones
  // `small`.  Forced: one size.  Otherwise `big` = C + kSkewEntries and
  // `small` = C - kSkewEntries when that fits the bound too, else both C.
  // Even chunk 2i goes to workgroup i and odd chunk 2i + 1 to workgroup
  // W / 2 + i: workgroups are dispatched in index order, one per compute
  // unit first, and a unit's first workgroup gets its loads served ahead
  // of its second, which with equal chunks finishes last, alone on the
  // unit.  Where a workgroup lands only changes the speed: the chunks, and
  // so the results, depend on indptr and the bound alone.
  const int32_t cap = (int32_t)p.bound;
  // Per row slot: the row's chunk counts (k0, k1) and their parity scan, for
  // the sizes in use; returns all rows' chunks (uncapped).
  int32_t K0[kPlanRowsPerLane], K1[kPlanRowsPerLane], S0[kPlanRowsPerLane], S1[kPlanRowsPerLane];
  auto scan_rows = [&](int32_t bg, int32_t sm) {
    const float rcp2 = 1.0f / (float)(bg + sm);
    int32_t f = 0;
#pragma unroll
    for (int j = 0; j < kPlanRowsPerLane; ++j) {
      K0[j] = K1[j] = S0[j] = S1[j] = 0;
      if (j >= nj) continue;
      row_chunk_counts(len[j], bg, sm, rcp2, K0[j], K1[j]);
      S0[j] = K0[j];
      S1[j] = K1[j];
      wave_scan_parity(S0[j], S1[j]);
      f += __builtin_amdgcn_readlane((f & 1) ? S1[j] : S0[j], 63);
    }
    return f;
  };
  int32_t big = p.forced_chunk, small = p.forced_chunk;
  bool scanned = false;
  if (p.forced_chunk <= 0) {
    // For a malformed (overlapping) indptr n may wrap; every chunk size
    // below is still in [kMinChunk - kSkewEntries, kMaxChunk + kSkewEntries],
    // and the caps keep chunks in range.
    int32_t nl = 0, rl = 0;
#pragma unroll
    for (int j = 0; j < kPlanRowsPerLane; ++j) {
      if (j >= nj) break;
      nl += len[j];
      rl += len[j] > 0;
    }
    const uint32_t n = (uint32_t)wave_sum(nl);
    const uint32_t rows = (uint32_t)wave_sum(rl);
    const uint32_t bound = (uint32_t)p.bound;  // the library's plan: twice the compute units
    auto cdiv = [](uint32_t a, uint32_t b) { return a / b + (a % b != 0u ? 1u : 0u); };
    auto up64 = [](uint32_t x) { return (min(x, kMaxChunk) + 63u) & ~63u; };
    const uint32_t lo = max(kMinChunk, up64(cdiv(n, bound)));
    const uint32_t slack = bound > rows ? bound - rows : 1u;
    const uint32_t hi = min(max(lo, up64(cdiv(n, slack))), kMaxChunk);
    const uint32_t step = max(64u, up64((hi - lo) / (kPlanCandidates - 1)));
    int32_t c = (int32_t)hi;  // always fits
#pragma unroll
    for (int k = kPlanCandidates - 1; k >= 0; --k) {
      const int32_t ck = (int32_t)min(lo + step * k, hi);
      const float rcp = 1.0f / (float)ck;
      int32_t cl = 0;
#pragma unroll
      for (int j = 0; j < kPlanRowsPerLane; ++j) {
        if (j >= nj) break;
        cl += ceil_div_rcp(len[j], ck, rcp);
      }
      if ((uint32_t)wave_sum(cl) <= bound) c = ck;
    }
    big = small = c;
    // the alternating sizes around the same C, where they fit too
    if ((bound & 1u) == 0u && (uint32_t)scan_rows(c + kSkewEntries, c - kSkewEntries) <= bound) {
      big = c + kSkewEntries;
      small = c - kSkewEntries;
      scanned = true;
    }
  }
  if (!scanned) scan_rows(big, small);

  // This workgroup's chunk index; each row's first chunk (a prefix in row
  // order, in which a row's chunk count depends on the parity of its first
  // chunk), capped at the bound; the row holding this workgroup's chunk;
  // the merge's copy of the prefix.
  const int32_t b = (int32_t)blockIdx.x;
  const int32_t jc = big == small ? b : (b < cap / 2 ? 2 * b : 2 * (b - cap / 2) + 1);
  const bool writer = blockIdx.x == 0 && threadIdx.x < 64;
  int32_t carry = 0;  // chunks of the rows so far (uncapped: its parity matters)
  bool found = false;
#pragma unroll
  for (int j = 0; j < kPlanRowsPerLane; ++j) {
    if (j >= nj) break;
    const int r = lane + 64 * j;
    const int32_t e0 = lane_below(S0[j]), e1 = lane_below(S1[j]);  // the rows before this lane's
    const int32_t fr = carry + ((carry & 1) ? e1 : e0);
    const int32_t kr = (fr & 1) ? K1[j] : K0[j];  // 0 past the last row (len 0)
    const int32_t f0 = min(fr, cap), f1 = min(fr + kr, cap);
    if (writer && r < tokens) p.ws_prefix[r] = f0;
    const uint64_t hit = __builtin_amdgcn_ballot_w64(r < tokens && f0 <= jc && jc < f1);
    if (hit != 0) {
      const int src = (int)__builtin_ctzll(hit);
      // chunk i of the row starts after e even and i - e odd chunks
      // (unsigned: only meaningful, and below 2^30, on the hit lane)
      const uint32_t fu = (uint32_t)fr, i = (uint32_t)(jc - fr);
      const uint32_t e = ((fu + i + 1u) >> 1) - ((fu + 1u) >> 1);
      const uint32_t start = e * (uint32_t)big + (i - e) * (uint32_t)small;
      const uint32_t size = ((fu + i) & 1u) ? (uint32_t)small : (uint32_t)big;
      rr.t = __builtin_amdgcn_readlane(r, src);
      rr.vb = __builtin_amdgcn_readlane((int32_t)start, src);
      const int32_t csize = __builtin_amdgcn_readlane((int32_t)size, src);
      const int32_t rlen = __builtin_amdgcn_readlane(len[j], src);
      rr.ve = rr.vb + csize < rlen ? rr.vb + csize : (int64_t)rlen;
      rr.beg = __builtin_amdgcn_readlane(rb[j], src);
      rr.lenp = __builtin_amdgcn_readlane(lp[j], src);
      rr.ebeg = __builtin_amdgcn_readlane(eb[j], src);
      rr.chunk = jc;
      rr.single = __builtin_amdgcn_readlane(kr, src) == 1;
      found = true;
    }
    carry += __builtin_amdgcn_readlane((carry & 1) ? S1[j] : S0[j], 63);
  }
  const int32_t total = min(carry, cap);
  if (writer && lane == 0) p.ws_prefix[tokens] = total;
  return found && jc < total;
}

// QK^T partial of latent tile B for this lane's key: the float32 sum over
// the tile's 128 dims of q * code, four bf16 MFMAs of 32 dims each; the
// key's tile scale is applied by the caller.  Lane (n, g) holds dims
// 16g + [0, 16) and 64 + 16g + [0, 16) of the tile, eight per MFMA, in the
// same order for the query (qa[B][0..3]) and the codes.
template <int B>
__device__ __forceinline__ floatx4_t qk_latent_tile(const uint8_t *krec, int g, const u32x4_t (&qa)[4][4]) {
  const u32x4_t c0 = *reinterpret_cast<const u32x4_t *>(krec + 128 * B + 16 * g);
  const u32x4_t c1 = *reinterpret_cast<const u32x4_t *>(krec + 128 * B + 64 + 16 * g);
  floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
  acc = mfma_16x16x32_bf16(as_bf16x8(qa[B][0]), e4m3x8_to_bf16x8(c0.x, c0.y), acc);
  acc = mfma_16x16x32_bf16(as_bf16x8(qa[B][1]), e4m3x8_to_bf16x8(c0.z, c0.w), acc);
  acc = mfma_16x16x32_bf16(as_bf16x8(qa[B][2]), e4m3x8_to_bf16x8(c1.x, c1.y), acc);
  acc = mfma_16x16x32_bf16(as_bf16x8(qa[B][3]), e4m3x8_to_bf16x8(c1.z, c1.w), acc);
  return acc;
}

template <typename IdxT, bool kSplit, bool kLse, bool kExtra>
__global__ __launch_bounds__(kThreads, 2) void sparse_fwd_kernel(FwdKernelArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t s_rec[kTileKeys * kRecordBytes];
  __shared__ __attribute__((aligned(16))) float s_logit[16 * kLogitPitch];
  __shared__ __attribute__((aligned(16))) float s_scale[4 * kTileKeys];
  __shared__ int s_slot[2][kTileKeys];
  __shared__ __attribute__((aligned(16))) uint16_t s_q[16 * kQPitch];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;  // MFMA row/column index of this lane
  const int g = lane >> 4;  // MFMA k-group of this lane

  // Lane roles used before the row is known: MFMA (n, g) for the query,
  // (record, 16-byte sub-chunk) for the gather (see below).
  const int grec = 16 * (tid >> 6) + ((tid >> 4) & 3) + 4 * ((tid >> 2) & 3);
  const int gsub = tid & 3;
  u32x4_t qr[2];     // query, rope part
  u32x4_t qa[4][4];  // query, latent part: [tile][MFMA] bf16 A operands
  // The query is held as bf16 MFMA A operands (row = head n) for the whole
  // row.  Every wave needs all of it, so the workgroup reads it from memory
  // once: each thread loads kQStage 16-byte pieces (stage_query, issued early
  // so that the first gather does not wait for it), they go to LDS with the
  // first tile, and each wave reads its operands from there (finish_query).
  // Heads past the last are zero.  rope part: lane (n, g) k-slots j of step
  // st <-> rope d = 16g + 8st + j; latent tile b, MFMA m: k-slots j <-> dim
  // 128b + 64(m / 2) + 16g + 8(m % 2) + j.  The records' bytes are read
  // with the same mappings.
  u32x4_t qst[kQStage];
  // The loads are unconditional (a piece past the last head reads the last
  // head's first piece and is zeroed when stored), so a later wait on the
  // slot ids counts them and does not wait for them.
  auto stage_query = [&](int64_t t) {
    const uint16_t *qbase = p.q + t * p.q_st;
#pragma unroll
    for (int i = 0; i < kQStage; ++i) {
      const int c = tid + kThreads * i;  // piece c % kQPieces of head c / kQPieces
      const int hh = c / kQPieces;
      const bool in = hh < p.heads;  // else piece 0 of the last head, in bounds
      const int hc = in ? hh : p.heads - 1, pc = in ? c - kQPieces * hh : 0;
      const uint32_t *src = reinterpret_cast<const uint32_t *>(qbase + (int64_t)hc * p.q_sh + 8 * pc);
      qst[i] = u32x4_t{src[0], src[1], src[2], src[3]};
    }
  };
  auto store_query = [&]() {  // before a barrier
#pragma unroll
    for (int i = 0; i < kQStage; ++i) {
      const int c = tid + kThreads * i;
      const int hh = c / kQPieces;
      const uint32_t keep = hh < p.heads ? 0xFFFFFFFFu : 0u;
      const u32x4_t v = qst[i];
      if (hh < 16)
        *reinterpret_cast<u32x4_t *>(s_q + hh * kQPitch + 8 * (c - kQPieces * hh)) =
            u32x4_t{v.x & keep, v.y & keep, v.z & keep, v.w & keep};
    }
  };
  auto finish_query = [&]() {  // after that barrier
    const uint16_t *qrow = s_q + n * kQPitch;
#pragma unroll
    for (int st = 0; st < 2; ++st) qr[st] = *reinterpret_cast<const u32x4_t *>(qrow + kLatent + 16 * g + 8 * st);
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int m = 0; m < 4; ++m)
        qa[b][m] = *reinterpret_cast<const u32x4_t *>(qrow + 128 * b + 64 * (m >> 1) + 16 * g + 8 * (m & 1));
  };

  // ---- this workgroup's entries: a whole row, or a chunk of one
  const IdxT *indices = static_cast<const IdxT *>(p.indices);
  const IdxT *eindices = static_cast<const IdxT *>(p.eindices);
  RowRange rr;
  // A top-k selection gives every row the same length L, laid out back to
  // back (nnz = T * L), so row t most likely starts at entry t * L.  The
  // first entries are requested at that guess, before the query and while
  // indptr is still on its way, and used if indptr agrees; so the first
  // gather waits for one round trip less.
  IdxT guess_id0 = 0, guess_t0 = 0, guess_t1 = 0;
  int64_t guess_beg = -1;
  if (kSplit) {
    if (!split_plan<IdxT, kExtra>(p, rr)) return;  // whole workgroup
  } else {
    const IdxT *indptr = static_cast<const IdxT *>(p.indptr);
    rr.t = blockIdx.x;
    const IdxT x0 = indptr[rr.t], x1 = indptr[rr.t + 1];
    if (!kExtra && p.guess_len > 0) {
      guess_beg = rr.t * p.guess_len;
      auto at = [&](int64_t v) { return indices[guess_beg + v < p.nnz ? guess_beg + v : 0]; };
      guess_id0 = at(grec);
      guess_t0 = at(lane);
      guess_t1 = at(kTileKeys + lane);
    }
    // the query after the ids: loads complete in order, so the first gather
    // waits for indptr and its slot id, not for the query
    stage_query(rr.t);
    __builtin_amdgcn_sched_barrier(0);  // all of the above in flight before indptr is used
    clamp_range((int64_t)x0, (int64_t)x1, p.nnz, rr.beg, rr.lenp);
    int64_t lene = 0;
    rr.ebeg = 0;
    if (kExtra) {
      const IdxT *eindptr = static_cast<const IdxT *>(p.eindptr);
      clamp_range((int64_t)eindptr[rr.t], (int64_t)eindptr[rr.t + 1], p.ennz, rr.ebeg, lene);
    }
    rr.vb = 0;
    rr.ve = rr.lenp + lene;
  }
  const int64_t t = rr.t;
  const int ntiles = (int)((rr.ve - rr.vb + kTileKeys - 1) / kTileKeys);

  // Raw id of entry j of tile `tile`.  The load is unconditional (an entry
  // past the end reads element 0 of the primary list instead, which exists:
  // with no indices the array is a placeholder that points at indptr) and its
  // value is not looked at here, so it stays in flight until slot_of turns it
  // into a slot, an iteration later for the index prefetch.
  auto fetch_entry = [&](int tile, int j) -> IdxT {
    const int64_t v = rr.vb + (int64_t)tile * kTileKeys + j;
    if (!kExtra) return indices[v < rr.ve ? rr.beg + v : 0];
    const IdxT *src = v < rr.lenp ? indices + (rr.beg + v) : eindices + (rr.ebeg + v - rr.lenp);
    return *(v < rr.ve ? src : indices);
  };
  // What entry j of tile `tile` names: a primary slot s as s, an extra-pool
  // slot s as -2 - s, and -1 when it is past the end, masked, or outside its
  // pool.  (Pools hold fewer than 2^31 - 2 records.)
  auto slot_of = [&](IdxT raw, int tile, int j) -> int {
    const int64_t x = (int64_t)raw;
    const int64_t v = rr.vb + (int64_t)tile * kTileKeys + j;
    const bool in_range = v < rr.ve;
    if (!kExtra) return (in_range && x >= 0 && x < p.num_records) ? (int)x : -1;
    const bool extra = v >= rr.lenp;
    const bool ok = in_range && x >= 0 && x < (extra ? p.enum_records : p.num_records);
    return ok ? (extra ? -2 - (int)x : (int)x) : -1;
  };

  // Gather mapping: 4 threads per record; thread (rec, sub) moves the 16-byte
  // chunks sub, sub + 4, ..., so one slot lookup serves all its loads and
  // every load / store sits at a constant offset from one address.  A
  // masked or past-the-end key is not loaded: its LDS row keeps whatever
  // finite chunks the registers held (zero at first), which is harmless
  // because its logit is -inf and its softmax weight exactly 0.
  // Records r, r+4, r+8, r+12 share a 16-lane group: at a 164-dword pitch
  // they start 16 banks apart, so each 16-lane LDS store pass is conflict-free.
  u32x4_t pf[kChunksPerThread];
#pragma unroll
  for (int i = 0; i < kChunksPerThread; ++i) pf[i] = u32x4_t{0u, 0u, 0u, 0u};
  auto issue_gather_slot = [&](int slot) {
    if (kExtra ? slot != -1 : slot >= 0) {
      const uint8_t *src = (slot >= 0 ? p.rec + (int64_t)slot * kRecordBytes
                                      : p.erec + (int64_t)(-2 - slot) * kRecordBytes) + 16 * gsub;
#pragma unroll
      for (int i = 0; i < kChunksPerThread - 1; ++i) pf[i] = *reinterpret_cast<const u32x4_t *>(src + 64 * i);
      if (gsub == 0) pf[kChunksPerThread - 1] = *reinterpret_cast<const u32x4_t *>(src + 64 * (kChunksPerThread - 1));
    }
  };
  auto issue_gather = [&](int buf) { issue_gather_slot(s_slot[buf][grec]); };
  auto store_gather = [&]() {
    uint8_t *dst = s_rec + grec * kRecordBytes + 16 * gsub;
#pragma unroll
    for (int i = 0; i < kChunksPerThread - 1; ++i) *reinterpret_cast<u32x4_t *>(dst + 64 * i) = pf[i];
    if (gsub == 0) *reinterpret_cast<u32x4_t *>(dst + 64 * (kChunksPerThread - 1)) = pf[kChunksPerThread - 1];
  };

  // ---- start the first tile early.  This thread's slot of tile 0 and the
  // slots of tiles 0 and 1 (for the masks) are taken from the guess or
  // requested now, ahead of the query; tile 0's gather is issued as soon as
  // its slot is in.  (The gather is conditional, so anything loaded after it
  // would wait for it.)
  const bool guessed = guess_beg == rr.beg && rr.vb == 0 && rr.ve == p.guess_len;
  IdxT my_id0, slot_t0, slot_t1;
  if (guessed) {
    my_id0 = guess_id0;
    slot_t0 = guess_t0;
    slot_t1 = guess_t1;
  } else {
    my_id0 = fetch_entry(0, grec);
    slot_t0 = fetch_entry(0, lane);
    slot_t1 = fetch_entry(1, lane);
  }
  if (kSplit) {
    stage_query(t);  // after the slot ids, for the same reason
    __builtin_amdgcn_sched_barrier(0);
  }

  issue_gather_slot(slot_of(my_id0, 0, grec));  // tile 0

  float m_run = -INFINITY;  // running max of head n's logits (exp2 domain)
  float l_run = 0.f;        // this lane's part of head n's running sum
  floatx4_t oacc[8];        // O^T[128*wave + 16*mt + 4*g + j][head n]
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) oacc[mt] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  auto compute_tile = [&](int buf) {
    // ---- QK^T for keys 16*wave + n
    const uint8_t *krec = s_rec + (wave * 16 + n) * kRecordBytes;
    const u32x4_t scv = *reinterpret_cast<const u32x4_t *>(krec + kScaleOffset);
    floatx4_t sacc = qk_latent_tile<0>(krec, g, qa) * as_float(scv[0]);
    sacc += qk_latent_tile<1>(krec, g, qa) * as_float(scv[1]);
    sacc += qk_latent_tile<2>(krec, g, qa) * as_float(scv[2]);
    sacc += qk_latent_tile<3>(krec, g, qa) * as_float(scv[3]);
    {
      const u32x4_t r0 = *reinterpret_cast<const u32x4_t *>(krec + kRopeOffset + 32 * g);
      const u32x4_t r1 = *reinterpret_cast<const u32x4_t *>(krec + kRopeOffset + 32 * g + 16);
      floatx4_t racc = {0.f, 0.f, 0.f, 0.f};
      racc = mfma_16x16x32_bf16(as_bf16x8(qr[0]), as_bf16x8(r0), racc);
      racc = mfma_16x16x32_bf16(as_bf16x8(qr[1]), as_bf16x8(r1), racc);
      sacc += racc;
    }
    const bool valid = kExtra ? s_slot[buf][wave * 16 + n] != -1 : s_slot[buf][wave * 16 + n] >= 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      s_logit[(4 * g + j) * kLogitPitch + wave * 16 + n] = valid ? sacc[j] * p.scale_log2 : -INFINITY;
    s_scale[g * kTileKeys + wave * 16 + n] = as_float(scv[g]);
    __syncthreads();

    // ---- online softmax of head n over the tile; lane (n, g) holds keys
    // 8g + [0, 8) and 32 + 8g + [0, 8) (the PV k-slots of this lane).
    float sv[16];
    {
      const float *xr = s_logit + n * kLogitPitch;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const floatx4_t a = *reinterpret_cast<const floatx4_t *>(xr + 32 * ks + 8 * g);
        const floatx4_t b = *reinterpret_cast<const floatx4_t *>(xr + 32 * ks + 8 * g + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sv[8 * ks + j] = a[j];
          sv[8 * ks + 4 + j] = b[j];
        }
      }
    }
    float mt = sv[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mt = fmaxf(mt, sv[i]);
    mt = fmaxf(mt, xor_shuffle(mt, 16));
    mt = fmaxf(mt, xor_shuffle(mt, 32));
    // Lazy rescale: the reference m_run only moves when the tile max passes
    // it by more than kLazyRescale (weights stay <= 2^kLazyRescale), so O
    // and the sum are rescaled rarely; any reference gives the same result.
    if (__builtin_amdgcn_ballot_w64(mt > m_run + kLazyRescale) != 0) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int m = 0; m < 8; ++m) oacc[m] *= alpha;
      m_run = m_new;
    }
    const float m_ref = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sv[i] = fast_exp2(sv[i] - m_ref);
      l_run += sv[i];
    }

    // ---- P^T operands (B: column = head n, k-slot j = key 32ks + 8g + j),
    // each weight times its key's scale for latent tile `wave`.
    u32x4_t pb[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const float *scp = s_scale + wave * kTileKeys + 32 * ks + 8 * g;
      const floatx4_t s0 = *reinterpret_cast<const floatx4_t *>(scp);
      const floatx4_t s1 = *reinterpret_cast<const floatx4_t *>(scp + 4);
      pb[ks].x = pack_bf16x2(sv[8 * ks + 0] * s0[0], sv[8 * ks + 1] * s0[1]);
      pb[ks].y = pack_bf16x2(sv[8 * ks + 2] * s0[2], sv[8 * ks + 3] * s0[3]);
      pb[ks].z = pack_bf16x2(sv[8 * ks + 4] * s1[0], sv[8 * ks + 5] * s1[1]);
      pb[ks].w = pack_bf16x2(sv[8 * ks + 6] * s1[2], sv[8 * ks + 7] * s1[3]);
    }

    // ---- PV.  In each 16-lane group g, lane n names record 32ks + 8g + n/2
    // at column 128*wave + 16*mt + 8*(n&1); the transposing read hands lane
    // n the bytes of column 128*wave + 16*mt + n of records 32ks + 8g + j,
    // j = 0..7: the A operand row n, k-slots j.
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint8_t *vbase = s_rec + (32 * ks + 8 * g + (n >> 1)) * kRecordBytes + 128 * wave + 8 * (n & 1);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const intx2_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_intx2_t *)(vbase + 16 * m));
        oacc[m] = mfma_16x16x32_bf16(e4m3x8_to_bf16x8((uint32_t)v.x, (uint32_t)v.y), as_bf16x8(pb[ks]), oacc[m]);
      }
    }
  };

  if (ntiles > 0) {
    IdxT next_slot = fetch_entry(2, lane);
    if (tid < kTileKeys) {
      s_slot[0][tid] = slot_of(slot_t0, 0, tid);
      s_slot[1][tid] = slot_of(slot_t1, 1, tid);
    }
    store_gather();  // tile 0
    store_query();
    __syncthreads();
    finish_query();
    if (ntiles > 1) issue_gather(1);
    for (int k = 0; k < ntiles; ++k) {
      const int buf = k & 1;
      compute_tile(buf);
      __syncthreads();
      if (k + 1 < ntiles) {
        store_gather();  // tile k + 1
        if (tid < kTileKeys) s_slot[buf][tid] = slot_of(next_slot, k + 2, tid);  // tile k + 2
        next_slot = fetch_entry(k + 3, lane);
        __syncthreads();
        if (k + 2 < ntiles) issue_gather(buf);
      }
    }
  }

  // ---- epilogue: head n's total sum over the four k-groups
  float l_tot = l_run + xor_shuffle(l_run, 16);
  l_tot += xor_shuffle(l_tot, 32);
  float o_scale = 1.f;  // applied to O with 1 / l
  if (!kSplit && p.sink) {
    // the sink: one more logit with a zero value (the split pass adds it in the merge)
    const float s2 = p.sink[n < p.heads ? n : 0] * kLog2e;
    if (m_run == -INFINITY) {
      m_run = s2;
      l_tot = s2 == -INFINITY ? 0.f : 1.f;
      o_scale = 0.f;
    } else if (s2 > m_run) {
      o_scale = fast_exp2(m_run - s2);
      l_tot = l_tot * o_scale + 1.f;
      m_run = s2;
    } else {
      l_tot += fast_exp2(s2 - m_run);
    }
  }
  const float inv = l_tot > 0.f ? o_scale / l_tot : 0.f;
  const bool empty = m_run == -INFINITY;
  if (n < p.heads) {
    if (!kSplit) {
      uint16_t *orow = p.out + t * p.o_st + (int64_t)n * p.o_sh + 128 * wave + 4 * g;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        uint32_t *dst = reinterpret_cast<uint32_t *>(orow + 16 * m);
        dst[0] = pack_bf16x2(oacc[m][0] * inv, oacc[m][1] * inv);
        dst[1] = pack_bf16x2(oacc[m][2] * inv, oacc[m][3] * inv);
      }
      if (kLse && wave == 0 && g == 0)
        p.lse[t * p.heads + n] = empty ? -INFINITY : (m_run + fast_log2(l_tot)) * kLn2;
    } else if (p.direct_single && rr.single) {
      // The row's only chunk: out and lse as the merge would make them of this
      // one partial (bit for bit: a single partial o merges to o * 1, its LSE
      // to lse + log2 1), so the merge skips the row.
      uint16_t *orow = p.out + t * p.o_st + (int64_t)n * p.o_sh + 128 * wave + 4 * g;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        uint32_t *dst = reinterpret_cast<uint32_t *>(orow + 16 * m);
        dst[0] = pack_bf16x2(oacc[m][0] * inv, oacc[m][1] * inv);
        dst[1] = pack_bf16x2(oacc[m][2] * inv, oacc[m][3] * inv);
      }
      if (p.lse && wave == 0 && g == 0)
        p.lse[t * p.heads + n] = empty ? -INFINITY : (m_run + fast_log2(l_tot)) * kLn2;
    } else {
      const int64_t row = rr.chunk * p.heads + n;  // chunk index * H + head
      float *wo = p.ws_out + row * kLatent + 128 * wave + 4 * g;
#pragma unroll
      for (int m = 0; m < 8; ++m) *reinterpret_cast<floatx4_t *>(wo + 16 * m) = oacc[m] * inv;
      if (wave == 0 && g == 0) p.ws_lse[row] = empty ? -INFINITY : m_run + fast_log2(l_tot);
    }
  }
}

// Combine a row's chunk partials: lse = log2 (sum_s 2^lse_s [+ 2^sink]),
// out = sum_s 2^(lse_s - lse) o_s (an empty partial, lse_s = -inf, weighs 0;
// the sink, when given, is one more term with a zero value; nothing at all
// -> out 0, lse -inf).  A workgroup takes kLanes chunk lanes x (256 / kLanes)
// column quads of one (row, head): 8 lanes cover a 128-column quarter of the
// head, 4 lanes half of it, 2 lanes all of it, so rows cut into few chunks
// use few, wide workgroups.  Each thread loads the LSEs and its column quad
// of its chunks (s = lane, lane + kLanes, ...) at once, accumulates them
// online (running max, rescaled sum and quad), and one LDS exchange combines
// the chunk lanes.
constexpr int kMergeThreads = 256;
constexpr int kMergeBatch = 8;  // chunks per thread with their loads in flight together

template <bool kLse, int kLanes>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const float *ws_out, const float *ws_lse,
                                                              const int32_t *prefix, int32_t heads, uint16_t *out,
                                                              int64_t o_st, int64_t o_sh, float *lse,
                                                              const float *sink, int32_t direct_single) {
  constexpr int kQuads = kMergeThreads / kLanes;
  constexpr int kParts = kLatent / (4 * kQuads);
  __shared__ MergeAcc s_acc[kLanes][kQuads];
  const int tid = threadIdx.x;
  const int part = (int)(blockIdx.x % kParts);
  const int64_t th = blockIdx.x / kParts;  // t * heads + h
  const int64_t t = th / heads;
  const int h = (int)(th - t * heads);
  const int64_t c0 = prefix[t];
  const int nc = prefix[t + 1] - (int)c0;
  if (direct_single && nc == 1) return;  // the partial pass wrote this row (whole workgroup)
  const float *lp = ws_lse + c0 * heads + h;  // chunk s at lp[s * heads]
  const int cl = tid / kQuads;  // chunk lane
  const int cq = tid % kQuads;  // column quad
  const int col = part * 4 * kQuads + 4 * cq;
  const float *op = ws_out + (c0 * heads + h) * kLatent + col;  // chunk s at op[s * heads * 512]

  MergeAcc acc = merge_acc_empty();
  for (int base = cl; base < nc; base += kLanes * kMergeBatch) {
    float ls[kMergeBatch];
    floatx4_t os[kMergeBatch];
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const int s = base + kLanes * k;
      const int sc = s < nc ? s : base;  // in range: base < nc
      ls[k] = lp[(int64_t)sc * heads];
      os[k] = *reinterpret_cast<const floatx4_t *>(op + (int64_t)sc * heads * kLatent);
      if (s >= nc) ls[k] = -INFINITY;
    }
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) merge_add(acc, ls[k], os[k]);
  }
  s_acc[cl][cq] = acc;
  __syncthreads();
  if (cl == 0) {
    // the sink: one more term with a zero value
    if (sink) merge_add(acc, sink[h] * kLog2e, floatx4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int k = 1; k < kLanes; ++k) merge_combine(acc, s_acc[k][cq]);
    const float inv = acc.l > 0.f ? 1.f / acc.l : 0.f;
    uint32_t *dst = reinterpret_cast<uint32_t *>(out + t * o_st + (int64_t)h * o_sh + col);
    dst[0] = pack_bf16x2(acc.o[0] * inv, acc.o[1] * inv);
    dst[1] = pack_bf16x2(acc.o[2] * inv, acc.o[3] * inv);
    if (kLse && part == 0 && cq == 0)
      lse[t * heads + h] = acc.m == -INFINITY ? -INFINITY : (acc.m + fast_log2(acc.l)) * kLn2;
  }
}

template <int kLanes>
void launch_merge(const FwdArgs &a, hipStream_t stream) {
  const dim3 mgrid((unsigned)((int64_t)a.num_tokens * a.num_heads * (kLanes / 2)));
  if (a.lse)
    merge_kernel<true, kLanes><<<mgrid, kMergeThreads, 0, stream>>>(a.ws_out, a.ws_lse, a.ws_prefix, a.num_heads, a.out,
                                                                    a.out_stride_token, a.out_stride_head, a.lse, a.sink,
                                                                    a.vp_w == nullptr && a.sink == nullptr);
  else
    merge_kernel<false, kLanes><<<mgrid, kMergeThreads, 0, stream>>>(a.ws_out, a.ws_lse, a.ws_prefix, a.num_heads, a.out,
                                                                     a.out_stride_token, a.out_stride_head, nullptr, a.sink,
                                                                     a.vp_w == nullptr && a.sink == nullptr);
}

template <typename IdxT, bool kExtra>
hipError_t launch_typed(const FwdArgs &a, hipStream_t stream) {
  FwdKernelArgs k;
  k.q = a.q;
  k.q_st = a.q_stride_token;
  k.q_sh = a.q_stride_head;
  k.rec = a.records;
  k.num_records = a.num_records;
  k.indptr = a.indptr;
  k.indices = a.indices;
  k.nnz = a.num_indices;
  k.scale_log2 = a.scale_log2;
  k.heads = a.num_heads;
  k.out = a.out;
  k.o_st = a.out_stride_token;
  k.o_sh = a.out_stride_head;
  k.lse = a.lse;
  k.ws_out = a.ws_out;
  k.ws_lse = a.ws_lse;
  k.ws_prefix = a.ws_prefix;
  k.tokens = a.num_tokens;
  k.forced_chunk = a.chunk_forced;
  k.bound = a.chunk_bound;
  k.erec = a.extra_records;
  k.enum_records = a.extra_num_records;
  k.eindptr = a.extra_indptr;
  k.eindices = a.extra_indices;
  k.ennz = a.extra_num_indices;
  k.sink = a.sink;
  k.guess_len = a.row_len_guess;
  // a row of one chunk is written by the partial pass unless a sink joins it
  // in the merge or the fused projection merges it
  k.direct_single = a.vp_w == nullptr && a.sink == nullptr;
  const dim3 block(kThreads);
  const bool lse = a.lse != nullptr;
  if (a.chunk_bound <= 0) {
    const dim3 grid((unsigned)a.num_tokens);
    if (lse)
      sparse_fwd_kernel<IdxT, false, true, kExtra><<<grid, block, 0, stream>>>(k);
    else
      sparse_fwd_kernel<IdxT, false, false, kExtra><<<grid, block, 0, stream>>>(k);
    return hipGetLastError();
  }
  hipError_t e;
  sparse_fwd_kernel<IdxT, true, false, kExtra><<<dim3((unsigned)a.chunk_bound), block, 0, stream>>>(k);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // chunk lanes for the average chunks per row (one batch of loads each when they fit)
  const int64_t per_row = (a.chunk_bound + a.num_tokens - 1) / a.num_tokens;
  const int lanes = per_row <= 2 * kMergeBatch ? 2 : (per_row <= 4 * kMergeBatch ? 4 : 8);
  if (a.vp_w) {
    MergeVUpProjArgs m;
    m.ws_out = a.ws_out;
    m.ws_lse = a.ws_lse;
    m.ws_prefix = a.ws_prefix;
    m.num_tokens = a.num_tokens;
    m.num_heads = a.num_heads;
    m.out = a.out;
    m.out_st = a.out_stride_token;
    m.out_sh = a.out_stride_head;
    m.lse = a.lse;
    m.w_prepared = a.vp_w;
    m.gate = a.vp_gate;
    m.gate_st = a.vp_gate_st;
    m.v_out = a.vp_out;
    m.v_st = a.vp_st;
    m.v_sh = a.vp_sh;
    return launch_merge_v_up_proj(m, lanes, stream);
  }
  if (lanes == 2)
    launch_merge<2>(a, stream);
  else if (lanes == 4)
    launch_merge<4>(a, stream);
  else
    launch_merge<8>(a, stream);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_fwd(const FwdArgs &a, hipStream_t stream) {
  const bool extra = a.extra_indptr != nullptr;
  if (a.index_i64) return extra ? launch_typed<int64_t, true>(a, stream) : launch_typed<int64_t, false>(a, stream);
  return extra ? launch_typed<int32_t, true>(a, stream) : launch_typed<int32_t, false>(a, stream);
}

}  // namespace mla
