// C ABI of the sparse MLA library: argument validation (host metadata only),
// split-KV planning, the library-owned workspace, and kernel launches.
//
// The validation restates the limits flydsl_sparse_mla_fp8ds_supported
// states on the flydsl_sparse_mla page (head count, 576-wide bf16 rows with
// even strides and a 4-byte aligned base, 16-byte aligned 656-byte records
// at their natural pitch, int32/int64 CSR arrays, fewer than 2^29 indices),
// in C terms: every rejection happens before anything is queued.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/mla.h"
#include "mla_internal.h"

namespace {

thread_local char g_error[512] = "";

mla_status_t fail(mla_status_t st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof(g_error), fmt, ap);
  va_end(ap);
  return st;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Whether a [rows, heads, width] view with these (non-negative) element
// strides spans at most 2^62 elements.  No buffer is that large, and the
// kernels' 64-bit address arithmetic must not wrap; a view past it is an
// argument error.
bool view_fits(int64_t rows, int64_t stride_row, int64_t heads, int64_t stride_head, int64_t width) {
  if (rows <= 0 || heads <= 0) return true;
  const __int128 last = (__int128)(rows - 1) * stride_row + (__int128)(heads - 1) * stride_head + width;
  return last <= ((__int128)1 << 62);
}

// Largest pool the insert / epilogue / gather kernels address (record
// offsets slot * 656 stay far inside 64 bits).
constexpr int64_t kMaxPoolRecords = (int64_t)1 << 40;

// Compute units of the current device (cached per device).
int device_cus(int device) {
  static std::mutex mu;
  static std::vector<int> cache;
  std::lock_guard<std::mutex> lock(mu);
  if (device < 0) return 0;
  if ((size_t)device >= cache.size()) cache.resize(device + 1, 0);
  if (cache[device] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) return 0;
    cache[device] = cus;
  }
  return cache[device];
}

// The library-owned split workspace of one device.  A buffer that is
// replaced by a larger one is retired, not freed: work queued earlier (or
// a graph captured earlier) may still name it, so it stays allocated until
// the process ends.  Growth at least doubles, so the retired buffers
// together stay smaller than the current one.
struct Workspace {
  void *ptr = nullptr;
  size_t bytes = 0;
  std::vector<void *> retired;
};
std::mutex g_ws_mu;
std::vector<Workspace> g_ws;

// Grow device `device`'s library-owned workspace to >= bytes; returns it.
mla_status_t workspace_get(int device, size_t bytes, void **out) {
  std::lock_guard<std::mutex> lock(g_ws_mu);
  if ((size_t)device >= g_ws.size()) g_ws.resize(device + 1);
  Workspace &w = g_ws[device];
  if (w.bytes < bytes) {
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) return fail(MLA_ERR_HIP, "hipGetDevice failed");
    if (prev != device && hipSetDevice(device) != hipSuccess) return fail(MLA_ERR_HIP, "hipSetDevice(%d) failed", device);
    const size_t grown = bytes > 2 * w.bytes ? bytes : 2 * w.bytes;
    const size_t want = (grown + ((size_t)1 << 20) - 1) & ~(((size_t)1 << 20) - 1);
    void *fresh = nullptr;
    hipError_t e = hipMalloc(&fresh, want);
    if (prev != device) (void)hipSetDevice(prev);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(MLA_ERR_OUT_OF_MEMORY, "workspace of %zu bytes could not be allocated on device %d: %s", want,
                  device, hipGetErrorString(e));
    }
    if (w.ptr) w.retired.push_back(w.ptr);
    w.ptr = fresh;
    w.bytes = want;
  }
  *out = w.ptr;
  return MLA_OK;
}

constexpr uint32_t kKnownFlags =
    MLA_FLAG_HAS_INVALID | MLA_FLAG_RETURN_LSE | MLA_FLAG_INDEX_I64 | MLA_FLAG_CHUNK_MASK;

// Smallest chunk the plan kernel picks on its own: eight 64-key tiles (the
// device side uses the same value).
constexpr int64_t kMinChunkEntries = 512;

// Split-KV plan from host values only (never index values): 0 = one
// workgroup per row; otherwise the number of workgroups of the partial pass,
// an upper bound on the chunks.  Split when the rows alone cannot give two
// workgroups per compute unit and the average row is longer than a minimum
// chunk, unless more than CU-many rows look equal (below); the plan kernel
// then sizes the chunks on the device so they fit those 2 x CU workgroups
// in one round.  A forced chunk size (flags) gives
// the bound ceil(nnz / chunk) + T.
int64_t plan_split(int64_t tokens, int64_t nnz, int32_t cus, uint32_t flags, int32_t *forced_chunk) {
  const uint32_t forced = (flags & MLA_FLAG_CHUNK_MASK) >> 16;
  *forced_chunk = 0;
  if (tokens <= 0) return 0;
  if (forced) {
    *forced_chunk = (int32_t)(forced * 64);
    return mla::forced_chunk_bound(tokens, nnz, *forced_chunk);
  }
  if (cus <= 0) return 0;
  const int64_t target = 2 * (int64_t)cus;
  if (tokens >= target || tokens > mla::kMaxSplitRows) return 0;
  if ((nnz + tokens - 1) / tokens <= kMinChunkEntries) return 0;
  // Rows of equal length (an entry count that T divides, as a top-k
  // selection gives) cannot be cut into two chunks each once 2T exceeds the
  // workgroups: the split pass would compute what one workgroup per row
  // does, plus a merge.
  if (2 * tokens > target && nnz % tokens == 0) return 0;
  return target;
}

// ---- Fixed split workspace of mla_sparse_fwd_noalloc: a device array of
// MLA_NOALLOC_SCRATCH_BYTES per GPU, allocated with the code object and held
// until the process ends.  Host code never names the array in a kernel
// argument or a copy (the name is only a host-side stand-in): its device
// address is looked up once per device, with that device current, and kept.
constexpr size_t kScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
std::vector<void *> g_scratch_ptr;  // per device; nullptr until looked up

// Device address of `device`'s scratch array (`device` must be current).
mla_status_t scratch_address(int device, void **out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((size_t)device >= g_scratch_ptr.size()) g_scratch_ptr.resize(device + 1, nullptr);
  if (!g_scratch_ptr[device]) {
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return fail(MLA_ERR_HIP, "mla_sparse_fwd_noalloc: no address for the scratch array on device %d: %s", device,
                  hipGetErrorString(e));
    }
    g_scratch_ptr[device] = ptr;
  }
  *out = g_scratch_ptr[device];
  return MLA_OK;
}

// The second segment and the sink of mla_sparse_fwd_ex (all absent for mla_sparse_fwd).
struct FwdExtra {
  bool scratch = false;  // split workspace from the static scratch array (mla_sparse_fwd_noalloc)
  const float *sink = nullptr;
  const void *records = nullptr;
  int64_t num_records = 0, record_stride = MLA_RECORD_BYTES;
  const void *indptr = nullptr, *indices = nullptr;
  int64_t num_indices = 0;
  // the gated up-projection on prepared weights (mla_sparse_fwd_v_up_proj):
  // fused into the merge of a split call, launched after the forward otherwise
  const void *vp_w = nullptr;
  const void *vp_gate = nullptr;
  int64_t vp_gate_st = 0;
  void *vp_out = nullptr;
  int64_t vp_st = 0, vp_sh = 0;
};

mla_status_t sparse_fwd_impl(const void *q, int64_t num_tokens, int32_t num_heads, int64_t q_stride_token,
                             int64_t q_stride_head, const void *kv_records, int64_t num_records, int64_t record_stride,
                             const void *kv_indptr, const void *kv_indices, int64_t num_indices, float softmax_scale,
                             uint32_t flags, void *out, int64_t out_stride_token, int64_t out_stride_head, float *lse,
                             void *workspace, size_t workspace_bytes, void *stream, const FwdExtra &x) {
  if (flags & ~kKnownFlags) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_sparse_fwd: unknown flag bits 0x%x", flags & ~kKnownFlags);
  if (num_tokens < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_sparse_fwd: num_tokens %lld < 0", (long long)num_tokens);
  if (num_tokens > INT32_MAX - 1) return fail(MLA_ERR_UNSUPPORTED, "mla_sparse_fwd: num_tokens %lld too large", (long long)num_tokens);
  if (num_heads < 1 || num_heads > MLA_MAX_HEADS)
    return fail(MLA_ERR_UNSUPPORTED, "mla_sparse_fwd: num_heads %d outside 1..%d", num_heads, MLA_MAX_HEADS);
  if (q_stride_token < 0 || q_stride_head < 0 || out_stride_token < 0 || out_stride_head < 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_sparse_fwd: negative stride");
  if ((q_stride_token | q_stride_head) & 1)
    return fail(MLA_ERR_UNSUPPORTED, "mla_sparse_fwd: q strides must be even (got %lld, %lld)", (long long)q_stride_token,
                (long long)q_stride_head);
  if ((out_stride_token | out_stride_head) & 1)
    return fail(MLA_ERR_UNSUPPORTED, "mla_sparse_fwd: out strides must be even (got %lld, %lld)",
                (long long)out_stride_token, (long long)out_stride_head);
  if (!view_fits(num_tokens, q_stride_token, num_heads, q_stride_head, MLA_QK_DIM) ||
      !view_fits(num_tokens, out_stride_token, num_heads, out_stride_head, MLA_KV_LORA_RANK))
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_sparse_fwd: q or out view spans more than 2^62 elements");
  if (record_stride != MLA_RECORD_BYTES)
    return fail(MLA_ERR_UNSUPPORTED, "mla_sparse_fwd: record pitch %lld, only %d (unpadded) is served", (long long)record_stride,
                MLA_RECORD_BYTES);
  if (num_records < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_sparse_fwd: num_records %lld < 0", (long long)num_records);
  if (num_records > INT32_MAX) return fail(MLA_ERR_UNSUPPORTED, "mla_sparse_fwd: num_records %lld >= 2^31", (long long)num_records);
  if (num_indices < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_sparse_fwd: num_indices %lld < 0", (long long)num_indices);
  if (num_indices >= MLA_MAX_INDICES)
    return fail(MLA_ERR_UNSUPPORTED, "mla_sparse_fwd: num_indices %lld >= 2^29", (long long)num_indices);
  const bool i64 = (flags & MLA_FLAG_INDEX_I64) != 0;
  const bool want_lse = (flags & MLA_FLAG_RETURN_LSE) != 0;
  const uintptr_t idx_align = i64 ? 8 : 4;
  const bool has_extra = x.indptr != nullptr;
  if (has_extra) {
    if (x.record_stride != MLA_RECORD_BYTES)
      return fail(MLA_ERR_UNSUPPORTED, "mla_sparse_fwd: extra record pitch %lld, only %d is served",
                  (long long)x.record_stride, MLA_RECORD_BYTES);
    if (x.num_records < 0 || x.num_indices < 0)
      return fail(MLA_ERR_INVALID_ARGUMENT, "mla_sparse_fwd: negative extra size");
    if (x.num_records > INT32_MAX - 2)
      return fail(MLA_ERR_UNSUPPORTED, "mla_sparse_fwd: extra_num_records %lld >= 2^31 - 2", (long long)x.num_records);
    if (x.num_indices >= MLA_MAX_INDICES - num_indices)  // num_indices < 2^29 here
      return fail(MLA_ERR_UNSUPPORTED, "mla_sparse_fwd: num_indices + extra_num_indices >= 2^29");
    if (!aligned(x.records, 16)) return fail(MLA_ERR_UNSUPPORTED, "mla_sparse_fwd: extra records not 16-byte aligned");
    if (!aligned(x.indptr, idx_align) || !aligned(x.indices, idx_align))
      return fail(MLA_ERR_INVALID_ARGUMENT, "mla_sparse_fwd: extra index arrays not aligned to their element size");
    if (x.num_indices > 0 && !x.indices) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_sparse_fwd: NULL extra_indices");
    if (x.num_records > 0 && !x.records) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_sparse_fwd: NULL extra_records");
  }
  if (x.sink && !aligned(x.sink, 4)) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_sparse_fwd: attn_sink not 4-byte aligned");
  const int64_t total_indices = num_indices + (has_extra ? x.num_indices : 0);
  if (!aligned(q, 4)) return fail(MLA_ERR_UNSUPPORTED, "mla_sparse_fwd: q base not 4-byte aligned");
  if (!aligned(out, 4)) return fail(MLA_ERR_UNSUPPORTED, "mla_sparse_fwd: out base not 4-byte aligned");
  if (!aligned(kv_records, 16)) return fail(MLA_ERR_UNSUPPORTED, "mla_sparse_fwd: kv_records base not 16-byte aligned");
  if (!aligned(kv_indptr, idx_align) || !aligned(kv_indices, idx_align))
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_sparse_fwd: index arrays not aligned to their element size");
  if (want_lse && !aligned(lse, 4)) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_sparse_fwd: lse not 4-byte aligned");
  if ((flags & MLA_FLAG_CHUNK_MASK) && num_tokens > mla::kMaxSplitRows)
    return fail(MLA_ERR_UNSUPPORTED, "mla_sparse_fwd: forced split-KV serves at most %lld rows",
                (long long)mla::kMaxSplitRows);
  if (num_tokens == 0) return MLA_OK;
  if (!q || !out || !kv_indptr) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_sparse_fwd: NULL q, out or kv_indptr");
  if (want_lse && !lse) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_sparse_fwd: MLA_FLAG_RETURN_LSE with lse == NULL");
  if (num_indices > 0 && !kv_indices) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_sparse_fwd: NULL kv_indices");
  if (num_records > 0 && !kv_records) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_sparse_fwd: NULL kv_records");

  int device = -1;
  if (hipGetDevice(&device) != hipSuccess) return fail(MLA_ERR_HIP, "mla_sparse_fwd: hipGetDevice failed");
  const bool forced = (flags & MLA_FLAG_CHUNK_MASK) != 0;
  const int cus = forced ? 0 : device_cus(device);
  if (!forced && cus <= 0) return fail(MLA_ERR_HIP, "mla_sparse_fwd: cannot query device %d", device);
  int32_t forced_chunk = 0;
  const int64_t bound = plan_split(num_tokens, total_indices, cus, flags, &forced_chunk);

  if (bound > INT32_MAX)
    return fail(MLA_ERR_UNSUPPORTED, "mla_sparse_fwd: %lld chunks exceed the grid", (long long)bound);

  mla::FwdArgs a;
  a.q = static_cast<const uint16_t *>(q);
  a.q_stride_token = q_stride_token;
  a.q_stride_head = q_stride_head;
  a.records = static_cast<const uint8_t *>(kv_records);
  a.num_records = num_records;
  a.indptr = kv_indptr;
  a.indices = num_indices > 0 ? kv_indices : kv_indptr;  // element 0 may be read, never used
  a.num_indices = num_indices;
  a.index_i64 = i64;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.num_tokens = (int32_t)num_tokens;
  a.num_heads = num_heads;
  a.out = static_cast<uint16_t *>(out);
  a.out_stride_token = out_stride_token;
  a.out_stride_head = out_stride_head;
  a.lse = want_lse ? lse : nullptr;
  a.chunk_forced = forced_chunk;
  a.chunk_bound = bound;
  // equal rows laid out back to back (a top-k selection) make nnz a multiple of T
  a.row_len_guess = (bound == 0 && !has_extra && num_indices > 0 && num_indices % num_tokens == 0)
                        ? num_indices / num_tokens
                        : 0;
  a.ws_out = nullptr;
  a.ws_lse = nullptr;
  a.ws_prefix = nullptr;
  a.sink = x.sink;
  if (has_extra) {
    a.extra_records = static_cast<const uint8_t *>(x.records);
    a.extra_num_records = x.num_records;
    a.extra_indptr = x.indptr;
    a.extra_indices = x.indices;
    a.extra_num_indices = x.num_indices;
  }
  if (bound > 0) {
    const mla::SplitLayout l = mla::split_layout(num_tokens, num_heads, bound);
    void *ws = workspace;
    if (x.scratch) {
      if (l.bytes > kScratchBytes)
        return fail(MLA_ERR_UNSUPPORTED,
                    "mla_sparse_fwd_noalloc: this call needs %zu bytes of split workspace, the fixed scratch holds %zu",
                    l.bytes, kScratchBytes);
      mla_status_t st = scratch_address(device, &ws);
      if (st != MLA_OK) return st;
    } else if (ws) {
      if (workspace_bytes < l.bytes)
        return fail(MLA_ERR_INVALID_ARGUMENT, "mla_sparse_fwd: workspace of %zu bytes, %zu needed", workspace_bytes, l.bytes);
      if (!aligned(ws, 256)) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_sparse_fwd: workspace not 256-byte aligned");
    } else {
      mla_status_t st = workspace_get(device, l.bytes, &ws);
      if (st != MLA_OK) return st;
    }
    char *base = static_cast<char *>(ws);
    a.ws_out = reinterpret_cast<float *>(base + l.out_off);
    a.ws_lse = reinterpret_cast<float *>(base + l.lse_off);
    a.ws_prefix = reinterpret_cast<int32_t *>(base + l.prefix_off);
  }
  if (x.vp_w) {
    a.vp_w = static_cast<const uint16_t *>(x.vp_w);
    a.vp_gate = static_cast<const uint16_t *>(x.vp_gate);
    a.vp_gate_st = x.vp_gate_st;
    a.vp_out = static_cast<uint16_t *>(x.vp_out);
    a.vp_st = x.vp_st;
    a.vp_sh = x.vp_sh;
  }
  hipError_t e = mla::launch_sparse_fwd(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "mla_sparse_fwd: launch failed: %s", hipGetErrorString(e));
  if (x.vp_w && bound <= 0) {  // no merge to fuse into: project the forward's output
    mla::VUpProjArgs v;
    v.latent = static_cast<const uint16_t *>(out);
    v.lat_st = out_stride_token;
    v.lat_sh = out_stride_head;
    v.w = static_cast<const uint16_t *>(x.vp_w);
    v.gate = static_cast<const uint16_t *>(x.vp_gate);
    v.gate_st = x.vp_gate_st;
    v.num_tokens = num_tokens;
    v.num_heads = num_heads;
    v.out = static_cast<uint16_t *>(x.vp_out);
    v.out_st = x.vp_st;
    v.out_sh = x.vp_sh;
    v.w_prepared = true;
    e = mla::launch_v_up_proj(v, device_cus(device), static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "mla_sparse_fwd_v_up_proj: launch failed: %s", hipGetErrorString(e));
  }
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status_t mla_sparse_fwd(const void *q, int64_t num_tokens, int32_t num_heads, int64_t q_stride_token,
                            int64_t q_stride_head, const void *kv_records, int64_t num_records, int64_t record_stride,
                            const void *kv_indptr, const void *kv_indices, int64_t num_indices, float softmax_scale,
                            uint32_t flags, void *out, int64_t out_stride_token, int64_t out_stride_head, float *lse,
                            void *workspace, size_t workspace_bytes, void *stream) {
  return sparse_fwd_impl(q, num_tokens, num_heads, q_stride_token, q_stride_head, kv_records, num_records,
                         record_stride, kv_indptr, kv_indices, num_indices, softmax_scale, flags, out,
                         out_stride_token, out_stride_head, lse, workspace, workspace_bytes, stream, FwdExtra());
}

mla_status_t mla_sparse_fwd_ex(const void *q, int64_t num_tokens, int32_t num_heads, int64_t q_stride_token,
                               int64_t q_stride_head, const void *kv_records, int64_t num_records,
                               int64_t record_stride, const void *kv_indptr, const void *kv_indices,
                               int64_t num_indices, const float *attn_sink, const void *extra_records,
                               int64_t extra_num_records, int64_t extra_record_stride, const void *extra_indptr,
                               const void *extra_indices, int64_t extra_num_indices, float softmax_scale,
                               uint32_t flags, void *out, int64_t out_stride_token, int64_t out_stride_head,
                               float *lse, void *workspace, size_t workspace_bytes, void *stream) {
  FwdExtra x;
  x.sink = attn_sink;
  x.records = extra_records;
  x.num_records = extra_num_records;
  x.record_stride = extra_record_stride;
  x.indptr = extra_indptr;
  x.indices = extra_indices;
  x.num_indices = extra_num_indices;
  return sparse_fwd_impl(q, num_tokens, num_heads, q_stride_token, q_stride_head, kv_records, num_records,
                         record_stride, kv_indptr, kv_indices, num_indices, softmax_scale, flags, out,
                         out_stride_token, out_stride_head, lse, workspace, workspace_bytes, stream, x);
}

mla_status_t mla_sparse_fwd_noalloc(const void *q, int64_t num_tokens, int32_t num_heads, int64_t q_stride_token,
                                    int64_t q_stride_head, const void *kv_records, int64_t num_records,
                                    int64_t record_stride, const void *kv_indptr, const void *kv_indices,
                                    int64_t num_indices, float softmax_scale, uint32_t flags, void *out,
                                    int64_t out_stride_token, int64_t out_stride_head, float *lse, void *stream) {
  FwdExtra x;
  x.scratch = true;
  return sparse_fwd_impl(q, num_tokens, num_heads, q_stride_token, q_stride_head, kv_records, num_records,
                         record_stride, kv_indptr, kv_indices, num_indices, softmax_scale, flags, out,
                         out_stride_token, out_stride_head, lse, nullptr, 0, stream, x);
}

mla_status_t mla_sparse_fwd_v_up_proj(const void *q, int64_t num_tokens, int32_t num_heads, int64_t q_stride_token,
                                      int64_t q_stride_head, const void *kv_records, int64_t num_records,
                                      int64_t record_stride, const void *kv_indptr, const void *kv_indices,
                                      int64_t num_indices, float softmax_scale, uint32_t flags, void *out,
                                      int64_t out_stride_token, int64_t out_stride_head, float *lse,
                                      const void *w_uv_prepared, const void *gate, int64_t gate_stride_token,
                                      void *v_out, int64_t v_out_stride_token, int64_t v_out_stride_head,
                                      void *workspace, size_t workspace_bytes, void *stream) {
  const char *fn = "mla_sparse_fwd_v_up_proj";
  // the projection's own conditions first (the forward checks the rest)
  if (num_tokens < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: num_tokens %lld < 0", fn, (long long)num_tokens);
  if (num_tokens > INT32_MAX - 1) return fail(MLA_ERR_UNSUPPORTED, "%s: num_tokens %lld too large", fn, (long long)num_tokens);
  if (out_stride_token < 0 || out_stride_head < 0 || gate_stride_token < 0 || v_out_stride_token < 0 ||
      v_out_stride_head < 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: negative stride", fn);
  if (!aligned(out, 16) || out_stride_token % 8 || out_stride_head % 8)
    return fail(MLA_ERR_UNSUPPORTED, "%s: out must be 16-byte aligned with strides that are multiples of 8", fn);
  if (!aligned(w_uv_prepared, 16)) return fail(MLA_ERR_UNSUPPORTED, "%s: prepared weights not 16-byte aligned", fn);
  if (!aligned(v_out, 4) || ((v_out_stride_token | v_out_stride_head) & 1) ||
      (gate && (!aligned(gate, 4) || (gate_stride_token & 1))))
    return fail(MLA_ERR_UNSUPPORTED, "%s: v_out / gate must be 4-byte aligned with even strides", fn);
  if (num_heads >= 1 && num_heads <= MLA_MAX_HEADS &&
      (!view_fits(num_tokens, v_out_stride_token, num_heads, v_out_stride_head, 128) ||
       (gate && !view_fits(num_tokens, gate_stride_token, 1, 0, (int64_t)num_heads * 128))))
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: v_out or gate view spans more than 2^62 elements", fn);
  if (num_tokens > 0 && (!w_uv_prepared || !v_out))
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: NULL w_uv_prepared or v_out", fn);
  FwdExtra x;
  x.vp_w = w_uv_prepared;
  x.vp_gate = gate;
  x.vp_gate_st = gate_stride_token;
  x.vp_out = v_out;
  x.vp_st = v_out_stride_token;
  x.vp_sh = v_out_stride_head;
  return sparse_fwd_impl(q, num_tokens, num_heads, q_stride_token, q_stride_head, kv_records, num_records,
                         record_stride, kv_indptr, kv_indices, num_indices, softmax_scale, flags, out,
                         out_stride_token, out_stride_head, lse, workspace, workspace_bytes, stream, x);
}

const char *mla_last_error(void) { return g_error; }

const char *mla_status_string(mla_status_t status) {
  // A C caller may pass any int: read the argument's bits as an int rather
  // than as the enumeration, whose value range in C++ is only 0..7.
  int st;
  std::memcpy(&st, &status, sizeof st);
  switch (st) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARGUMENT: return "MLA_ERR_INVALID_ARGUMENT";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
    case MLA_ERR_OUT_OF_MEMORY: return "MLA_ERR_OUT_OF_MEMORY";
  }
  return "MLA_ERR_UNKNOWN";
}

int32_t mla_abi_version(void) { return MLA_ABI_VERSION; }

int64_t mla_sparse_fwd_split_workgroups(int64_t num_tokens, int64_t num_indices, int32_t num_cus, uint32_t flags) {
  // the forward's own limits: beyond them no call exists to plan for
  if (num_tokens < 0 || num_tokens > INT32_MAX - 1 || num_indices < 0 || num_indices >= MLA_MAX_INDICES ||
      num_cus < 0 || (flags & ~kKnownFlags))
    return -1;
  int32_t forced = 0;
  return plan_split(num_tokens, num_indices, num_cus, flags, &forced);
}

size_t mla_sparse_fwd_workspace_size(int64_t num_tokens, int32_t num_heads, int64_t num_indices, uint32_t flags,
                                     int device) {
  if (num_tokens < 0 || num_tokens > INT32_MAX - 1 || num_indices < 0 || num_indices >= MLA_MAX_INDICES ||
      num_heads < 1 || num_heads > MLA_MAX_HEADS || (flags & ~kKnownFlags)) {
    fail(MLA_ERR_INVALID_ARGUMENT, "mla_sparse_fwd_workspace_size: invalid arguments");
    return (size_t)-1;
  }
  int cus = 0;
  if (!(flags & MLA_FLAG_CHUNK_MASK)) {
    cus = device_cus(device);
    if (cus <= 0) {
      fail(MLA_ERR_HIP, "mla_sparse_fwd_workspace_size: cannot query device %d", device);
      return (size_t)-1;
    }
  }
  int32_t forced = 0;
  const int64_t bound = plan_split(num_tokens, num_indices, cus, flags, &forced);
  if (bound <= 0) return 0;
  return mla::split_layout(num_tokens, num_heads, bound).bytes;
}

mla_status_t mla_workspace_reserve(int device, size_t bytes) {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || device < 0 || device >= count)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_workspace_reserve: no device %d", device);
  void *p = nullptr;
  return workspace_get(device, bytes, &p);
}


mla_status_t mla_cache_insert(const void *kv_c, int64_t kv_c_stride_token, const void *k_pe, int64_t k_pe_stride_token,
                              const int64_t *slot_mapping, int64_t num_tokens, void *kv_records, int64_t num_records,
                              int64_t record_stride, void *stream) {
  if (num_tokens < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_cache_insert: num_tokens %lld < 0", (long long)num_tokens);
  if (kv_c_stride_token < 0 || k_pe_stride_token < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_cache_insert: negative stride");
  if ((kv_c_stride_token | k_pe_stride_token) & 1)
    return fail(MLA_ERR_UNSUPPORTED, "mla_cache_insert: kv_c / k_pe row strides must be even");
  if (record_stride != MLA_RECORD_BYTES)
    return fail(MLA_ERR_UNSUPPORTED, "mla_cache_insert: record pitch %lld, only %d (unpadded) is served", (long long)record_stride,
                MLA_RECORD_BYTES);
  if (num_records < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_cache_insert: num_records %lld < 0", (long long)num_records);
  if (num_records > kMaxPoolRecords) return fail(MLA_ERR_UNSUPPORTED, "mla_cache_insert: num_records %lld >= 2^40", (long long)num_records);
  if (!view_fits(num_tokens, kv_c_stride_token, 1, 0, MLA_KV_LORA_RANK) || !view_fits(num_tokens, k_pe_stride_token, 1, 0, MLA_ROPE_DIM))
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_cache_insert: kv_c or k_pe view spans more than 2^62 elements");
  if (!aligned(kv_c, 4) || !aligned(k_pe, 4)) return fail(MLA_ERR_UNSUPPORTED, "mla_cache_insert: kv_c / k_pe not 4-byte aligned");
  if (!aligned(slot_mapping, 8)) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_cache_insert: slot_mapping not 8-byte aligned");
  if (!aligned(kv_records, 16)) return fail(MLA_ERR_UNSUPPORTED, "mla_cache_insert: kv_records base not 16-byte aligned");
  if (num_tokens == 0) return MLA_OK;
  if (!kv_c || !k_pe || !slot_mapping) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_cache_insert: NULL kv_c, k_pe or slot_mapping");
  if (num_records > 0 && !kv_records) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_cache_insert: NULL kv_records");
  if (num_tokens > ((int64_t)INT32_MAX) * 4) return fail(MLA_ERR_UNSUPPORTED, "mla_cache_insert: too many tokens");
  mla::InsertArgs a;
  a.kv_c = static_cast<const uint16_t *>(kv_c);
  a.kv_c_stride = kv_c_stride_token;
  a.k_pe = static_cast<const uint16_t *>(k_pe);
  a.k_pe_stride = k_pe_stride_token;
  a.slots = slot_mapping;
  a.num_tokens = num_tokens;
  a.records = static_cast<uint8_t *>(kv_records);
  a.num_records = num_records;
  hipError_t e = mla::launch_cache_insert(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "mla_cache_insert: launch failed: %s", hipGetErrorString(e));
  return MLA_OK;
}

mla_status_t mla_decode_q_concat_insert(const void *ql_nope, int64_t ql_stride_token, int64_t ql_stride_head,
                                        const void *q_pe, int64_t q_pe_stride_token, int64_t q_pe_stride_head,
                                        const void *kv_c, int64_t kv_c_stride_token, const void *k_pe,
                                        int64_t k_pe_stride_token, const int64_t *slot_mapping, int64_t num_tokens,
                                        int32_t num_heads, const int64_t *positions, const float *cos_sin_cache,
                                        int64_t max_position, void *mqa_q, int64_t mqa_stride_token,
                                        int64_t mqa_stride_head, void *kv_records, int64_t num_records,
                                        int64_t record_stride, void *stream) {
  const char *fn = "mla_decode_q_concat_insert";
  if (num_tokens < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: num_tokens %lld < 0", fn, (long long)num_tokens);
  if (num_heads < 1 || num_heads > MLA_MAX_EPILOGUE_HEADS)
    return fail(MLA_ERR_UNSUPPORTED, "%s: num_heads %d outside 1..%d", fn, num_heads, MLA_MAX_EPILOGUE_HEADS);
  const int64_t strides[8] = {ql_stride_token,  ql_stride_head,   q_pe_stride_token, q_pe_stride_head,
                              kv_c_stride_token, k_pe_stride_token, mqa_stride_token,  mqa_stride_head};
  for (int64_t st : strides) {
    if (st < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: negative stride", fn);
    if (st & 1) return fail(MLA_ERR_UNSUPPORTED, "%s: strides must be even (4-byte words)", fn);
  }
  if (!aligned(ql_nope, 4) || !aligned(q_pe, 4) || !aligned(kv_c, 4) || !aligned(k_pe, 4) || !aligned(mqa_q, 4))
    return fail(MLA_ERR_UNSUPPORTED, "%s: bf16 arrays must be 4-byte aligned", fn);
  if (record_stride != MLA_RECORD_BYTES)
    return fail(MLA_ERR_UNSUPPORTED, "%s: record pitch %lld, only %d (unpadded) is served", fn, (long long)record_stride,
                MLA_RECORD_BYTES);
  if (num_records < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: num_records %lld < 0", fn, (long long)num_records);
  if (!aligned(kv_records, 16)) return fail(MLA_ERR_UNSUPPORTED, "%s: kv_records base not 16-byte aligned", fn);
  if (!aligned(slot_mapping, 8)) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: slot_mapping not 8-byte aligned", fn);
  if ((positions == nullptr) != (cos_sin_cache == nullptr))
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: positions and cos_sin_cache come together", fn);
  if (positions) {
    if (max_position < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: max_position %lld < 1", fn, (long long)max_position);
    if (!aligned(positions, 8) || !aligned(cos_sin_cache, 4))
      return fail(MLA_ERR_INVALID_ARGUMENT, "%s: misaligned positions or cos_sin_cache", fn);
  }
  if (num_records > kMaxPoolRecords) return fail(MLA_ERR_UNSUPPORTED, "%s: num_records %lld >= 2^40", fn, (long long)num_records);
  if (positions && max_position > ((int64_t)1 << 40))
    return fail(MLA_ERR_UNSUPPORTED, "%s: max_position %lld >= 2^40", fn, (long long)max_position);
  if (!view_fits(num_tokens, ql_stride_token, num_heads, ql_stride_head, MLA_KV_LORA_RANK) ||
      !view_fits(num_tokens, q_pe_stride_token, num_heads, q_pe_stride_head, MLA_ROPE_DIM) ||
      !view_fits(num_tokens, kv_c_stride_token, 1, 0, MLA_KV_LORA_RANK) ||
      !view_fits(num_tokens, k_pe_stride_token, 1, 0, MLA_ROPE_DIM) ||
      !view_fits(num_tokens, mqa_stride_token, num_heads, mqa_stride_head, MLA_QK_DIM))
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: a view spans more than 2^62 elements", fn);
  if (num_tokens == 0) return MLA_OK;
  if (num_tokens > INT32_MAX) return fail(MLA_ERR_UNSUPPORTED, "%s: too many tokens", fn);
  if (!ql_nope || !q_pe || !kv_c || !k_pe || !slot_mapping || !mqa_q)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: NULL input or output", fn);
  if (num_records > 0 && !kv_records) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: NULL kv_records", fn);
  mla::DecodeEpilogueArgs a;
  a.ql_nope = static_cast<const uint16_t *>(ql_nope);
  a.ql_stride_token = ql_stride_token;
  a.ql_stride_head = ql_stride_head;
  a.q_pe = static_cast<const uint16_t *>(q_pe);
  a.qpe_stride_token = q_pe_stride_token;
  a.qpe_stride_head = q_pe_stride_head;
  a.kv_c = static_cast<const uint16_t *>(kv_c);
  a.kv_c_stride = kv_c_stride_token;
  a.k_pe = static_cast<const uint16_t *>(k_pe);
  a.k_pe_stride = k_pe_stride_token;
  a.slots = slot_mapping;
  a.num_tokens = num_tokens;
  a.num_heads = num_heads;
  a.positions = positions;
  a.cos_sin = cos_sin_cache;
  a.max_position = max_position;
  a.mqa_q = static_cast<uint16_t *>(mqa_q);
  a.mq_stride_token = mqa_stride_token;
  a.mq_stride_head = mqa_stride_head;
  a.records = static_cast<uint8_t *>(kv_records);
  a.num_records = num_records;
  hipError_t e = mla::launch_decode_epilogue(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return MLA_OK;
}

mla_status_t mla_gather_upconvert(const void *kv_records, int64_t num_records, int64_t record_stride,
                                  int64_t block_size, const int32_t *block_table, int64_t block_table_stride,
                                  int64_t block_table_width, const int32_t *cu_seq_lens, const int32_t *seq_starts,
                                  int32_t batch_size, int64_t num_tokens, void *dst, int64_t dst_stride_token,
                                  void *stream) {
  const char *fn = "mla_gather_upconvert";
  if (num_tokens < 0 || num_records < 0 || batch_size < 0 || block_table_width < 0 || block_table_stride < 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: negative size or stride", fn);
  if (block_size < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: block_size %lld < 1", fn, (long long)block_size);
  if (block_size > ((int64_t)1 << 31)) return fail(MLA_ERR_UNSUPPORTED, "%s: block_size %lld > 2^31", fn, (long long)block_size);
  if (record_stride != MLA_RECORD_BYTES)
    return fail(MLA_ERR_UNSUPPORTED, "%s: record pitch %lld, only %d (unpadded) is served", fn, (long long)record_stride,
                MLA_RECORD_BYTES);
  if (!aligned(kv_records, 16)) return fail(MLA_ERR_UNSUPPORTED, "%s: kv_records base not 16-byte aligned", fn);
  if (!aligned(dst, 16) || dst_stride_token % 8 != 0 || dst_stride_token < MLA_QK_DIM)
    return fail(MLA_ERR_UNSUPPORTED, "%s: dst must be 16-byte aligned with a row stride >= 576 and a multiple of 8", fn);
  if (!aligned(block_table, 4) || !aligned(cu_seq_lens, 4) || !aligned(seq_starts, 4))
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: misaligned int32 array", fn);
  if (num_tokens == 0) return MLA_OK;
  if (num_records > kMaxPoolRecords) return fail(MLA_ERR_UNSUPPORTED, "%s: num_records %lld >= 2^40", fn, (long long)num_records);
  if (!view_fits(num_tokens, dst_stride_token, 1, 0, MLA_QK_DIM) ||
      !view_fits(batch_size, block_table_stride, 1, 0, block_table_width))
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: dst or block_table view spans more than 2^62 elements", fn);
  if (num_tokens > INT32_MAX) return fail(MLA_ERR_UNSUPPORTED, "%s: too many tokens", fn);
  if (!dst) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: NULL dst", fn);
  if (batch_size > 0 && !cu_seq_lens) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: NULL cu_seq_lens", fn);
  if (batch_size > 0 && block_table_width > 0 && !block_table)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: NULL block_table", fn);
  if (num_records > 0 && !kv_records) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: NULL kv_records", fn);
  mla::GatherArgs a;
  a.records = static_cast<const uint8_t *>(kv_records);
  a.num_records = num_records;
  a.block_size = block_size;
  a.block_table = block_table;
  a.bt_stride = block_table_stride;
  a.bt_width = block_table ? block_table_width : 0;
  a.cu = cu_seq_lens;
  a.starts = seq_starts;
  a.batch = cu_seq_lens ? batch_size : 0;
  a.num_tokens = num_tokens;
  a.dst = static_cast<uint16_t *>(dst);
  a.dst_stride = dst_stride_token;
  hipError_t e = mla::launch_gather_upconvert(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return MLA_OK;
}

namespace {

mla_status_t v_up_proj_impl(const char *fn, bool prepared, const void *latent, int64_t latent_stride_token,
                            int64_t latent_stride_head, const void *w_uv, const void *gate,
                            int64_t gate_stride_token, int64_t num_tokens, int32_t num_heads, void *out,
                            int64_t out_stride_token, int64_t out_stride_head, void *stream) {
  if (num_tokens < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: num_tokens %lld < 0", fn, (long long)num_tokens);
  if (num_heads < 1 || num_heads > MLA_MAX_EPILOGUE_HEADS)
    return fail(MLA_ERR_UNSUPPORTED, "%s: num_heads %d outside 1..%d", fn, num_heads, MLA_MAX_EPILOGUE_HEADS);
  if (latent_stride_token < 0 || latent_stride_head < 0 || gate_stride_token < 0 || out_stride_token < 0 ||
      out_stride_head < 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: negative stride", fn);
  if (!view_fits(num_tokens, latent_stride_token, num_heads, latent_stride_head, MLA_KV_LORA_RANK) ||
      !view_fits(num_tokens, out_stride_token, num_heads, out_stride_head, 128) ||
      (gate && !view_fits(num_tokens, gate_stride_token, 1, 0, (int64_t)num_heads * 128)))
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: a view spans more than 2^62 elements", fn);
  if (!aligned(latent, 16) || latent_stride_token % 8 || latent_stride_head % 8)
    return fail(MLA_ERR_UNSUPPORTED, "%s: latent must be 16-byte aligned with strides that are multiples of 8", fn);
  if (!aligned(out, 4) || (out_stride_token | out_stride_head) & 1 || !aligned(w_uv, prepared ? 16 : 2) ||
      (gate && (!aligned(gate, 4) || (gate_stride_token & 1))))
    return fail(MLA_ERR_UNSUPPORTED, "%s: out / gate must be 4-byte aligned with even strides", fn);
  if (num_tokens == 0) return MLA_OK;
  if (!latent || !w_uv || !out) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: NULL latent, w_uv or out", fn);
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) return fail(MLA_ERR_HIP, "%s: hipGetDevice failed", fn);
  mla::VUpProjArgs a;
  a.latent = static_cast<const uint16_t *>(latent);
  a.lat_st = latent_stride_token;
  a.lat_sh = latent_stride_head;
  a.w = static_cast<const uint16_t *>(w_uv);
  a.gate = static_cast<const uint16_t *>(gate);
  a.gate_st = gate_stride_token;
  a.num_tokens = num_tokens;
  a.num_heads = num_heads;
  a.out = static_cast<uint16_t *>(out);
  a.out_st = out_stride_token;
  a.out_sh = out_stride_head;
  a.w_prepared = prepared;
  hipError_t e = mla::launch_v_up_proj(a, device_cus(device), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return MLA_OK;
}

}  // namespace

mla_status_t mla_v_up_proj(const void *latent, int64_t latent_stride_token, int64_t latent_stride_head,
                           const void *w_uv, const void *gate, int64_t gate_stride_token, int64_t num_tokens,
                           int32_t num_heads, void *out, int64_t out_stride_token, int64_t out_stride_head,
                           void *stream) {
  return v_up_proj_impl("mla_v_up_proj", false, latent, latent_stride_token, latent_stride_head, w_uv, gate,
                        gate_stride_token, num_tokens, num_heads, out, out_stride_token, out_stride_head, stream);
}

mla_status_t mla_v_up_proj_prepared(const void *latent, int64_t latent_stride_token, int64_t latent_stride_head,
                                    const void *w_prepared, const void *gate, int64_t gate_stride_token,
                                    int64_t num_tokens, int32_t num_heads, void *out, int64_t out_stride_token,
                                    int64_t out_stride_head, void *stream) {
  return v_up_proj_impl("mla_v_up_proj_prepared", true, latent, latent_stride_token, latent_stride_head, w_prepared,
                        gate, gate_stride_token, num_tokens, num_heads, out, out_stride_token, out_stride_head,
                        stream);
}

mla_status_t mla_v_up_proj_prepare_weights(const void *w_uv, int32_t num_heads, void *w_prepared, void *stream) {
  const char *fn = "mla_v_up_proj_prepare_weights";
  if (num_heads < 1 || num_heads > MLA_MAX_EPILOGUE_HEADS)
    return fail(MLA_ERR_UNSUPPORTED, "%s: num_heads %d outside 1..%d", fn, num_heads, MLA_MAX_EPILOGUE_HEADS);
  if (!w_uv || !w_prepared) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: NULL w_uv or w_prepared", fn);
  if (!aligned(w_uv, 2) || !aligned(w_prepared, 16))
    return fail(MLA_ERR_UNSUPPORTED, "%s: w_uv must be 2-byte and w_prepared 16-byte aligned", fn);
  const char *a = static_cast<const char *>(w_uv), *b = static_cast<const char *>(w_prepared);
  const int64_t bytes = (int64_t)num_heads * MLA_KV_LORA_RANK * 128 * 2;
  if (a < b + bytes && b < a + bytes) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: w_uv and w_prepared overlap", fn);
  hipError_t e = mla::launch_prepare_w_uv(static_cast<const uint16_t *>(w_uv), static_cast<uint16_t *>(w_prepared),
                                          num_heads, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return MLA_OK;
}

mla_status_t mla_prefill_key_concat_insert(void *q, int64_t q_stride_token, int64_t q_stride_head,
                                           int32_t qk_nope_head_dim, const void *k_nope, int64_t k_nope_stride_token,
                                           int64_t k_nope_stride_head, const void *kv_c, int64_t kv_c_stride_token,
                                           const void *k_pe, int64_t k_pe_stride_token, const int64_t *slot_mapping,
                                           int64_t num_tokens, int32_t num_heads, const int64_t *positions,
                                           const float *cos_sin_cache, int64_t max_position, void *k_out,
                                           int64_t k_out_stride_token, int64_t k_out_stride_head, void *kv_records,
                                           int64_t num_records, int64_t record_stride, void *stream) {
  const char *fn = "mla_prefill_key_concat_insert";
  if (num_tokens < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: num_tokens %lld < 0", fn, (long long)num_tokens);
  if (num_heads < 1 || num_heads > MLA_MAX_EPILOGUE_HEADS)
    return fail(MLA_ERR_UNSUPPORTED, "%s: num_heads %d outside 1..%d", fn, num_heads, MLA_MAX_EPILOGUE_HEADS);
  if (qk_nope_head_dim < 8 || qk_nope_head_dim > 1024 || qk_nope_head_dim % 8)
    return fail(MLA_ERR_UNSUPPORTED, "%s: qk_nope_head_dim %d (a multiple of 8 in 8..1024 is served)", fn,
                qk_nope_head_dim);
  const int64_t strides[8] = {q_stride_token,    q_stride_head,     k_nope_stride_token, k_nope_stride_head,
                              kv_c_stride_token, k_pe_stride_token, k_out_stride_token,  k_out_stride_head};
  for (int64_t st : strides) {
    if (st < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: negative stride", fn);
    if (st & 1) return fail(MLA_ERR_UNSUPPORTED, "%s: strides must be even (4-byte words)", fn);
  }
  if (!aligned(q, 4) || !aligned(k_nope, 4) || !aligned(kv_c, 4) || !aligned(k_pe, 4) || !aligned(k_out, 4))
    return fail(MLA_ERR_UNSUPPORTED, "%s: bf16 arrays must be 4-byte aligned", fn);
  if (record_stride != MLA_RECORD_BYTES)
    return fail(MLA_ERR_UNSUPPORTED, "%s: record pitch %lld, only %d (unpadded) is served", fn, (long long)record_stride,
                MLA_RECORD_BYTES);
  if (num_records < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: num_records %lld < 0", fn, (long long)num_records);
  if (!aligned(kv_records, 16)) return fail(MLA_ERR_UNSUPPORTED, "%s: kv_records base not 16-byte aligned", fn);
  if (!aligned(slot_mapping, 8)) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: slot_mapping not 8-byte aligned", fn);
  if ((positions == nullptr) != (cos_sin_cache == nullptr))
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: positions and cos_sin_cache come together", fn);
  if (positions) {
    if (max_position < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: max_position %lld < 1", fn, (long long)max_position);
    if (!aligned(positions, 8) || !aligned(cos_sin_cache, 4))
      return fail(MLA_ERR_INVALID_ARGUMENT, "%s: misaligned positions or cos_sin_cache", fn);
  }
  if (num_records > kMaxPoolRecords) return fail(MLA_ERR_UNSUPPORTED, "%s: num_records %lld >= 2^40", fn, (long long)num_records);
  if (positions && max_position > ((int64_t)1 << 40))
    return fail(MLA_ERR_UNSUPPORTED, "%s: max_position %lld >= 2^40", fn, (long long)max_position);
  if (!view_fits(num_tokens, q_stride_token, num_heads, q_stride_head, qk_nope_head_dim + MLA_ROPE_DIM) ||
      !view_fits(num_tokens, k_nope_stride_token, num_heads, k_nope_stride_head, qk_nope_head_dim) ||
      !view_fits(num_tokens, kv_c_stride_token, 1, 0, MLA_KV_LORA_RANK) ||
      !view_fits(num_tokens, k_pe_stride_token, 1, 0, MLA_ROPE_DIM) ||
      !view_fits(num_tokens, k_out_stride_token, num_heads, k_out_stride_head, qk_nope_head_dim + MLA_ROPE_DIM))
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: a view spans more than 2^62 elements", fn);
  if (num_tokens == 0) return MLA_OK;
  if (num_tokens > INT32_MAX) return fail(MLA_ERR_UNSUPPORTED, "%s: too many tokens", fn);
  if (!k_nope || !kv_c || !k_pe || !slot_mapping || !k_out || (positions && !q))
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: NULL input or output", fn);
  if (num_records > 0 && !kv_records) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: NULL kv_records", fn);
  mla::PrefillEpilogueArgs a;
  a.q = static_cast<uint16_t *>(q);
  a.q_stride_token = q_stride_token;
  a.q_stride_head = q_stride_head;
  a.nope = qk_nope_head_dim;
  a.k_nope = static_cast<const uint16_t *>(k_nope);
  a.kn_stride_token = k_nope_stride_token;
  a.kn_stride_head = k_nope_stride_head;
  a.kv_c = static_cast<const uint16_t *>(kv_c);
  a.kv_c_stride = kv_c_stride_token;
  a.k_pe = static_cast<const uint16_t *>(k_pe);
  a.k_pe_stride = k_pe_stride_token;
  a.slots = slot_mapping;
  a.num_tokens = num_tokens;
  a.num_heads = num_heads;
  a.positions = positions;
  a.cos_sin = cos_sin_cache;
  a.max_position = max_position;
  a.k_out = static_cast<uint16_t *>(k_out);
  a.ko_stride_token = k_out_stride_token;
  a.ko_stride_head = k_out_stride_head;
  a.records = static_cast<uint8_t *>(kv_records);
  a.num_records = num_records;
  hipError_t e = mla::launch_prefill_epilogue(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return MLA_OK;
}

}  // extern "C"
