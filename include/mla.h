/*
 * mla.h - sparse absorbed multi-head latent attention (MLA) over an
 * fp8_ds_mla latent cache, for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every pointer argument is a DEVICE pointer unless stated
 * otherwise; the caller owns every buffer and the stream.  No call
 * synchronizes the host: work is queued on `stream` (a hipStream_t passed
 * as void*, NULL = the default stream) and the call returns.
 *
 * Record format (vLLM API pages, flydsl_sparse_mla module docstring and
 * flydsl_sparse_mla_fp8ds_supported docstring; fused_mla_key_concat_kv_cache
 * page, fused_mla_key_concat_ds_mla_insert docstring): one 656-byte record
 * per cache slot,
 *     bytes   0 .. 511  latent d = 0..511 as OCP E4M3 ("e4m3fn")
 *     bytes 512 .. 527  4 little-endian float32 scales; scale b covers
 *                       latent [128b, 128b + 128)
 *     bytes 528 .. 655  64 little-endian bf16 rope values
 * latent[d] = e4m3(byte d) * scale[d / 128].  Slot s is record s of the
 * pool; for an unpadded paged pool [num_blocks, block_size, 656] that is
 * block s / block_size, offset s % block_size.
 *
 * Errors: a call that returns anything but MLA_OK has queued nothing and
 * written nothing; mla_last_error() then holds a message for the calling
 * thread.  Validation reads argument values only (no device reads), so a
 * rejected call is safe at any time, including during stream capture.
 *
 * Views: a strided view [rows, heads, width] must span at most 2^62
 * elements, (rows - 1) * row_stride + (heads - 1) * head_stride + width,
 * or the call returns MLA_ERR_INVALID_ARGUMENT (no buffer is that large,
 * and the kernels' 64-bit address arithmetic must not wrap).  The insert,
 * the epilogues and the gather serve pools of at most 2^40 records, tables
 * of at most 2^40 positions and blocks of at most 2^31 records
 * (MLA_ERR_UNSUPPORTED beyond).
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARGUMENT = 1, /* NULL / misaligned pointer, negative size or stride, bad flag bits */
  MLA_ERR_UNSUPPORTED = 2,      /* well-formed, but outside what the library serves */
  MLA_ERR_HIP = 3,              /* a HIP runtime call or a kernel launch failed */
  MLA_ERR_OUT_OF_MEMORY = 4     /* the library-owned split-KV workspace could not be allocated */
} mla_status_t;

#define MLA_RECORD_BYTES 656
#define MLA_KV_LORA_RANK 512
#define MLA_ROPE_DIM 64
#define MLA_QK_DIM 576
#define MLA_MAX_HEADS 16
#define MLA_MAX_INDICES (1 << 29) /* num_indices must be below this */

/* mla_sparse_fwd flags */
#define MLA_FLAG_HAS_INVALID (1u << 0) /* negative slot ids may occur (they are masked either way) */
#define MLA_FLAG_RETURN_LSE (1u << 1)  /* write lse */
#define MLA_FLAG_INDEX_I64 (1u << 2)   /* kv_indptr and kv_indices are int64 (default int32) */
/* Force split-KV with chunks of n 64-key tiles (1 .. 65535); 0 = the
 * library's plan (mla_sparse_fwd_split_workgroups).  Split-KV serves at most
 * 512 rows: a forced split with more is MLA_ERR_UNSUPPORTED. */
#define MLA_FLAG_CHUNK_TILES(n) (((uint32_t)(n)) << 16)
#define MLA_FLAG_CHUNK_MASK (0xFFFFu << 16)

/*
 * mla_sparse_fwd - sparse attention of absorbed MLA queries over records.
 *
 * Defined by the flydsl_sparse_mla page (flydsl_sparse_mla_fp8ds_fwd
 * docstring; the argument limits of flydsl_sparse_mla_fp8ds_supported):
 * for query row t and head h, with J the entries of
 * kv_indices[kv_indptr[t] .. kv_indptr[t+1]) that are >= 0 (and, in this
 * library, < num_records),
 *     k_j = [latent_j | rope_j] (576),   v_j = latent_j (512),
 *     z_j = softmax_scale * <q[t,h,:], k_j>,
 *     out[t,h,:] = sum_j softmax(z)_j v_j      (bf16, round to nearest even),
 *     lse[t,h]   = ln sum_j exp(z_j)           (float32, natural log).
 * A row with no such entry gives out = 0 and lse = -inf.  A slot listed
 * twice counts twice.  When there are too few rows to fill the GPU (and at
 * most 512; above CU-many rows, not when T divides the entry count, rows of
 * one length then having no room for two chunks each), each row's entries
 * are cut into chunks (split-KV): every
 * workgroup of a partial pass plans the chunks from indptr on the device
 * and computes one chunk's float32 partial and LSE, and a second
 * launch combines each row's partials by their LSEs (the merge named by
 * merge_attn_states on the kimi_k3 nvidia mla page).
 *
 *  q            bf16 [num_tokens, num_heads, 576], element (t,h,d) at
 *               q + t*q_stride_token + h*q_stride_head + d (strides in
 *               elements, even, >= 0; base 4-byte aligned).
 *  num_tokens   T >= 0.  T == 0 returns MLA_OK and queues nothing.
 *  num_heads    1 .. 16 (else MLA_ERR_UNSUPPORTED).
 *  kv_records   uint8 records, base 16-byte aligned; num_records >= 0
 *               records at record_stride bytes (must be 656: a padded
 *               page pitch is MLA_ERR_UNSUPPORTED).  Addressed in 64 bits.
 *  kv_indptr    [T + 1] int32 (int64 with MLA_FLAG_INDEX_I64) CSR offsets
 *               into kv_indices, non-decreasing; offsets are clamped to
 *               [0, num_indices] on the device.
 *  kv_indices   [num_indices] int32 (int64 with MLA_FLAG_INDEX_I64) slot ids;
 *               0 <= num_indices < 2^29; may be NULL when num_indices == 0.
 *  softmax_scale  the layer's scale (used as this float32).
 *  flags        MLA_FLAG_* bits; unknown bits are MLA_ERR_INVALID_ARGUMENT.
 *  out          bf16, element (t,h,d) at out + t*out_stride_token +
 *               h*out_stride_head + d for d < 512 (rows may be wider; only
 *               the first 512 columns are written); strides even, >= 0;
 *               base 4-byte aligned.
 *  lse          float32 [T, num_heads] contiguous; required with
 *               MLA_FLAG_RETURN_LSE, ignored otherwise.
 *  workspace    scratch for the split-KV partials and row prefix, of at
 *               least mla_sparse_fwd_workspace_size(...) bytes, 256-byte
 *               aligned; used only when the call splits.  A caller-provided
 *               buffer must not be used by another call that may run at the
 *               same time.  NULL: the library uses a buffer it owns per
 *               device (allocated with hipMalloc on first need and grown,
 *               to at least twice its size, when too small; so call
 *               mla_workspace_reserve before stream capture).  A buffer
 *               that is replaced stays allocated until the process ends,
 *               so work queued earlier and graphs captured earlier keep
 *               valid memory (a graph keeps using the buffer it was
 *               captured with, not the larger one).  Every call
 *               that passes NULL on a device shares that device's buffer:
 *               two such calls that may overlap (different streams, or
 *               several host threads) race, so give each its own workspace.
 *  stream       hipStream_t as void*.
 * Returns MLA_OK when the work is queued.
 */
mla_status_t mla_sparse_fwd(const void *q, int64_t num_tokens, int32_t num_heads,
                            int64_t q_stride_token, int64_t q_stride_head,
                            const void *kv_records, int64_t num_records, int64_t record_stride,
                            const void *kv_indptr, const void *kv_indices, int64_t num_indices,
                            float softmax_scale, uint32_t flags,
                            void *out, int64_t out_stride_token, int64_t out_stride_head,
                            float *lse, void *workspace, size_t workspace_bytes, void *stream);

/*
 * mla_sparse_fwd_ex - mla_sparse_fwd with an attention sink and a second KV
 * segment, the attn_sink and extra_kv / extra_indptr / extra_indices
 * arguments of sparse_mla_fwd that the flydsl_sparse_mla page lists (in the
 * flydsl_sparse_mla_fp8ds_supported docstring) without defining them.
 * Reading taken:
 *   - attn_sink: float32 [num_heads] or NULL; head h gets one more logit
 *     attn_sink[h] (natural-log units, compared with softmax_scale * q.k)
 *     whose value vector is zero, so
 *         out = sum_j e^{z_j} v_j / (e^{s_h} + sum_j e^{z_j}),
 *         lse = ln(e^{s_h} + sum_j e^{z_j});
 *     a row with no key then gives out 0 and lse = s_h; s_h = -inf is no sink.
 *   - extra segment (extra_indptr != NULL): a second pool of fp8_ds_mla
 *     records with its own CSR list; row t attends its primary entries and
 *     extra_indices[extra_indptr[t] .. extra_indptr[t+1]) of the second
 *     pool in one softmax (entries < 0 or >= extra_num_records masked).
 *     Same index dtype as the primary list; extra_record_stride must be
 *     656; extra_num_records < 2^31 - 2; num_indices + extra_num_indices
 *     < 2^29.  With MLA_FLAG_CHUNK_TILES or the library's split plan, the
 *     chunks run over both lists of a row; for the workspace size and the
 *     split plan pass num_indices + extra_num_indices as num_indices.
 * Every other argument is as for mla_sparse_fwd.  With attn_sink and
 * extra_indptr both NULL this is mla_sparse_fwd.
 */
mla_status_t mla_sparse_fwd_ex(const void *q, int64_t num_tokens, int32_t num_heads, int64_t q_stride_token,
                               int64_t q_stride_head, const void *kv_records, int64_t num_records,
                               int64_t record_stride, const void *kv_indptr, const void *kv_indices,
                               int64_t num_indices, const float *attn_sink, const void *extra_records,
                               int64_t extra_num_records, int64_t extra_record_stride, const void *extra_indptr,
                               const void *extra_indices, int64_t extra_num_indices, float softmax_scale,
                               uint32_t flags, void *out, int64_t out_stride_token, int64_t out_stride_head,
                               float *lse, void *workspace, size_t workspace_bytes, void *stream);

/*
 * mla_sparse_fwd_noalloc - mla_sparse_fwd for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.  It takes no workspace and allocates
 * nothing (no hipMalloc, hipFree or allocating library call): a call that
 * splits keeps its partials in a fixed device array of
 * MLA_NOALLOC_SCRATCH_BYTES per GPU, which the library holds from its load
 * until the process ends.  A call whose split workspace
 * (mla_sparse_fwd_workspace_size) is larger returns MLA_ERR_UNSUPPORTED and
 * queues nothing.  All calls on one GPU share that array, which keeps the
 * last call's contents: two calls that may overlap on one GPU (different
 * streams or host threads) race.  Arguments as for mla_sparse_fwd without
 * workspace / workspace_bytes; results equal mla_sparse_fwd's bit for bit.
 */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
mla_status_t mla_sparse_fwd_noalloc(const void *q, int64_t num_tokens, int32_t num_heads, int64_t q_stride_token,
                                    int64_t q_stride_head, const void *kv_records, int64_t num_records,
                                    int64_t record_stride, const void *kv_indptr, const void *kv_indices,
                                    int64_t num_indices, float softmax_scale, uint32_t flags, void *out,
                                    int64_t out_stride_token, int64_t out_stride_head, float *lse, void *stream);

/*
 * mla_sparse_fwd_v_up_proj - mla_sparse_fwd followed by the W_UV
 * up-projection with the optional sigmoid gate, with the projection fused
 * into the merge of a split call.
 *
 * The step right after the attention in MultiHeadLatentAttention
 * (vllm.models.kimi_k3.nvidia.mla page: _v_up_proj, then the gate of
 * forward); on the kimi_k3 specialized-decode page the value kernels
 * (MlaValue, and DcpValue, which first merges the ranks' partials) apply it
 * right after the attention core.  Computes exactly what
 * mla_sparse_fwd then mla_v_up_proj_prepared compute on the same arguments,
 * bit for bit: out and lse as mla_sparse_fwd writes them, and
 *     v_out[t, h, v] = bf16( (sum_l out[t, h, l] * W_UV[h, l, v]) * sigmoid(gate[t, 128h + v]) )
 * reading the bf16 `out` values.  A call that splits (see
 * mla_sparse_fwd_split_workgroups) merges the partials and projects the
 * merged rows in one launch, which saves the up-projection's launch and its
 * read of `out`; a call that does not split runs the forward, then the
 * up-projection.
 *
 * Arguments as for mla_sparse_fwd (no sink or second segment), except:
 *  out          as for mla_sparse_fwd, but 16-byte aligned with strides
 *               that are multiples of 8 elements.
 *  w_uv_prepared  W_UV[num_heads, 512, 128] as mla_v_up_proj_prepare_weights
 *               wrote it, 16-byte aligned.
 *  gate         bf16 [T, num_heads * 128], row stride gate_stride_token
 *               (even), or NULL for no gate.
 *  v_out        bf16, element (t, h, v) at v_out + t*v_out_stride_token +
 *               h*v_out_stride_head + v (strides even), base 4-byte aligned.
 */
mla_status_t mla_sparse_fwd_v_up_proj(const void *q, int64_t num_tokens, int32_t num_heads, int64_t q_stride_token,
                                      int64_t q_stride_head, const void *kv_records, int64_t num_records,
                                      int64_t record_stride, const void *kv_indptr, const void *kv_indices,
                                      int64_t num_indices, float softmax_scale, uint32_t flags, void *out,
                                      int64_t out_stride_token, int64_t out_stride_head, float *lse,
                                      const void *w_uv_prepared, const void *gate, int64_t gate_stride_token,
                                      void *v_out, int64_t v_out_stride_token, int64_t v_out_stride_head,
                                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * mla_sparse_fwd_split_workgroups - the split-KV plan mla_sparse_fwd uses
 * (host only, no device access): 0 = one workgroup per row; otherwise the
 * number of workgroups of the partial pass, an upper bound on the number of
 * chunks.  It depends on T, num_indices, the device's compute-unit count and
 * the forced chunk in flags, never on index values: the launch is fixed from
 * bounds known on the host, as the split counts of the decode cores on the
 * kimi_k3 specialized-decode page are (PreparedMla.fill_splits / max_seq).
 * Without a forced chunk the chunk size is then picked on the device from
 * the actual row lengths: the smallest multiple C of 64 entries (at least
 * 512) whose chunks fit that many workgroups, then, where they fit too,
 * sizes alternating C + 128 and C - 128 along the chunk order.  The chunks
 * depend on indptr and this count alone, so results are reproducible.
 * Returns -1 for invalid arguments
 * (negative sizes, num_tokens >= 2^31 - 1 or num_indices >= 2^29, the
 * forward's own limits, or unknown flag bits).
 */
int64_t mla_sparse_fwd_split_workgroups(int64_t num_tokens, int64_t num_indices, int32_t num_cus, uint32_t flags);

/*
 * mla_sparse_fwd_workspace_size - bytes of split-KV workspace a call with
 * these arguments needs on device `device` (0 when it does not split).
 * Host only; queries the device's compute-unit count once.
 * Returns (size_t)-1 on error (see mla_last_error): the argument limits of
 * mla_sparse_fwd_split_workgroups, num_heads outside 1..16, or no device.
 */
size_t mla_sparse_fwd_workspace_size(int64_t num_tokens, int32_t num_heads, int64_t num_indices,
                                     uint32_t flags, int device);

/*
 * mla_workspace_reserve - grow the library-owned split workspace of `device`
 * to at least `bytes` now (it never shrinks), so that later calls that pass
 * workspace = NULL allocate nothing; call it before stream capture.  The
 * library owns this buffer as the decode cores on the kimi_k3
 * specialized-decode page own theirs (trtllm_decode: one workspace per
 * device, sized once and reused by every call).  A buffer replaced by a
 * larger one is kept until the process ends (see mla_sparse_fwd).
 * Returns MLA_ERR_OUT_OF_MEMORY if the allocation fails, MLA_ERR_HIP if the
 * device cannot be selected.
 */
mla_status_t mla_workspace_reserve(int device, size_t bytes);

/*
 * mla_cache_insert - quantize tokens' [kv_c_normed | k_pe] into records.
 *
 * The ds_mla insert of fused_mla_key_concat_ds_mla_insert and of
 * fused_mla_decode_q_concat_kv_cache_insert(ds_mla=True)
 * (fused_mla_key_concat_kv_cache page): for token i with
 * p = slot_mapping[i] >= 0, record p becomes, per 128-wide tile b,
 *     scale_b = max_d |kv_c[i, 128b + d]| / 448        (float32, correctly rounded)
 *     code[d] = E4M3(clamp(kv_c[i, d] / scale_b, -448, 448))
 *               (float32 correctly rounded division, round to nearest even;
 *                a tile of zeros gets scale 0 and codes 0)
 * followed by the 64 bf16 rope values k_pe[i, :] copied bit for bit.
 * Tokens with a negative slot, or a slot >= num_records, are skipped and
 * their records keep their bytes.  Two tokens with the same slot in one
 * call race (undefined which one lands).
 *
 *  kv_c         bf16 [num_tokens, 512], row stride kv_c_stride_token
 *               elements (even), base 4-byte aligned.
 *  k_pe         bf16 [num_tokens, 64], row stride k_pe_stride_token
 *               elements (even), base 4-byte aligned.
 *  slot_mapping int64 [num_tokens], 8-byte aligned.
 *  num_tokens   >= 0; 0 returns MLA_OK and queues nothing.
 *  kv_records   as for mla_sparse_fwd (written in place).
 */
mla_status_t mla_cache_insert(const void *kv_c, int64_t kv_c_stride_token,
                              const void *k_pe, int64_t k_pe_stride_token,
                              const int64_t *slot_mapping, int64_t num_tokens,
                              void *kv_records, int64_t num_records, int64_t record_stride,
                              void *stream);

/*
 * mla_decode_q_concat_insert - the MLA decode epilogue in one launch: the
 * latent decode query mqa_q = [ql_nope | RoPE(q_pe)] and the insert of
 * [kv_c_normed | RoPE(k_pe)] into the fp8_ds_mla cache.
 *
 * Defined by fused_mla_decode_q_concat_kv_cache_insert with ds_mla=True
 * (fused_mla_key_concat_kv_cache page, function docstring: bf16 mqa_q and
 * the 656-byte block-scaled cache, one launch, right before the latent
 * attention).  With positions and cos_sin_cache, GPT-J-style RoPE (module
 * docstring) is applied to q_pe and k_pe in float32 from the fp32 table
 * (vllm.models.kimi_k3.nvidia.mla page, MultiHeadLatentAttention): pair i = (x[2i], x[2i+1]) of the 64 rope
 * values, c = cos_sin_cache[pos][i], s = cos_sin_cache[pos][32 + i],
 *     y[2i] = x[2i]*c - x[2i+1]*s,   y[2i+1] = x[2i+1]*c + x[2i]*s,
 * each product and sum rounded to float32 (no fused multiply-add), the
 * result rounded to bf16 (nearest even).  Without them q_pe and k_pe are
 * copied bit for bit.  The record is written as by mla_cache_insert, with
 * the rotated k_pe as its rope part; a token with a negative slot or a slot
 * >= num_records writes mqa_q only.
 *
 *  ql_nope      bf16 [num_tokens, num_heads, 512], element (b,h,d) at
 *               ql_nope + b*ql_stride_token + h*ql_stride_head + d.
 *  q_pe         bf16 [num_tokens, num_heads, 64], likewise.
 *  kv_c         bf16 [num_tokens, 512], row stride kv_c_stride_token.
 *  k_pe         bf16 [num_tokens, 64], row stride k_pe_stride_token.
 *  slot_mapping int64 [num_tokens], 8-byte aligned.
 *  num_tokens   >= 0; 0 returns MLA_OK and queues nothing.
 *  num_heads    1 .. MLA_MAX_EPILOGUE_HEADS.
 *  positions    int64 [num_tokens] or NULL; a position outside
 *               [0, max_position) is clamped into it (keeps reads in the table).
 *  cos_sin_cache float32 [max_position, 64] (row b: 32 cosines, then 32
 *               sines), contiguous, 4-byte aligned; NULL exactly when
 *               positions is NULL.
 *  mqa_q        bf16 output [num_tokens, num_heads, 576], element (b,h,d) at
 *               mqa_q + b*mqa_stride_token + h*mqa_stride_head + d.
 *  kv_records   as for mla_sparse_fwd (written in place).
 * Strides are in elements, even and >= 0; bf16 bases 4-byte aligned.
 * Two tokens with the same slot race, as in mla_cache_insert.
 */
#define MLA_MAX_EPILOGUE_HEADS 1024
mla_status_t mla_decode_q_concat_insert(const void *ql_nope, int64_t ql_stride_token, int64_t ql_stride_head,
                                        const void *q_pe, int64_t q_pe_stride_token, int64_t q_pe_stride_head,
                                        const void *kv_c, int64_t kv_c_stride_token, const void *k_pe,
                                        int64_t k_pe_stride_token, const int64_t *slot_mapping, int64_t num_tokens,
                                        int32_t num_heads, const int64_t *positions, const float *cos_sin_cache,
                                        int64_t max_position, void *mqa_q, int64_t mqa_stride_token,
                                        int64_t mqa_stride_head, void *kv_records, int64_t num_records,
                                        int64_t record_stride, void *stream);

/*
 * mla_prefill_key_concat_insert - the MLA prefill epilogue in one launch:
 * GPT-J RoPE on the rope part of q in place, the bf16 full key
 * k_out = [k_nope | RoPE(k_pe)] for every head, and the insert of
 * [kv_c_normed | RoPE(k_pe)] into the fp8_ds_mla cache.
 *
 * Defined by fused_mla_key_concat_ds_mla_insert (fused_mla_key_concat_kv_cache
 * page: it builds the bf16 full key and writes the latent into the
 * fp8_ds_mla cache; q is [Tp, H, qk_head_dim] with RoPE applied in place, k_nope
 * [Tp, H, qk_nope_head_dim], k_pe [Tp, 64], the returned key
 * [Tp, H, qk_nope_head_dim + 64]).  RoPE, positions and cos_sin_cache as
 * for mla_decode_q_concat_insert; without them q is left untouched and the
 * key's rope part is k_pe bit for bit.  The record is written as by
 * mla_cache_insert with the rotated k_pe.
 *
 *  q            bf16, element (t,h,d) at q + t*q_stride_token + h*q_stride_head
 *               + d, d < qk_nope_head_dim + 64; only d >= qk_nope_head_dim is
 *               written (and only with RoPE).  May be NULL without RoPE.
 *  qk_nope_head_dim  a multiple of 8 in 8 .. 1024 (128 for the pages' model).
 *  k_nope       bf16 [num_tokens, num_heads, qk_nope_head_dim] (strided).
 *  kv_c, k_pe, slot_mapping, positions, cos_sin_cache, kv_records  as for
 *               mla_decode_q_concat_insert.
 *  k_out        bf16 output [num_tokens, num_heads, qk_nope_head_dim + 64].
 * Strides in elements, even, >= 0; bf16 bases 4-byte aligned; outputs must
 * not overlap inputs (q is updated in place only in its rope columns).
 */
mla_status_t mla_prefill_key_concat_insert(void *q, int64_t q_stride_token, int64_t q_stride_head,
                                           int32_t qk_nope_head_dim, const void *k_nope, int64_t k_nope_stride_token,
                                           int64_t k_nope_stride_head, const void *kv_c, int64_t kv_c_stride_token,
                                           const void *k_pe, int64_t k_pe_stride_token, const int64_t *slot_mapping,
                                           int64_t num_tokens, int32_t num_heads, const int64_t *positions,
                                           const float *cos_sin_cache, int64_t max_position, void *k_out,
                                           int64_t k_out_stride_token, int64_t k_out_stride_head, void *kv_records,
                                           int64_t num_records, int64_t record_stride, void *stream);

/*
 * mla_gather_upconvert - gather a context chunk's records through the block
 * table into a bf16 [num_tokens, 576] workspace (dequantized latent | rope).
 *
 * Defined by cp_gather_and_upconvert_fp8_kv_cache as the kimi_k3 nvidia mla
 * page calls it in _gather_context_latent (src_cache, dst = workspace[:toks],
 * block_table, workspace_starts = the chunk's cu_seq_lens, batch_size,
 * seq_starts): for request r and j < cu_seq_lens[r+1] - cu_seq_lens[r],
 * context position p = seq_starts[r] + j (seq_starts NULL: 0) is read from
 * record block_table[r][p / block_size] * block_size + p % block_size and
 * written to row cu_seq_lens[r] + j as
 *     dst[row, d]       = bf16(f32(E4M3(code[d])) * scale[d / 128]), d < 512
 *     dst[row, 512 + i] = rope[i] (bit copy), i < 64
 * (float32 product, then bf16 round to nearest even: the model dtype of the
 * workspace).  Rows of [0, num_tokens) with no valid source - outside every
 * request, a position past block_table_width, a block id < 0 or a slot
 * >= num_records - are written as zeros.
 *
 *  kv_records   the record pool (num_records records at record_stride = 656
 *               bytes, 16-byte aligned base), as for mla_sparse_fwd.
 *  block_size   records per block (>= 1).
 *  block_table  int32 [batch_size, >= block_table_width], row r at
 *               block_table + r*block_table_stride.
 *  cu_seq_lens  int32 [batch_size + 1], non-decreasing workspace rows.
 *  seq_starts   int32 [batch_size] first context position per request, or NULL.
 *  dst          bf16 [num_tokens, 576] output, 16-byte aligned, row stride
 *               dst_stride_token elements (a multiple of 8, >= 576).
 *  num_tokens   rows to write, 0 .. 2^31 - 1 (0 queues nothing).
 */
mla_status_t mla_gather_upconvert(const void *kv_records, int64_t num_records, int64_t record_stride,
                                  int64_t block_size, const int32_t *block_table, int64_t block_table_stride,
                                  int64_t block_table_width, const int32_t *cu_seq_lens, const int32_t *seq_starts,
                                  int32_t batch_size, int64_t num_tokens, void *dst, int64_t dst_stride_token,
                                  void *stream);

/*
 * mla_v_up_proj - project the latent attention output back to v with
 * W_UV, optionally times the sigmoid gate:
 *     out[t,h,v] = bf16( (sum_l latent[t,h,l] * w_uv[h,l,v]) * sigmoid(gate[t, 128h + v]) )
 * (float32 accumulation; without a gate the sigmoid factor is 1; one round
 * to nearest even).
 *
 * Defined by _v_up_proj on the vllm.models.kimi_k3.nvidia.mla page (the
 * per-head bmm of the [T, H, 512] latent output with W_UV, the (N, L, V)
 * weight process_weights_after_loading splits from kv_b_proj) and the
 * layer's gate (forward: attn_out = _gate_sigmoid_mul(attn_out, gate), the
 * gate being g_proj's [T, H * 128] output); v_head_dim is 128.
 *
 *  latent       bf16, element (t,h,l) at latent + t*latent_stride_token +
 *               h*latent_stride_head + l, l < 512; 16-byte aligned base,
 *               strides multiples of 8 (e.g. mla_sparse_fwd's out).
 *  w_uv         bf16 [num_heads, 512, 128] contiguous.
 *  gate         bf16, element (t, 128h + v) at gate + t*gate_stride_token +
 *               128h + v, or NULL (no gate).  4-byte aligned, even stride.
 *  out          bf16, element (t,h,v) at out + t*out_stride_token +
 *               h*out_stride_head + v, v < 128; 4-byte aligned, even strides.
 *  num_tokens   >= 0 (0 queues nothing); num_heads 1 .. MLA_MAX_EPILOGUE_HEADS.
 */
mla_status_t mla_v_up_proj(const void *latent, int64_t latent_stride_token, int64_t latent_stride_head,
                           const void *w_uv, const void *gate, int64_t gate_stride_token, int64_t num_tokens,
                           int32_t num_heads, void *out, int64_t out_stride_token, int64_t out_stride_head,
                           void *stream);

/*
 * mla_v_up_proj_prepare_weights - W_UV in the up-projection's own order,
 * once, after the weights are loaded (the page's
 * process_weights_after_loading prepares W_UV from kv_b_proj at the same
 * point).  Writes num_heads * 512 * 128 * 2 bytes to w_prepared: the same
 * values, laid out as the matrix-core fragments mla_v_up_proj_prepared
 * loads directly (an internal order: use the buffer only with that call and
 * the same num_heads).
 *
 *  w_uv         bf16 [num_heads, 512, 128] contiguous, 2-byte aligned.
 *  num_heads    1 .. MLA_MAX_EPILOGUE_HEADS.
 *  w_prepared   num_heads * 131072 bytes, 16-byte aligned, not overlapping w_uv.
 */
mla_status_t mla_v_up_proj_prepare_weights(const void *w_uv, int32_t num_heads, void *w_prepared, void *stream);

/*
 * mla_v_up_proj_prepared - mla_v_up_proj with the weights from
 * mla_v_up_proj_prepare_weights: the same results bit for bit, without the
 * per-call weight transposition.  Arguments as for mla_v_up_proj, with
 * w_prepared (16-byte aligned) in place of w_uv.
 */
mla_status_t mla_v_up_proj_prepared(const void *latent, int64_t latent_stride_token, int64_t latent_stride_head,
                                    const void *w_prepared, const void *gate, int64_t gate_stride_token,
                                    int64_t num_tokens, int32_t num_heads, void *out, int64_t out_stride_token,
                                    int64_t out_stride_head, void *stream);

/* Message for the last failed call on this thread ("" if none).  Host memory
 * owned by the library, valid until the thread's next failing call. */
const char *mla_last_error(void);

/* Static name of a status code. */
const char *mla_status_string(mla_status_t status);

/* ABI version of this header (MLA_ABI_VERSION). */
#define MLA_ABI_VERSION 10
int32_t mla_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
