"""Thin Python binding over libmla.so (ctypes).

Argument marshalling only: tensors are turned into pointers, sizes and
strides, and every step of the computation runs in the library's HIP
kernels.  PyTorch provides device memory (outputs, the split-KV workspace)
and the current stream.  There is no fallback: if libmla.so is missing or
fails to load, every call raises.

Names and keyword arguments follow flydsl_sparse_mla_fp8ds_fwd on the
flydsl_sparse_mla page and the ds_mla insert and decode epilogue
(fused_mla_decode_q_concat_kv_cache_insert) on the
fused_mla_key_concat_kv_cache page.
"""

import ctypes
import os
import threading

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla.so")

RECORD_BYTES = 656
KV_LORA_RANK = 512
QK_ROPE_HEAD_DIM = 64
MAX_HEADS = 16
MAX_CHUNK_TILES = 65535
MAX_EPILOGUE_HEADS = 1024

FLAG_HAS_INVALID = 1 << 0
FLAG_RETURN_LSE = 1 << 1
FLAG_INDEX_I64 = 1 << 2
CHUNK_SHIFT = 16

STATUS = {0: "MLA_OK", 1: "MLA_ERR_INVALID_ARGUMENT", 2: "MLA_ERR_UNSUPPORTED", 3: "MLA_ERR_HIP",
          4: "MLA_ERR_OUT_OF_MEMORY"}

# Exported entry points and their C signatures (include/mla.h).
_I64, _I32, _U32, _F32, _P, _SZ = (ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_float,
                                   ctypes.c_void_p, ctypes.c_size_t)
SIGNATURES = {
    "mla_sparse_fwd": (_I32, [_P, _I64, _I32, _I64, _I64, _P, _I64, _I64, _P, _P, _I64, _F32, _U32, _P, _I64, _I64,
                              _P, _P, _SZ, _P]),
    "mla_sparse_fwd_ex": (_I32, [_P, _I64, _I32, _I64, _I64, _P, _I64, _I64, _P, _P, _I64, _P, _P, _I64, _I64, _P, _P,
                                 _I64, _F32, _U32, _P, _I64, _I64, _P, _P, _SZ, _P]),
    "mla_sparse_fwd_noalloc": (_I32, [_P, _I64, _I32, _I64, _I64, _P, _I64, _I64, _P, _P, _I64, _F32, _U32, _P, _I64,
                                      _I64, _P, _P]),
    "mla_sparse_fwd_v_up_proj": (_I32, [_P, _I64, _I32, _I64, _I64, _P, _I64, _I64, _P, _P, _I64, _F32, _U32, _P,
                                        _I64, _I64, _P, _P, _P, _I64, _P, _I64, _I64, _P, _SZ, _P]),
    "mla_sparse_fwd_split_workgroups": (_I64, [_I64, _I64, _I32, _U32]),
    "mla_sparse_fwd_workspace_size": (_SZ, [_I64, _I32, _I64, _U32, ctypes.c_int]),
    "mla_workspace_reserve": (_I32, [ctypes.c_int, _SZ]),
    "mla_cache_insert": (_I32, [_P, _I64, _P, _I64, _P, _I64, _P, _I64, _I64, _P]),
    "mla_v_up_proj": (_I32, [_P, _I64, _I64, _P, _P, _I64, _I64, _I32, _P, _I64, _I64, _P]),
    "mla_v_up_proj_prepared": (_I32, [_P, _I64, _I64, _P, _P, _I64, _I64, _I32, _P, _I64, _I64, _P]),
    "mla_v_up_proj_prepare_weights": (_I32, [_P, _I32, _P, _P]),
    "mla_gather_upconvert": (_I32, [_P, _I64, _I64, _I64, _P, _I64, _I64, _P, _P, _I32, _I64, _P, _I64, _P]),
    "mla_prefill_key_concat_insert": (_I32, [_P, _I64, _I64, _I32, _P, _I64, _I64, _P, _I64, _P, _I64, _P, _I64,
                                             _I32, _P, _P, _I64, _P, _I64, _I64, _P, _I64, _I64, _P]),
    "mla_decode_q_concat_insert": (_I32, [_P, _I64, _I64, _P, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, _I32, _P,
                                          _P, _I64, _P, _I64, _I64, _P, _I64, _I64, _P]),
    "mla_last_error": (ctypes.c_char_p, []),
    "mla_status_string": (ctypes.c_char_p, [_I32]),
    "mla_abi_version": (_I32, []),
}

_lib = None
_lock = threading.Lock()


class MlaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def lib():
    """The loaded library with its C signatures set (raises if it cannot load)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        f"{LIB_PATH} is missing: build it with "
                        "`python -m head_latent_attention_sparse_amd.build`")
                handle = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in SIGNATURES.items():
                    fn = getattr(handle, name)
                    fn.restype = res
                    fn.argtypes = args
                _lib = handle
    return _lib


def _check(status, unsupported_is_value_error=True):
    if status == 0:
        return
    msg = lib().mla_last_error().decode()
    if status in (1, 2) and unsupported_is_value_error:
        raise ValueError(f"{STATUS[status]}: {msg}")
    raise MlaError(status, msg)


def _record_pool(kv):
    """(base pointer, number of records, record pitch in bytes) of a pool view.

    A pool is any 1-byte tensor of rank 2 to 4 whose last dim holds one
    656-byte record contiguously, e.g. a flat [N, 656] pool, [N, 1, 656],
    [N, 1, 1, 656], or a paged pool [num_blocks, block_size, 656].  The
    dims before the record dim must step through memory as one evenly
    spaced run (each dim's stride equal to the next inner dim's stride
    times its size, size-1 dims ignored); the pitch is that run's innermost
    stride.  A run that is not even (a padded page pitch) gives pitch -1,
    and the library serves only pitch 656, so both are refused there.
    """
    if not torch.is_tensor(kv) or kv.element_size() != 1 or not 2 <= kv.ndim <= 4:
        raise ValueError("kv cache must be a 1-byte tensor of rank 2, 3 or 4")
    if kv.shape[-1] != RECORD_BYTES or kv.stride(-1) != 1:
        raise ValueError("kv cache rows must be 656 contiguous bytes")
    count = 1
    for size in kv.shape[:-1]:
        count *= size
    walk = [(size, stride) for size, stride in zip(kv.shape[:-1], kv.stride()[:-1]) if size > 1]
    if not walk:
        return kv.data_ptr(), count, RECORD_BYTES
    pitch = walk[-1][1]
    span = pitch
    for size, stride in reversed(walk):
        if stride != span:
            return kv.data_ptr(), count, -1
        span = stride * size
    return kv.data_ptr(), count, pitch


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def split_workgroups(num_tokens, num_indices, num_cus, chunk_tiles=0):
    """The split-KV plan (host only): 0 = one workgroup per row, else the
    workgroups of the partial pass; ``chunk_tiles`` forces chunks of that
    many 64-key tiles."""
    return lib().mla_sparse_fwd_split_workgroups(num_tokens, num_indices, num_cus, chunk_tiles << CHUNK_SHIFT)


def _fwd_query_and_lists(q, kv_indptr, kv_indices):
    """The forward's checks of q and the CSR lists; returns (T, H)."""
    if not (torch.is_tensor(q) and q.is_cuda and q.ndim == 3 and q.dtype == torch.bfloat16):
        raise ValueError("q must be a CUDA bf16 tensor [T, H, 576]")
    t_count, heads, dqk = q.shape
    if dqk != KV_LORA_RANK + QK_ROPE_HEAD_DIM or q.stride(2) != 1:
        raise ValueError("q rows must be 576 contiguous bf16 values")
    if not 1 <= heads <= MAX_HEADS:
        raise ValueError(f"{heads} heads: 1 .. {MAX_HEADS} are served")
    for name, x in (("kv_indptr", kv_indptr), ("kv_indices", kv_indices)):
        if not (torch.is_tensor(x) and x.device == q.device and x.ndim == 1 and x.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous 1-D tensor on q's device")
        if x.dtype not in (torch.int32, torch.int64):
            raise ValueError(f"{name} must be int32 or int64")
    if kv_indptr.dtype != kv_indices.dtype:
        raise ValueError("kv_indptr and kv_indices must have the same dtype")
    if kv_indptr.numel() != t_count + 1:
        raise ValueError("kv_indptr must have T + 1 entries")
    return t_count, heads


def _fwd_workspace(L, q, t_count, heads, total_nnz, flags, workspace):
    """The split workspace a forward call needs: (pointer, bytes, the
    workspace tensor), pointer None and 0 bytes when the call does not
    split.  A caller's workspace is used if large enough, else one is
    allocated."""
    dev = q.device.index if q.device.index is not None else torch.cuda.current_device()
    if t_count == 0:
        return None, 0, workspace
    need = L.mla_sparse_fwd_workspace_size(t_count, heads, total_nnz, flags, dev)
    if need == ctypes.c_size_t(-1).value:
        _check(3)
    if need == 0:
        return None, 0, workspace
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace.numel() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, {need} needed")
    return workspace.data_ptr(), workspace.numel(), workspace


def sparse_fwd(q, kv_cache, kv_indptr, kv_indices, softmax_scale, *, has_invalid=False, out=None,
               return_lse=False, chunk_tiles=0, workspace=None, attn_sink=None, extra_kv=None,
               extra_indptr=None, extra_indices=None):
    """Sparse MLA forward over fp8_ds_mla records -> (out, lse or None).

    q [T, H, 576] bf16 (H <= 16, stride(2) == 1); kv_cache a record pool
    view; kv_indptr [T + 1] and kv_indices [nnz] int32 or int64 (the same
    dtype, contiguous); out optional [T, H, >= 512] bf16.  ``chunk_tiles``
    forces split-KV with chunks of that many 64-key tiles (0 = the library's
    plan).  ``workspace`` optionally supplies the split partial buffer (a
    CUDA uint8 tensor).  ``attn_sink`` (float32 [H]) adds a per-head sink
    logit; ``extra_kv`` / ``extra_indptr`` / ``extra_indices`` give a second
    record pool and CSR list attended jointly with the first
    (mla_sparse_fwd_ex).
    """
    t_count, heads = _fwd_query_and_lists(q, kv_indptr, kv_indices)
    use_extra = extra_indptr is not None or extra_indices is not None or extra_kv is not None
    if use_extra:
        if extra_kv is None or extra_indptr is None or extra_indices is None:
            raise ValueError("extra_kv, extra_indptr and extra_indices come together")
        for name, x in (("extra_indptr", extra_indptr), ("extra_indices", extra_indices)):
            if not (torch.is_tensor(x) and x.device == q.device and x.ndim == 1 and x.is_contiguous()
                    and x.dtype == kv_indices.dtype):
                raise ValueError(f"{name} must be a contiguous 1-D tensor of kv_indices' dtype on q's device")
        if extra_indptr.numel() != t_count + 1:
            raise ValueError("extra_indptr must have T + 1 entries")
        if not (torch.is_tensor(extra_kv) and extra_kv.device == q.device):
            raise ValueError("extra_kv must be on q's device")
        ekv_ptr, en_rec, epitch = _record_pool(extra_kv)
    if attn_sink is not None and not (torch.is_tensor(attn_sink) and attn_sink.dtype == torch.float32
                                      and attn_sink.device == q.device and attn_sink.ndim == 1
                                      and attn_sink.numel() == heads and attn_sink.is_contiguous()):
        raise ValueError("attn_sink must be a contiguous float32 [H] tensor on q's device")
    if not (torch.is_tensor(kv_cache) and kv_cache.device == q.device):
        raise ValueError("kv cache must be on q's device")
    kv_ptr, n_rec, pitch = _record_pool(kv_cache)
    if out is None:
        out = torch.empty((t_count, heads, KV_LORA_RANK), dtype=torch.bfloat16, device=q.device)
    else:
        if not (out.dtype == torch.bfloat16 and out.device == q.device and out.ndim == 3
                and out.shape[0] == t_count and out.shape[1] == heads and out.shape[2] >= KV_LORA_RANK
                and out.stride(2) == 1):
            raise ValueError("out must be bf16 [T, H, >= 512] with stride(2) == 1 on q's device")
    lse = torch.empty((t_count, heads), dtype=torch.float32, device=q.device) if return_lse else None
    flags = (FLAG_HAS_INVALID if has_invalid else 0) | (FLAG_RETURN_LSE if return_lse else 0)
    if kv_indices.dtype == torch.int64:
        flags |= FLAG_INDEX_I64
    if not 0 <= chunk_tiles <= MAX_CHUNK_TILES:
        raise ValueError(f"chunk_tiles must be in 0 .. {MAX_CHUNK_TILES}")
    flags |= chunk_tiles << CHUNK_SHIFT
    L = lib()
    dev = q.device.index if q.device.index is not None else torch.cuda.current_device()
    with torch.cuda.device(dev):
        total_nnz = kv_indices.numel() + (extra_indices.numel() if use_extra else 0)
        ws_ptr, ws_bytes, workspace = _fwd_workspace(L, q, t_count, heads, total_nnz, flags, workspace)
        if use_extra or attn_sink is not None:
            st = L.mla_sparse_fwd_ex(
                q.data_ptr(), t_count, heads, q.stride(0), q.stride(1),
                kv_ptr, n_rec, pitch,
                kv_indptr.data_ptr(), kv_indices.data_ptr() if kv_indices.numel() else None, kv_indices.numel(),
                attn_sink.data_ptr() if attn_sink is not None else None,
                ekv_ptr if use_extra else None, en_rec if use_extra else 0, epitch if use_extra else RECORD_BYTES,
                extra_indptr.data_ptr() if use_extra else None,
                extra_indices.data_ptr() if use_extra and extra_indices.numel() else None,
                extra_indices.numel() if use_extra else 0,
                float(softmax_scale), flags,
                out.data_ptr(), out.stride(0), out.stride(1),
                lse.data_ptr() if lse is not None else None,
                ws_ptr, ws_bytes, _stream(q.device))
        else:
            st = L.mla_sparse_fwd(
                q.data_ptr(), t_count, heads, q.stride(0), q.stride(1),
                kv_ptr, n_rec, pitch,
                kv_indptr.data_ptr(), kv_indices.data_ptr() if kv_indices.numel() else None, kv_indices.numel(),
                float(softmax_scale), flags,
                out.data_ptr(), out.stride(0), out.stride(1),
                lse.data_ptr() if lse is not None else None,
                ws_ptr, ws_bytes, _stream(q.device))
    _check(st)
    return out, lse


def sparse_fwd_v_up_proj(q, kv_cache, kv_indptr, kv_indices, softmax_scale, w_uv_prepared, *, gate=None,
                         has_invalid=False, out=None, v_out=None, return_lse=False, chunk_tiles=0, workspace=None):
    """sparse_fwd followed by the gated W_UV up-projection on prepared
    weights (mla_sparse_fwd_v_up_proj) -> (v_out [T, H, 128] bf16, out, lse
    or None).  Bit for bit what sparse_fwd then v_up_proj(prepared=True)
    return; a call that splits merges and projects in one launch.

    w_uv_prepared: prepare_w_uv's result for W_UV [H, 512, 128]; gate bf16
    [T, H * 128] with a contiguous last dim, or None; out optional bf16
    [T, H, >= 512] (16-byte aligned rows, strides multiples of 8); v_out
    optional bf16 [T, H, >= 128].
    """
    t_count, heads = _fwd_query_and_lists(q, kv_indptr, kv_indices)
    dev = q.device
    if not (torch.is_tensor(w_uv_prepared) and w_uv_prepared.dtype == torch.bfloat16 and w_uv_prepared.device == dev
            and tuple(w_uv_prepared.shape) == (heads, KV_LORA_RANK, V_HEAD_DIM) and w_uv_prepared.is_contiguous()):
        raise ValueError(f"w_uv_prepared must be prepare_w_uv's bf16 [{heads}, 512, 128] result on q's device")
    if gate is not None and not (torch.is_tensor(gate) and gate.dtype == torch.bfloat16 and gate.device == dev
                                 and tuple(gate.shape) == (t_count, heads * V_HEAD_DIM) and gate.stride(1) == 1):
        raise ValueError(f"gate must be bf16 [{t_count}, {heads * V_HEAD_DIM}] with a contiguous last dim")
    if not (torch.is_tensor(kv_cache) and kv_cache.device == dev):
        raise ValueError("kv cache must be on q's device")
    kv_ptr, n_rec, pitch = _record_pool(kv_cache)
    if out is None:
        out = torch.empty((t_count, heads, KV_LORA_RANK), dtype=torch.bfloat16, device=dev)
    elif not (out.dtype == torch.bfloat16 and out.device == dev and out.ndim == 3 and out.shape[0] == t_count
              and out.shape[1] == heads and out.shape[2] >= KV_LORA_RANK and out.stride(2) == 1):
        raise ValueError("out must be bf16 [T, H, >= 512] with stride(2) == 1 on q's device")
    if v_out is None:
        v_out = torch.empty((t_count, heads, V_HEAD_DIM), dtype=torch.bfloat16, device=dev)
    elif not (v_out.dtype == torch.bfloat16 and v_out.device == dev and v_out.ndim == 3
              and v_out.shape[0] == t_count and v_out.shape[1] == heads and v_out.shape[2] >= V_HEAD_DIM
              and v_out.stride(2) == 1):
        raise ValueError("v_out must be bf16 [T, H, >= 128] with a contiguous last dim on q's device")
    lse = torch.empty((t_count, heads), dtype=torch.float32, device=dev) if return_lse else None
    flags = (FLAG_HAS_INVALID if has_invalid else 0) | (FLAG_RETURN_LSE if return_lse else 0)
    if kv_indices.dtype == torch.int64:
        flags |= FLAG_INDEX_I64
    if not 0 <= chunk_tiles <= MAX_CHUNK_TILES:
        raise ValueError(f"chunk_tiles must be in 0 .. {MAX_CHUNK_TILES}")
    flags |= chunk_tiles << CHUNK_SHIFT
    L = lib()
    with torch.cuda.device(dev):
        ws_ptr, ws_bytes, workspace = _fwd_workspace(L, q, t_count, heads, kv_indices.numel(), flags, workspace)
        st = L.mla_sparse_fwd_v_up_proj(
            q.data_ptr(), t_count, heads, q.stride(0), q.stride(1), kv_ptr, n_rec, pitch,
            kv_indptr.data_ptr(), kv_indices.data_ptr() if kv_indices.numel() else None, kv_indices.numel(),
            float(softmax_scale), flags, out.data_ptr(), out.stride(0), out.stride(1),
            lse.data_ptr() if lse is not None else None, w_uv_prepared.data_ptr(),
            gate.data_ptr() if gate is not None else None, gate.stride(0) if gate is not None else 0,
            v_out.data_ptr(), v_out.stride(0), v_out.stride(1), ws_ptr, ws_bytes, _stream(dev))
    _check(st)
    return v_out, out, lse


def cache_insert(kv_c, k_pe, slot_mapping, kv_cache):
    """Quantize [kv_c | k_pe] of each token into its record (in place).

    kv_c [Tn, 512] bf16 (stride(1) == 1); k_pe [Tn, 64] or [Tn, 1, 64] bf16;
    slot_mapping [Tn] int64 (negative = skip); kv_cache a record pool view.
    """
    if not (torch.is_tensor(kv_c) and kv_c.is_cuda and kv_c.dtype == torch.bfloat16 and kv_c.ndim == 2
            and kv_c.shape[1] == KV_LORA_RANK and kv_c.stride(1) == 1):
        raise ValueError("kv_c must be a CUDA bf16 [T, 512] tensor with stride(1) == 1")
    n = kv_c.shape[0]
    if not (torch.is_tensor(k_pe) and k_pe.dtype == torch.bfloat16 and k_pe.device == kv_c.device
            and k_pe.shape[0] == n):
        raise ValueError("k_pe must be bf16 [T, 64] or [T, 1, 64] on kv_c's device")
    if k_pe.numel() != n * QK_ROPE_HEAD_DIM:
        raise ValueError("k_pe must hold 64 values per token")
    k_pe2 = k_pe.reshape(n, QK_ROPE_HEAD_DIM)
    if k_pe2.shape[1] != QK_ROPE_HEAD_DIM or k_pe2.stride(1) != 1:
        raise ValueError("k_pe rows must be 64 contiguous bf16 values")
    if not (torch.is_tensor(slot_mapping) and slot_mapping.dtype == torch.int64 and slot_mapping.ndim == 1
            and slot_mapping.numel() == n and slot_mapping.is_contiguous()
            and slot_mapping.device == kv_c.device):
        raise ValueError("slot_mapping must be a contiguous int64 [T] tensor on kv_c's device")
    if not (torch.is_tensor(kv_cache) and kv_cache.device == kv_c.device):
        raise ValueError("kv cache must be on kv_c's device")
    kv_ptr, n_rec, pitch = _record_pool(kv_cache)
    L = lib()
    with torch.cuda.device(kv_c.device):
        st = L.mla_cache_insert(kv_c.data_ptr(), kv_c.stride(0), k_pe2.data_ptr(), k_pe2.stride(0),
                                slot_mapping.data_ptr(), n, kv_ptr, n_rec, pitch, _stream(kv_c.device))
    _check(st)
    return kv_cache


def _bf16_rows(x, name, shape_tail, device):
    """Check a CUDA bf16 tensor whose last dim is contiguous; returns it."""
    if not (torch.is_tensor(x) and x.dtype == torch.bfloat16 and x.device == device):
        raise ValueError(f"{name} must be a bf16 tensor on {device}")
    if tuple(x.shape[1:]) != tuple(shape_tail) or x.stride(-1) != 1:
        raise ValueError(f"{name} must be [B, {', '.join(map(str, shape_tail))}] with a contiguous last dim")
    return x


def decode_q_concat_insert(ql_nope, q_pe, kv_c_normed, k_pe, kv_cache, slot_mapping, *, positions=None,
                           cos_sin_cache=None, mqa_q=None):
    """MLA decode epilogue in one launch -> mqa_q [B, H, 576] bf16.

    mqa_q = [ql_nope | q_pe], and [kv_c_normed | k_pe] is inserted into the
    fp8_ds_mla cache at slot_mapping (negative = skip), with GPT-J RoPE on
    q_pe and k_pe when ``positions`` [B] int64 and the fp32
    ``cos_sin_cache`` [max_position, 64] are given.  ql_nope [B, H, 512],
    q_pe [B, H, 64], kv_c_normed [B, 512], k_pe [B, 64] or [B, 1, 64], all
    bf16 with a contiguous last dim.
    """
    if not (torch.is_tensor(ql_nope) and ql_nope.is_cuda and ql_nope.ndim == 3):
        raise ValueError("ql_nope must be a CUDA bf16 tensor [B, H, 512]")
    dev = ql_nope.device
    b, heads = ql_nope.shape[0], ql_nope.shape[1]
    if not 1 <= heads <= MAX_EPILOGUE_HEADS:
        raise ValueError(f"{heads} heads: 1 .. {MAX_EPILOGUE_HEADS} are served")
    _bf16_rows(ql_nope, "ql_nope", (heads, KV_LORA_RANK), dev)
    _bf16_rows(q_pe, "q_pe", (heads, QK_ROPE_HEAD_DIM), dev)
    _bf16_rows(kv_c_normed, "kv_c_normed", (KV_LORA_RANK,), dev)
    if not (torch.is_tensor(k_pe) and k_pe.numel() == b * QK_ROPE_HEAD_DIM):
        raise ValueError("k_pe must hold 64 values per token")
    k_pe2 = _bf16_rows(k_pe.reshape(b, QK_ROPE_HEAD_DIM), "k_pe", (QK_ROPE_HEAD_DIM,), dev)
    for name, x in (("q_pe", q_pe), ("kv_c_normed", kv_c_normed), ("k_pe", k_pe2)):
        if x.shape[0] != b:
            raise ValueError(f"{name} must have {b} tokens")
    if not (torch.is_tensor(slot_mapping) and slot_mapping.dtype == torch.int64 and slot_mapping.ndim == 1
            and slot_mapping.numel() == b and slot_mapping.is_contiguous() and slot_mapping.device == dev):
        raise ValueError("slot_mapping must be a contiguous int64 [B] tensor on ql_nope's device")
    if (positions is None) != (cos_sin_cache is None):
        raise ValueError("positions and cos_sin_cache come together")
    max_position = 0
    if positions is not None:
        if not (positions.dtype == torch.int64 and positions.ndim == 1 and positions.numel() == b
                and positions.is_contiguous() and positions.device == dev):
            raise ValueError("positions must be a contiguous int64 [B] tensor on ql_nope's device")
        if not (cos_sin_cache.dtype == torch.float32 and cos_sin_cache.ndim == 2
                and cos_sin_cache.shape[1] == QK_ROPE_HEAD_DIM and cos_sin_cache.is_contiguous()
                and cos_sin_cache.device == dev):
            raise ValueError("cos_sin_cache must be a contiguous float32 [max_position, 64] tensor")
        max_position = cos_sin_cache.shape[0]
    if mqa_q is None:
        mqa_q = torch.empty((b, heads, KV_LORA_RANK + QK_ROPE_HEAD_DIM), dtype=torch.bfloat16, device=dev)
    else:
        _bf16_rows(mqa_q, "mqa_q", (heads, KV_LORA_RANK + QK_ROPE_HEAD_DIM), dev)
        if mqa_q.shape[0] != b:
            raise ValueError(f"mqa_q must have {b} tokens")
    if not (torch.is_tensor(kv_cache) and kv_cache.device == dev):
        raise ValueError("kv cache must be on ql_nope's device")
    kv_ptr, n_rec, pitch = _record_pool(kv_cache)
    L = lib()
    with torch.cuda.device(dev):
        st = L.mla_decode_q_concat_insert(
            ql_nope.data_ptr(), ql_nope.stride(0), ql_nope.stride(1),
            q_pe.data_ptr(), q_pe.stride(0), q_pe.stride(1),
            kv_c_normed.data_ptr(), kv_c_normed.stride(0), k_pe2.data_ptr(), k_pe2.stride(0),
            slot_mapping.data_ptr(), b, heads,
            positions.data_ptr() if positions is not None else None,
            cos_sin_cache.data_ptr() if cos_sin_cache is not None else None, max_position,
            mqa_q.data_ptr(), mqa_q.stride(0), mqa_q.stride(1),
            kv_ptr, n_rec, pitch, _stream(dev))
    _check(st)
    return mqa_q


def gather_upconvert(kv_cache, block_table, cu_seq_lens, num_tokens, *, seq_starts=None, block_size=None,
                     dst=None):
    """Gather a context chunk through the block table -> bf16 [num_tokens, 576].

    kv_cache: the paged pool [num_blocks, block_size, 656] (or a flat record
    view with ``block_size`` given); block_table int32 [B, W];
    cu_seq_lens int32 [B + 1] (the chunk's workspace rows); seq_starts int32
    [B] or None.  Row cu[r] + j holds context position seq_starts[r] + j of
    request r, as [dequantized latent | rope] in bf16; rows with no valid
    source are zero.
    """
    if not (torch.is_tensor(kv_cache) and kv_cache.is_cuda):
        raise ValueError("kv cache must be a CUDA tensor")
    dev = kv_cache.device
    if block_size is None:
        if kv_cache.ndim != 3:
            raise ValueError("pass block_size for a kv cache that is not [num_blocks, block_size, 656]")
        block_size = kv_cache.shape[1]
    kv_ptr, n_rec, pitch = _record_pool(kv_cache)
    if not (torch.is_tensor(block_table) and block_table.dtype == torch.int32 and block_table.ndim == 2
            and block_table.device == dev and block_table.stride(1) == 1):
        raise ValueError("block_table must be an int32 [B, W] tensor with contiguous rows on the cache's device")
    batch = block_table.shape[0]
    for name, x, n in (("cu_seq_lens", cu_seq_lens, batch + 1), ("seq_starts", seq_starts, batch)):
        if x is None and name == "seq_starts":
            continue
        if not (torch.is_tensor(x) and x.dtype == torch.int32 and x.ndim == 1 and x.numel() == n
                and x.is_contiguous() and x.device == dev):
            raise ValueError(f"{name} must be a contiguous int32 [{n}] tensor on the cache's device")
    if dst is None:
        dst = torch.empty((num_tokens, KV_LORA_RANK + QK_ROPE_HEAD_DIM), dtype=torch.bfloat16, device=dev)
    elif not (dst.dtype == torch.bfloat16 and dst.ndim == 2 and dst.shape[0] == num_tokens
              and dst.shape[1] == KV_LORA_RANK + QK_ROPE_HEAD_DIM and dst.stride(1) == 1 and dst.device == dev):
        raise ValueError("dst must be bf16 [num_tokens, 576] with contiguous rows on the cache's device")
    L = lib()
    with torch.cuda.device(dev):
        st = L.mla_gather_upconvert(
            kv_ptr, n_rec, pitch, int(block_size),
            block_table.data_ptr() if block_table.numel() else None, block_table.stride(0), block_table.shape[1],
            cu_seq_lens.data_ptr(), seq_starts.data_ptr() if seq_starts is not None else None, batch,
            num_tokens, dst.data_ptr() if num_tokens else None, dst.stride(0), _stream(dev))
    _check(st)
    return dst


V_HEAD_DIM = 128


def prepare_w_uv(w_uv):
    """W_UV bf16 [H, 512, 128] -> the same values in the up-projection's
    fragment order (a bf16 tensor of the same shape whose layout is internal:
    pass it to v_up_proj with prepared=True).  Done once, after loading."""
    if not (torch.is_tensor(w_uv) and w_uv.is_cuda and w_uv.dtype == torch.bfloat16 and w_uv.ndim == 3
            and tuple(w_uv.shape[1:]) == (KV_LORA_RANK, V_HEAD_DIM) and w_uv.is_contiguous()):
        raise ValueError("w_uv must be a contiguous CUDA bf16 [H, 512, 128] tensor")
    heads = w_uv.shape[0]
    if not 1 <= heads <= MAX_EPILOGUE_HEADS:
        raise ValueError(f"{heads} heads: 1 .. {MAX_EPILOGUE_HEADS} are served")
    dev = w_uv.device
    prepared = torch.empty_like(w_uv)
    with torch.cuda.device(dev):
        st = lib().mla_v_up_proj_prepare_weights(w_uv.data_ptr(), heads, prepared.data_ptr(), _stream(dev))
    _check(st)
    return prepared


def v_up_proj(latent, w_uv, *, gate=None, out=None, prepared=False):
    """out[t, h, :] = latent[t, h, :512] @ w_uv[h] (times sigmoid(gate)) -> bf16 [T, H, 128].

    latent: bf16 [T, H, >= 512] (e.g. sparse_fwd's out) with a contiguous last
    dim, 16-byte aligned rows; w_uv: bf16 [H, 512, 128] contiguous (or, with
    prepared=True, prepare_w_uv's result for it); gate: bf16 [T, H * 128]
    with a contiguous last dim, or None.
    """
    if not (torch.is_tensor(latent) and latent.is_cuda and latent.dtype == torch.bfloat16 and latent.ndim == 3
            and latent.shape[2] >= KV_LORA_RANK and latent.stride(2) == 1):
        raise ValueError("latent must be a CUDA bf16 [T, H, >= 512] tensor with a contiguous last dim")
    dev = latent.device
    t_count, heads = latent.shape[0], latent.shape[1]
    if not 1 <= heads <= MAX_EPILOGUE_HEADS:
        raise ValueError(f"{heads} heads: 1 .. {MAX_EPILOGUE_HEADS} are served")
    if not (torch.is_tensor(w_uv) and w_uv.dtype == torch.bfloat16 and w_uv.device == dev
            and tuple(w_uv.shape) == (heads, KV_LORA_RANK, V_HEAD_DIM) and w_uv.is_contiguous()):
        raise ValueError(f"w_uv must be a contiguous bf16 [{heads}, 512, 128] tensor on latent's device")
    if gate is not None and not (torch.is_tensor(gate) and gate.dtype == torch.bfloat16 and gate.device == dev
                                 and tuple(gate.shape) == (t_count, heads * V_HEAD_DIM) and gate.stride(1) == 1):
        raise ValueError(f"gate must be bf16 [{t_count}, {heads * V_HEAD_DIM}] with a contiguous last dim")
    if out is None:
        out = torch.empty((t_count, heads, V_HEAD_DIM), dtype=torch.bfloat16, device=dev)
    elif not (out.dtype == torch.bfloat16 and out.device == dev and out.ndim == 3 and out.shape[0] == t_count
              and out.shape[1] == heads and out.shape[2] >= V_HEAD_DIM and out.stride(2) == 1):
        raise ValueError("out must be bf16 [T, H, >= 128] with a contiguous last dim")
    L = lib()
    with torch.cuda.device(dev):
        fn = L.mla_v_up_proj_prepared if prepared else L.mla_v_up_proj
        st = fn(latent.data_ptr(), latent.stride(0), latent.stride(1), w_uv.data_ptr(),
                gate.data_ptr() if gate is not None else None, gate.stride(0) if gate is not None else 0,
                t_count, heads, out.data_ptr(), out.stride(0), out.stride(1), _stream(dev))
    _check(st)
    return out


def _key_concat_args(q, k_nope, k_pe, kv_c_normed, slot_mapping, positions, cos_sin_cache, k_out):
    """Shape, dtype and device checks of key_concat_insert's tensors, on
    k_nope's device (any device, so the checks run without a GPU too).
    Every tensor the kernel reads or writes per token must hold exactly Tp
    tokens.  Returns (k_pe as [Tp, 64], max_position)."""
    if not (torch.is_tensor(k_nope) and k_nope.ndim == 3):
        raise ValueError("k_nope must be a bf16 tensor [Tp, H, nope]")
    dev = k_nope.device
    tp, heads, nope = k_nope.shape
    if not 1 <= heads <= MAX_EPILOGUE_HEADS:
        raise ValueError(f"{heads} heads: 1 .. {MAX_EPILOGUE_HEADS} are served")
    _bf16_rows(k_nope, "k_nope", (heads, nope), dev)
    if q is not None:
        _bf16_rows(q, "q", (heads, nope + QK_ROPE_HEAD_DIM), dev)
        if q.shape[0] != tp:
            raise ValueError(f"q must have {tp} tokens")
    elif positions is not None:
        raise ValueError("q is needed with RoPE (it is rotated in place)")
    _bf16_rows(kv_c_normed, "kv_c_normed", (KV_LORA_RANK,), dev)
    if not (torch.is_tensor(k_pe) and k_pe.numel() == tp * QK_ROPE_HEAD_DIM):
        raise ValueError("k_pe must hold 64 values per token")
    k_pe2 = _bf16_rows(k_pe.reshape(tp, QK_ROPE_HEAD_DIM), "k_pe", (QK_ROPE_HEAD_DIM,), dev)
    if kv_c_normed.shape[0] != tp:
        raise ValueError(f"kv_c_normed must have {tp} tokens")
    if not (torch.is_tensor(slot_mapping) and slot_mapping.dtype == torch.int64 and slot_mapping.ndim == 1
            and slot_mapping.numel() == tp and slot_mapping.is_contiguous() and slot_mapping.device == dev):
        raise ValueError("slot_mapping must be a contiguous int64 [Tp] tensor on k_nope's device")
    if (positions is None) != (cos_sin_cache is None):
        raise ValueError("positions and cos_sin_cache come together")
    max_position = 0
    if positions is not None:
        if not (positions.dtype == torch.int64 and positions.ndim == 1 and positions.numel() == tp
                and positions.is_contiguous() and positions.device == dev):
            raise ValueError("positions must be a contiguous int64 [Tp] tensor on k_nope's device")
        if not (cos_sin_cache.dtype == torch.float32 and cos_sin_cache.ndim == 2
                and cos_sin_cache.shape[1] == QK_ROPE_HEAD_DIM and cos_sin_cache.is_contiguous()
                and cos_sin_cache.device == dev):
            raise ValueError("cos_sin_cache must be a contiguous float32 [max_position, 64] tensor")
        max_position = cos_sin_cache.shape[0]
    if k_out is not None:
        _bf16_rows(k_out, "k_out", (heads, nope + QK_ROPE_HEAD_DIM), dev)
        if k_out.shape[0] != tp:
            raise ValueError(f"k_out must have {tp} tokens (got {k_out.shape[0]})")
    return k_pe2, max_position


def key_concat_insert(q, k_nope, k_pe, kv_c_normed, kv_cache, slot_mapping, *, positions=None,
                      cos_sin_cache=None, k_out=None):
    """MLA prefill epilogue in one launch -> k_out [Tp, H, nope + 64] bf16.

    k_out = [k_nope | k_pe] per head, [kv_c_normed | k_pe] inserted into the
    fp8_ds_mla cache at slot_mapping (negative = skip); with ``positions`` /
    ``cos_sin_cache`` GPT-J RoPE is applied to k_pe (in k_out and the
    record) and to q[..., nope:] in place.  q [Tp, H, nope + 64] (may be
    None without RoPE), k_nope [Tp, H, nope], k_pe [Tp, 64] or [Tp, 1, 64],
    kv_c_normed [Tp, 512]; bf16 with a contiguous last dim.
    """
    if not (torch.is_tensor(k_nope) and k_nope.is_cuda and k_nope.ndim == 3):
        raise ValueError("k_nope must be a CUDA bf16 tensor [Tp, H, nope]")
    dev = k_nope.device
    tp, heads, nope = k_nope.shape
    k_pe2, max_position = _key_concat_args(q, k_nope, k_pe, kv_c_normed, slot_mapping, positions,
                                           cos_sin_cache, k_out)
    if k_out is None:
        k_out = torch.empty((tp, heads, nope + QK_ROPE_HEAD_DIM), dtype=torch.bfloat16, device=dev)
    if not (torch.is_tensor(kv_cache) and kv_cache.device == dev):
        raise ValueError("kv cache must be on k_nope's device")
    kv_ptr, n_rec, pitch = _record_pool(kv_cache)
    L = lib()
    with torch.cuda.device(dev):
        st = L.mla_prefill_key_concat_insert(
            q.data_ptr() if q is not None else None, q.stride(0) if q is not None else 0,
            q.stride(1) if q is not None else 0, nope,
            k_nope.data_ptr(), k_nope.stride(0), k_nope.stride(1),
            kv_c_normed.data_ptr(), kv_c_normed.stride(0), k_pe2.data_ptr(), k_pe2.stride(0),
            slot_mapping.data_ptr(), tp, heads,
            positions.data_ptr() if positions is not None else None,
            cos_sin_cache.data_ptr() if cos_sin_cache is not None else None, max_position,
            k_out.data_ptr(), k_out.stride(0), k_out.stride(1),
            kv_ptr, n_rec, pitch, _stream(dev))
    _check(st)
    return k_out
