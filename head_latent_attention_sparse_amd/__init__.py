"""Sparse absorbed-MLA forward over an fp8_ds_mla latent cache, for MI355X (gfx950).

The computation lives in libmla.so (hand-written HIP kernels behind the C
ABI of include/mla.h); this package is its thin Python binding.
"""

from .ops import (  # noqa: F401
    FLAG_HAS_INVALID,
    FLAG_INDEX_I64,
    FLAG_RETURN_LSE,
    KV_LORA_RANK,
    MAX_HEADS,
    MAX_CHUNK_TILES,
    MAX_EPILOGUE_HEADS,
    QK_ROPE_HEAD_DIM,
    RECORD_BYTES,
    MlaError,
    cache_insert,
    decode_q_concat_insert,
    gather_upconvert,
    key_concat_insert,
    lib,
    prepare_w_uv,
    split_workgroups,
    sparse_fwd,
    sparse_fwd_v_up_proj,
    v_up_proj,
)
