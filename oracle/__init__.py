"""CPU oracle for the sparse absorbed-MLA forward and the fp8_ds_mla cache insert.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, links or
calls this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` do.  It shares no code with the HIP
library (no kernels, headers, tables or helpers), and it never consumes a
value produced by the HIP path.

Everything here is plain numpy in float64 (float32 only where the pages fix
the arithmetic of the insert writer), written from the definitions on the
vLLM API pages:

* ``vllm.models.kimi_k3.amd.ops.flydsl_sparse_mla`` (module docstring, and
  the ``flydsl_sparse_mla_fp8ds_fwd`` / ``..._supported`` docstrings): the
  656-byte record, the CSR slot lists, masking of negative ids, the
  empty-row convention and the natural-log LSE;
* ``vllm.models.kimi_k3.nvidia.ops.fused_mla_key_concat_kv_cache``
  (``fused_mla_key_concat_ds_mla_insert`` docstring): the self-scaling
  record writer with per-128-tile dynamic fp8 scales;
* ``vllm.models.kimi_k3.nvidia.mla`` (``_compute_prefill_context`` and
  ``merge_attn_states`` call): combining attention partials by their LSEs;
* ``fused_mla_decode_q_concat_kv_cache_insert`` (same fused_mla_key_concat
  page) and ``MultiHeadLatentAttention`` on the ``vllm.models.kimi_k3.nvidia.mla``
  page: the decode epilogue's query concat and GPT-J RoPE in float32;
* ``cp_gather_and_upconvert_fp8_kv_cache`` as ``_gather_context_latent``
  calls it (``vllm.models.kimi_k3.nvidia.mla`` page): a context chunk's
  records, through the block table, into a bf16 workspace;
* ``_v_up_proj``, ``process_weights_after_loading`` and the gate of
  ``forward`` (``vllm.models.kimi_k3.nvidia.mla`` page): the W_UV
  up-projection and the sigmoid gate.

Modules:
  e4m3       OCP float8 E4M3 ("fn") decode table and saturating RNE encoder.
  records    656-byte record encode (the insert writer) and decode.
  attention  Sparse attention forward over records, and the LSE merge.
  epilogue   Decode and prefill epilogues: query / key concat, GPT-J RoPE,
             record insert.
  gather     Context gather through the block table, upconverted to bf16.
  value      W_UV up-projection of the latent output, with the sigmoid gate.

Parity pins for every function live in ``tests/test_oracle_*.py``.
"""

from .e4m3 import E4M3_MAX, decode_table, e4m3_decode, e4m3_encode  # noqa: F401
from .records import (  # noqa: F401
    RECORD_BYTES,
    decode_records,
    encode_records,
    insert_records,
)
from .attention import merge_partials, sparse_fwd  # noqa: F401
from .epilogue import decode_q_concat_insert, f32_to_bf16_bits, key_concat_insert, rope_gptj_bits  # noqa: F401
from .gather import gather_upconvert, upconvert_records  # noqa: F401
from .value import v_up_proj  # noqa: F401
