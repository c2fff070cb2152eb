"""The MLA decode epilogue: query concat, GPT-J RoPE, and the record insert.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows ``fused_mla_decode_q_concat_kv_cache_insert`` with ``ds_mla=True``
on the vLLM API page
``vllm.models.kimi_k3.nvidia.ops.fused_mla_key_concat_kv_cache``: the
latent decode query is ``mqa_q = [ql_nope | q_pe]`` in bf16, and
``[kv_c_normed | k_pe]`` goes into the 656-byte cache at ``slot_mapping``.
The optional ``positions`` / ``cos_sin_cache`` pair turns on GPT-J-style
RoPE (module docstring of that page), and on the ``vllm.models.kimi_k3.nvidia.mla``
page ``MultiHeadLatentAttention`` builds its rotary table in float32 with
``is_neox_style=False`` and hands it to the fused epilogues, which read it in
float32 and do the RoPE arithmetic in float32.

Readings taken where the pages leave it open: the
table row of a position holds the 32 cosines then the 32 sines of the 32
rotation pairs; GPT-J style pairs adjacent values (2i, 2i+1); each product
and each sum is one float32 rounding (no fused multiply-add), and the
result is rounded to bf16 to nearest even.  RoPE applies to q_pe of every
head and to k_pe before it is stored.
"""

import numpy as np

from .records import LATENT, ROPE, bf16_bits_to_f32, encode_records

HALF = ROPE // 2


def f32_to_bf16_bits(x):
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs;
    an overflow rounds to infinity as the rule gives)."""
    b = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def rope_gptj_bits(x_bits, cos_sin_rows):
    """GPT-J RoPE of bf16 rope vectors.

    x_bits: uint16 [..., 64] bf16 patterns; cos_sin_rows: float32 [..., 64]
    (broadcast against x_bits), cosines in [:32] and sines in [32:].  For
    pair i, (x0, x1) = (x[2i], x[2i+1]):
        y[2i] = x0 * c - x1 * s,   y[2i+1] = x1 * c + x0 * s
    with numpy float32 operations (one rounding each).  Returns uint16 [..., 64].
    """
    x = bf16_bits_to_f32(x_bits)
    cs = np.asarray(cos_sin_rows, dtype=np.float32)
    c, s = cs[..., :HALF], cs[..., HALF:]
    x0, x1 = x[..., 0::2], x[..., 1::2]
    y = np.empty(np.broadcast_shapes(x.shape, cs.shape), dtype=np.float32)
    y[..., 0::2] = x0 * c - x1 * s
    y[..., 1::2] = x1 * c + x0 * s
    return f32_to_bf16_bits(y)


def decode_q_concat_insert(ql_nope_bits, q_pe_bits, kv_c_bits, k_pe_bits, slot_mapping, pool,
                           positions=None, cos_sin_cache=None):
    """(mqa_q bits uint16 [B, H, 576], pool) for one decode step.

    ql_nope_bits uint16 [B, H, 512], q_pe_bits [B, H, 64], kv_c_bits [B, 512],
    k_pe_bits [B, 64]; slot_mapping int64 [B]; pool uint8 [N, 656], written in
    place at slots 0 <= slot < N (others skipped); positions int64 [B] and
    cos_sin_cache float32 [max_position, 64], both or neither (positions
    clamped to [0, max_position), as the library documents).
    """
    ql = np.asarray(ql_nope_bits, dtype=np.uint16)
    qp = np.asarray(q_pe_bits, dtype=np.uint16)
    kp = np.asarray(k_pe_bits, dtype=np.uint16).reshape(-1, ROPE)
    b, h = ql.shape[0], ql.shape[1]
    if positions is not None:
        table = np.asarray(cos_sin_cache, dtype=np.float32)
        pos = np.clip(np.asarray(positions, dtype=np.int64), 0, table.shape[0] - 1)
        rows = table[pos]                                  # [B, 64]
        qp = rope_gptj_bits(qp, rows[:, None, :])
        kp = rope_gptj_bits(kp, rows)
    mqa = np.empty((b, h, LATENT + ROPE), dtype=np.uint16)
    mqa[:, :, :LATENT] = ql
    mqa[:, :, LATENT:] = qp
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = (slots >= 0) & (slots < pool.shape[0])
    if keep.any():
        pool[slots[keep]] = encode_records(np.asarray(kv_c_bits, dtype=np.uint16)[keep], kp[keep])
    return mqa, pool


def key_concat_insert(q_bits, k_nope_bits, kv_c_bits, k_pe_bits, slot_mapping, pool,
                      positions=None, cos_sin_cache=None):
    """(q bits after RoPE, k_out bits uint16 [Tp, H, nope + 64], pool) for one
    prefill step: ``fused_mla_key_concat_ds_mla_insert`` on the
    fused_mla_key_concat_kv_cache page (full key [k_nope | k_pe] for every
    head, q's rope part rotated in place, the latent inserted).

    q_bits uint16 [Tp, H, nope + 64] (or None without RoPE); k_nope_bits
    [Tp, H, nope]; kv_c_bits [Tp, 512]; k_pe_bits [Tp, 64]; the rest as for
    decode_q_concat_insert.
    """
    kn = np.asarray(k_nope_bits, dtype=np.uint16)
    kp = np.asarray(k_pe_bits, dtype=np.uint16).reshape(-1, ROPE)
    tp, h, nope = kn.shape
    q_out = None if q_bits is None else np.array(q_bits, dtype=np.uint16, copy=True)
    if positions is not None:
        table = np.asarray(cos_sin_cache, dtype=np.float32)
        pos = np.clip(np.asarray(positions, dtype=np.int64), 0, table.shape[0] - 1)
        rows = table[pos]
        kp = rope_gptj_bits(kp, rows)
        q_out[:, :, nope:] = rope_gptj_bits(q_out[:, :, nope:], rows[:, None, :])
    k_out = np.empty((tp, h, nope + ROPE), dtype=np.uint16)
    k_out[:, :, :nope] = kn
    k_out[:, :, nope:] = kp[:, None, :]
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = (slots >= 0) & (slots < pool.shape[0])
    if keep.any():
        pool[slots[keep]] = encode_records(np.asarray(kv_c_bits, dtype=np.uint16)[keep], kp[keep])
    return q_out, k_out, pool
