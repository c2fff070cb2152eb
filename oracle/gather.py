"""Gather + upconvert of a context chunk's records into a bf16 workspace.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows ``cp_gather_and_upconvert_fp8_kv_cache`` as the
``vllm.models.kimi_k3.nvidia.mla`` page calls it in ``_gather_context_latent``
(``dst = workspace[:toks]``, ``workspace_starts = chunk.cu_seq_lens``,
``seq_starts = chunk.starts``, a block table per request).

Readings taken where the page gives only the call:
workspace row ``cu[r] + j`` holds context position ``starts[r] + j`` of
request r for ``j < cu[r+1] - cu[r]``; position p lives in record
``block_table[r][p // block_size] * block_size + p % block_size``; the row is
``[latent | rope]`` in the model dtype, bf16, with
``latent[d] = bf16(f32(E4M3(code[d])) * scale[d // 128])`` (one float32
product, then round to nearest even) and the rope bits copied; rows without
a valid source are zero.
"""

import numpy as np

from .e4m3 import e4m3_decode
from .epilogue import f32_to_bf16_bits
from .records import LATENT, ROPE, ROPE_OFF, SCALE_OFF, TILE


def upconvert_records(records):
    """uint8 [n, 656] records -> uint16 [n, 576] bf16 rows [latent | rope]."""
    rec = np.asarray(records, dtype=np.uint8).reshape(-1, 656)
    n = rec.shape[0]
    vals = e4m3_decode(rec[:, :LATENT]).astype(np.float32).reshape(n, 4, TILE)  # exact
    scale = np.ascontiguousarray(rec[:, SCALE_OFF:ROPE_OFF]).view("<f4").astype(np.float32)  # [n, 4]
    lat = f32_to_bf16_bits((vals * scale[:, :, None]).reshape(n, LATENT))  # float32 product, then bf16
    out = np.empty((n, LATENT + ROPE), dtype=np.uint16)
    out[:, :LATENT] = lat
    out[:, LATENT:] = np.ascontiguousarray(rec[:, ROPE_OFF:]).view("<u2")
    return out


def gather_upconvert(pool, block_size, block_table, cu_seq_lens, seq_starts, num_tokens):
    """bf16 bits uint16 [num_tokens, 576] of the gathered chunk.

    pool uint8 [N, 656] (flat records); block_table int [B, W];
    cu_seq_lens int [B + 1]; seq_starts int [B] or None.
    """
    pool = np.asarray(pool, dtype=np.uint8).reshape(-1, 656)
    bt = np.asarray(block_table, dtype=np.int64).reshape(len(cu_seq_lens) - 1, -1)
    cu = np.asarray(cu_seq_lens, dtype=np.int64)
    out = np.zeros((num_tokens, LATENT + ROPE), dtype=np.uint16)
    for r in range(len(cu) - 1):
        j = np.arange(max(cu[r + 1] - cu[r], 0))
        rows = cu[r] + j
        pos = (0 if seq_starts is None else int(seq_starts[r])) + j
        bi = pos // block_size
        ok = (rows >= 0) & (rows < num_tokens) & (pos >= 0) & (bi < bt.shape[1])
        blk = np.where(ok, bt[r, np.clip(bi, 0, max(bt.shape[1] - 1, 0))] if bt.shape[1] else -1, -1)
        slot = blk * block_size + pos % block_size
        ok &= (blk >= 0) & (slot < pool.shape[0])
        if ok.any():
            out[rows[ok]] = upconvert_records(pool[slot[ok]])
    return out
