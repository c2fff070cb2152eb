"""656-byte fp8_ds_mla records: the insert writer and the decoder.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Record layout (flydsl_sparse_mla page, module and ``_supported``
docstrings; fused_mla_key_concat_kv_cache page,
``fused_mla_key_concat_ds_mla_insert`` docstring):

    bytes   0 .. 511   latent d = 0..511 as E4M3, one byte each
    bytes 512 .. 527   four float32 scales, tile b covers latent [128b, 128b+128)
    bytes 528 .. 655   64 bf16 rope values

Readings taken where the pages leave the writer open: little-endian
scales and rope; the per-tile scale is the tile's absolute maximum
divided by 448, in float32; codes are
E4M3(x / scale) with a correctly rounded float32 division and the
saturating RNE encoder; an all-zero tile gets scale 0 and codes 0;
records at negative slots are not written.  A slot addresses record
``slot`` of the flat pool, which equals ``block * block_size + offset`` of
an unpadded paged pool (mono/attention/mla page, ``stage_norm``).
"""

import numpy as np

from .e4m3 import E4M3_MAX, e4m3_decode, e4m3_encode

RECORD_BYTES = 656
LATENT = 512
ROPE = 64
TILE = 128
SCALE_OFF = 512
ROPE_OFF = 528


def bf16_bits_to_f32(bits):
    """uint16 bf16 bit patterns -> float32 (exact: bf16 is the top half of f32)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def encode_records(kv_c_bits, k_pe_bits):
    """Encode tokens into records (the ds_mla insert writer).

    kv_c_bits: uint16 [n, 512] bf16 bit patterns of kv_c_normed.
    k_pe_bits: uint16 [n, 64] bf16 bit patterns of k_pe.
    Returns uint8 [n, 656].
    """
    kv_c_bits = np.asarray(kv_c_bits, dtype=np.uint16).reshape(-1, LATENT)
    k_pe_bits = np.asarray(k_pe_bits, dtype=np.uint16).reshape(-1, ROPE)
    n = kv_c_bits.shape[0]
    x = bf16_bits_to_f32(kv_c_bits).reshape(n, 4, TILE)  # float32, exact

    amax = np.max(np.abs(x), axis=2)  # float32 [n, 4]; a max is order-free
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)  # IEEE f32 RNE

    codes = np.zeros((n, 4, TILE), dtype=np.uint8)
    live = scale > 0
    # float32 / float32 in numpy is the correctly rounded IEEE quotient.
    y = np.zeros_like(x)
    np.divide(x, scale[:, :, None], out=y, where=live[:, :, None])
    codes[live] = e4m3_encode(y[live])

    rec = np.zeros((n, RECORD_BYTES), dtype=np.uint8)
    rec[:, :LATENT] = codes.reshape(n, LATENT)
    rec[:, SCALE_OFF:ROPE_OFF] = scale.astype("<f4").view(np.uint8).reshape(n, 16)
    rec[:, ROPE_OFF:] = k_pe_bits.astype("<u2").view(np.uint8).reshape(n, 2 * ROPE)
    return rec


def insert_records(pool, kv_c_bits, k_pe_bits, slot_mapping):
    """Write encoded records into ``pool`` (uint8 [N, 656]) in place.

    Tokens whose slot is negative are skipped; the pool keeps its bytes
    there.  Returns ``pool``.
    """
    slot_mapping = np.asarray(slot_mapping, dtype=np.int64)
    rec = encode_records(kv_c_bits, k_pe_bits)
    keep = slot_mapping >= 0
    pool[slot_mapping[keep]] = rec[keep]
    return pool


def decode_records(records):
    """Records uint8 [n, 656] -> (K float64 [n, 576], V float64 [n, 512]).

    latent[d] = E4M3(code[d]) * scale[d // 128], exact in float64; the key is
    [latent | rope] and the value is the latent alone (the output is 512
    wide on the flydsl_sparse_mla page).
    """
    records = np.asarray(records, dtype=np.uint8).reshape(-1, RECORD_BYTES)
    n = records.shape[0]
    codes = records[:, :LATENT]
    scale = (
        np.ascontiguousarray(records[:, SCALE_OFF:ROPE_OFF]).view("<f4").astype(np.float64)
    )  # [n, 4]
    latent = e4m3_decode(codes).reshape(n, 4, TILE) * scale[:, :, None]
    latent = latent.reshape(n, LATENT)
    rope_bits = np.ascontiguousarray(records[:, ROPE_OFF:]).view("<u2")
    rope = bf16_bits_to_f32(rope_bits).astype(np.float64)
    k = np.concatenate([latent, rope], axis=1)
    return k, latent
