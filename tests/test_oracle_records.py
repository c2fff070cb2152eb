"""Pins for the oracle's record writer and decoder (no GPU).

* a hand-worked record (tests/golden/record_worked.json);
* an independent formulation of the writer through torch's float32 division
  and float8_e4m3fn cast (library routines) on varied data;
* properties the format fixes: the tile maximum codes to +-448, the
  round-trip error bound of a 3-bit mantissa, rope bytes copied verbatim,
  skipped slots untouched, re-inserting is idempotent;
* the decoder against torch's float8 view times the stored scales.
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import RECORD_BYTES, decode_records, encode_records, insert_records
from head_latent_attention_sparse_amd.workloads import bf16_bits


def bf16_from_f32(x):
    return bf16_bits(torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16))


def torch_writer(kv_c_bf16, k_pe_bf16):
    """The writer restated with torch ops (independent of the oracle's codec)."""
    x = kv_c_bf16.to(torch.float32).reshape(-1, 4, 128)
    amax = x.abs().amax(dim=2)
    scale = amax / 448.0  # float32 tensor / python float -> float32 IEEE division
    y = torch.where(scale[:, :, None] > 0, x / scale[:, :, None], torch.zeros_like(x))
    codes = y.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).reshape(-1, 512)
    n = codes.shape[0]
    rec = torch.zeros((n, RECORD_BYTES), dtype=torch.uint8)
    rec[:, :512] = codes
    rec[:, 512:528] = scale.contiguous().view(torch.uint8).reshape(n, 16)
    rec[:, 528:] = k_pe_bf16.reshape(n, 64).contiguous().view(torch.uint8)
    return rec.numpy()


def test_worked_record(golden_dir):
    with open(os.path.join(golden_dir, "record_worked.json")) as f:
        fx = json.load(f)
    x = np.zeros(512, dtype=np.float32)
    for span, v in fx["kv_c_fill"].items():
        a, b = map(int, span.split(":"))
        x[a:b] = v
    for d, v in fx["kv_c_nonzero"]:
        x[d] = v
    rope = 0.25 * np.arange(64, dtype=np.float32) - 8.0
    rec = encode_records(bf16_from_f32(x)[None], bf16_from_f32(rope)[None])[0]

    want = np.zeros(512, dtype=np.uint8)
    for span, c in fx["expected_codes_fill"].items():
        a, b = map(int, span.split(":"))
        want[a:b] = int(c, 16)
    for d, c in fx["expected_codes"]:
        want[d] = int(c, 16)
    assert np.array_equal(rec[:512], want)
    scale_bits = rec[512:528].view("<u4")
    assert [int(s, 16) for s in fx["expected_scale_bits"]] == scale_bits.tolist()
    assert np.array_equal(rec[528:].view("<u2"), bf16_from_f32(rope))


def _random_tokens(seed, n, kind):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((n, 512), generator=g)
    if kind == "std2":
        x = x * 2
    elif kind == "heavy":
        x = x * torch.exp(3 * torch.randn((n, 512), generator=g))
    elif kind == "tiny":  # bf16 subnormal / near-underflow magnitudes
        x = x * 2.0**-128
    elif kind == "huge":
        x = x * 2.0**100
    elif kind == "zero_tiles":
        x[:, 128:256] = 0
        x[::2, :] = 0
    elif kind == "ties":  # values whose scaled form hits E4M3 ties exactly
        x = torch.randint(-64, 65, (n, 512), generator=g).to(torch.float32) * 0.0625
        x[:, ::128] = 448.0 / 8  # amax 56 -> scale 0.125
    kv_c = x.to(torch.bfloat16)
    k_pe = torch.randn((n, 64), generator=g).to(torch.bfloat16)
    return kv_c, k_pe


@pytest.mark.parametrize("kind", ["std1", "std2", "heavy", "tiny", "huge", "zero_tiles", "ties"])
def test_writer_matches_torch_formulation(kind):
    kv_c, k_pe = _random_tokens(7, 512, kind)
    got = encode_records(bf16_bits(kv_c), bf16_bits(k_pe))
    assert np.array_equal(got, torch_writer(kv_c, k_pe))


@pytest.mark.parametrize("kind", ["std1", "heavy"])
def test_writer_properties(kind):
    kv_c, k_pe = _random_tokens(11, 256, kind)
    rec = encode_records(bf16_bits(kv_c), bf16_bits(k_pe))
    x = kv_c.to(torch.float64).numpy().reshape(-1, 4, 128)
    amax = np.abs(x).max(axis=2)
    scale = rec[:, 512:528].copy().view("<f4").astype(np.float64)
    # the stored scale is the float32 quotient amax / 448
    assert np.array_equal(scale, (amax.astype(np.float32) / np.float32(448)).astype(np.float64))
    codes = rec[:, :512].reshape(-1, 4, 128)
    arg = np.abs(x).argmax(axis=2)
    top = np.take_along_axis(codes, arg[:, :, None], axis=2)[..., 0]
    assert np.all((top & 0x7F) == 0x7E)
    # round trip: 3 mantissa bits -> relative error <= 2^-4 in the normal range,
    # absolute error <= 2^-10 * scale in the subnormal range (plus the f32 division)
    k, v = decode_records(rec)
    err = np.abs(v.reshape(-1, 4, 128) - x)
    y = np.abs(x) / scale[:, :, None]
    bound = np.where(y >= 2.0**-6, 2.0**-4 * np.abs(x), 2.0**-10 * scale[:, :, None]) * (1 + 2.0**-20)
    assert np.all(err <= bound)
    # rope is copied bit for bit, and the key is [latent | rope]
    assert np.array_equal(rec[:, 528:].copy().view("<u2"), bf16_bits(k_pe))
    assert np.array_equal(k[:, :512], v)
    assert np.array_equal(k[:, 512:], k_pe.to(torch.float64).numpy())


def test_decoder_matches_torch_view():
    kv_c, k_pe = _random_tokens(3, 128, "heavy")
    rec = encode_records(bf16_bits(kv_c), bf16_bits(k_pe))
    t = torch.from_numpy(rec)
    lat = t[:, :512].view(torch.float8_e4m3fn).to(torch.float64)
    sc = t[:, 512:528].contiguous().view(torch.float32).to(torch.float64)
    lat = lat * sc.repeat_interleave(128, dim=1)
    rope = t[:, 528:].contiguous().view(torch.bfloat16).to(torch.float64)
    k, v = decode_records(rec)
    assert np.array_equal(v, lat.numpy())
    assert np.array_equal(k, torch.cat([lat, rope], 1).numpy())


def test_insert_skips_negative_slots_and_is_idempotent():
    kv_c, k_pe = _random_tokens(5, 40, "std1")
    pool = np.full((64, RECORD_BYTES), 0xA5, dtype=np.uint8)
    slots = np.arange(40, dtype=np.int64) + 10
    slots[::7] = -1
    insert_records(pool, bf16_bits(kv_c), bf16_bits(k_pe), slots)
    rec = encode_records(bf16_bits(kv_c), bf16_bits(k_pe))
    for i, s in enumerate(slots):
        if s >= 0:
            assert np.array_equal(pool[s], rec[i])
    written = set(int(s) for s in slots if s >= 0)
    for s in range(64):
        if s not in written:
            assert np.all(pool[s] == 0xA5)
    again = pool.copy()
    insert_records(again, bf16_bits(kv_c), bf16_bits(k_pe), slots)
    assert np.array_equal(again, pool)
