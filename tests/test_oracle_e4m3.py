"""Pins for the oracle's E4M3 codec (no GPU).

The decoder is checked against torch's own float8_e4m3fn -> float32 cast (a
library routine) for all 256 codes and against textbook values; the encoder
against torch's float32 -> float8_e4m3fn cast after a clamp to +-448 (the
saturating quant) over every bf16 pattern, every rounding boundary and a
strided sweep of float32, and against hand-worked values in
tests/golden/e4m3_worked.txt.
"""

import os

import numpy as np
import pytest
import torch

from oracle import e4m3_decode, e4m3_encode


def torch_encode(x32):
    t = torch.from_numpy(np.asarray(x32, dtype=np.float32))
    return t.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(got[~nan], ref[~nan].astype(np.float64))
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_decode_textbook_values():
    d = dict(zip(range(256), e4m3_decode(np.arange(256, dtype=np.uint8))))
    assert d[0x38] == 1.0
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0
    assert d[0x08] == 2.0**-6
    assert d[0x01] == 2.0**-9
    assert d[0x07] == 7 * 2.0**-9
    assert d[0x00] == 0.0 and not np.signbit(d[0x00])
    assert d[0x80] == 0.0 and np.signbit(d[0x80])
    finite = [v for c, v in d.items() if not np.isnan(v)]
    assert max(finite) == 448.0 and min(finite) == -448.0


def test_encode_worked_examples(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "e4m3_worked.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                value, code = line.split()[:2]
                rows.append((float(value), int(code, 16)))
    x = np.array([v for v, _ in rows], dtype=np.float32)
    want = np.array([c for _, c in rows], dtype=np.uint8)
    assert np.array_equal(e4m3_encode(x), want)
    assert np.array_equal(torch_encode(x), want)  # the fixture agrees with the library


def test_encode_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(e4m3_encode(e4m3_decode(codes)), codes)


def test_encode_every_bf16_pattern():
    bits = np.arange(65536, dtype=np.uint32) << 16
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    assert np.array_equal(e4m3_encode(x), torch_encode(x))


def test_encode_rounding_boundaries():
    vals = e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))  # 0 .. 448, ascending
    mids = (vals[:-1] + vals[1:]) / 2.0  # exact in float32 (few significant bits)
    mids32 = mids.astype(np.float32)
    assert np.array_equal(mids32.astype(np.float64), mids)
    probes = [mids32, vals.astype(np.float32)]
    for k in (1, 2, 3):
        probes.append(np.nextafter(mids32, np.float32(np.inf)))
        probes.append(np.nextafter(mids32, np.float32(0)))
        mids32 = probes[-1]
    x = np.concatenate(probes)
    x = np.concatenate([x, -x, np.array([448.5, 460, 464, 479.9, 480, 1e38, np.inf], np.float32)])
    assert np.array_equal(e4m3_encode(x), torch_encode(x))


def test_encode_strided_float32_sweep():
    # Every 61st float32 bit pattern in [0, 448] (about 18.7M values), both signs.
    top = np.float32(448.0).view(np.uint32)
    bits = np.arange(0, int(top) + 1, 61, dtype=np.uint32)
    for chunk in np.array_split(bits, 8):
        x = chunk.view(np.float32)
        assert np.array_equal(e4m3_encode(x), torch_encode(x))
        assert np.array_equal(e4m3_encode(-x), torch_encode(-x))


@pytest.mark.parametrize("seed", [0, 1])
def test_encode_random_float32(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(1_000_000) * np.exp2(rng.uniform(-14, 10, 1_000_000))).astype(np.float32)
    assert np.array_equal(e4m3_encode(x), torch_encode(x))
