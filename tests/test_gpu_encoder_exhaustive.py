"""The record writer's E4M3 codes over its whole input domain.

A tile's codes depend only on its maximum magnitude A (through the scale
A / 448) and on each value x; both are bf16.  So every pair of a positive
finite bf16 maximum A (0x0001 .. 0x7F7F) and a bf16 value x with |x| <= A
(both signs, both zeros, the subnormals) covers every code the writer can
produce: 1.07e9 pairs in 8.4 M tiles, each tile led by its maximum and
holding 127 of that maximum's values (the last tile of a maximum padded with
zeros).  They go through mla_cache_insert in batches and every record is
compared byte for byte with the oracle writer (encode_records: the float32
scale, numpy's IEEE float32 quotient, the saturating RNE encode written from
the format; fused_mla_key_concat_kv_cache page, the ds_mla insert).  This is
the exhaustive check behind the writer's use of the hardware convert and of
the reciprocal in place of the division.
"""

import numpy as np
import pytest
import torch

import head_latent_attention_sparse_amd as mla
from oracle import encode_records
from tests.helpers import _parallel, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
MAX_FINITE = 0x7F7F        # largest finite bf16 bit pattern
VALUES_PER_BATCH = 1 << 25  # padded values per batch (about 260 K tiles)


def _maxima():
    a = np.arange(1, MAX_FINITE + 1, dtype=np.int64)
    padded = 127 * ((2 * (a + 1) + 126) // 127)  # each maximum's values, padded to whole tiles
    return a, padded


def _batches():
    """[lo, hi) ranges of maxima, each about VALUES_PER_BATCH padded values."""
    a, padded = _maxima()
    cum = np.cumsum(padded)
    edges = [0]
    while edges[-1] < a.size:
        target = (cum[edges[-1] - 1] if edges[-1] else 0) + VALUES_PER_BATCH
        nxt = int(np.searchsorted(cum, target, side="right"))
        edges.append(max(nxt, edges[-1] + 1))
    edges[-1] = min(edges[-1], a.size)
    return [(int(a[lo]), int(a[hi - 1]) + 1) for lo, hi in zip(edges[:-1], edges[1:])]


def _tiles(a_lo, a_hi):
    """Tiles (uint16 [n, 128]) for maxima a_lo .. a_hi - 1: column 0 holds the
    maximum, columns 1..127 its values 0..A, then 0x8000 | 0..A, then zeros."""
    a = np.arange(a_lo, a_hi, dtype=np.int32)
    tiles_per = (2 * (a + 1) + 126) // 127
    padded = 127 * tiles_per
    starts = np.cumsum(padded, dtype=np.int64) - padded
    owner = np.repeat(np.arange(a.size, dtype=np.int32), padded)
    j = (np.arange(int(padded.sum()), dtype=np.int64) - starts[owner]).astype(np.int32)
    a1 = (a + 1)[owner]
    vals = np.where(j < 2 * a1, np.where(j >= a1, (j - a1) | 0x8000, j), 0).astype(np.uint16)
    tiles = np.empty((int(tiles_per.sum()), 128), np.uint16)
    tiles[:, 0] = np.repeat(a, tiles_per).astype(np.uint16)
    tiles[:, 1:] = vals.reshape(-1, 127)
    pad = (-tiles.shape[0]) % 4  # whole tokens of 4 tiles: repeat the first tile
    if pad:
        tiles = np.concatenate([tiles, np.repeat(tiles[:1], pad, axis=0)])
    return tiles


def _prepare(rng):
    """Tokens of one batch and their oracle records."""
    tiles = _tiles(*rng)
    kv = tiles.reshape(-1, 512)
    pe = np.zeros((kv.shape[0], 64), np.uint16)
    return kv, encode_records(kv, pe)


def test_encoder_exhaustive_over_bf16_maxima_and_values():
    batches = _batches()
    a, padded = _maxima()
    assert batches[0][0] == 1 and batches[-1][1] == MAX_FINITE + 1
    assert all(hi == lo2 for (_, hi), (lo2, _) in zip(batches[:-1], batches[1:]))
    say(f"encoder, exhaustive: {int((2 * (a + 1)).sum()):,} (maximum, value) pairs in "
        f"{int((padded // 127).sum()):,} tiles, {len(batches)} batches")
    done = 0
    for k, (kv, want) in enumerate(_parallel(_prepare, batches)):
        n = kv.shape[0]
        kv_t = torch.from_numpy(kv.view(np.int16)).view(torch.bfloat16).to(DEV)
        pe_t = torch.zeros((n, 64), dtype=torch.bfloat16, device=DEV)
        pool = torch.empty((n, 656), dtype=torch.uint8, device=DEV)
        mla.cache_insert(kv_t, pe_t, torch.arange(n, dtype=torch.int64, device=DEV), pool)
        got = pool.cpu().numpy()
        bad = np.nonzero(np.any(got != want, axis=1))[0]
        if bad.size:
            t0 = int(bad[0])
            col = int(np.nonzero(got[t0] != want[t0])[0][0])
            tile = kv[t0, 128 * (col // 128) : 128 * (col // 128) + 128] if col < 512 else kv[t0, :128]
            raise AssertionError(f"batch {k} {batches[k]}: {bad.size} records differ; token {t0}, byte {col}: "
                                 f"got {got[t0, col]:#04x} want {want[t0, col]:#04x}, tile maximum "
                                 f"{int(tile[0]):#06x}")
        done += n
        if k % 8 == 0 or k == len(batches) - 1:
            say(f"  batch {k + 1}/{len(batches)}: maxima {batches[k][0]:#06x}..{batches[k][1] - 1:#06x}, "
                f"{done:,} tokens checked")
