"""Pins for the oracle's context gather + upconvert (no GPU).

* the upconvert against torch: the codes viewed as float8_e4m3fn, cast to
  float32, times the float32 scale, cast to bfloat16 (library routines);
* within one bf16 ulp of the exact latent the record decoder gives (float64),
  and equal to its bf16 rounding except for rare double-rounding ties;
* the block-table addressing against a per-row brute force written from the
  same rule (row -> request by a linear scan, position -> block -> slot);
* rows without a valid source (block id -1, position past the table, rows
  beyond the chunk) are zero.
"""

import numpy as np
import torch

from oracle import decode_records, encode_records, gather_upconvert, upconvert_records
from head_latent_attention_sparse_amd.workloads import bf16_bits


def rand_records(n, seed, std=1.0):
    rng = np.random.default_rng(seed)
    kv = bf16_bits(torch.from_numpy((rng.standard_normal((n, 512)) * std).astype(np.float32)).to(torch.bfloat16))
    pe = bf16_bits(torch.from_numpy(rng.standard_normal((n, 64)).astype(np.float32)).to(torch.bfloat16))
    return encode_records(kv, pe)


def test_upconvert_matches_torch_casts():
    for seed, std in ((1, 1.0), (2, 1e-3), (3, 300.0)):
        rec = rand_records(300, seed, std)
        got = upconvert_records(rec)
        codes = torch.from_numpy(rec[:, :512].copy()).view(torch.float8_e4m3fn).to(torch.float32)
        scale = torch.from_numpy(rec[:, 512:528].copy()).view(torch.float32)
        lat = (codes.reshape(-1, 4, 128) * scale[:, :, None]).reshape(-1, 512).to(torch.bfloat16)
        np.testing.assert_array_equal(got[:, :512], bf16_bits(lat))
        np.testing.assert_array_equal(got[:, 512:], rec[:, 528:].copy().view("<u2"))


def test_upconvert_is_the_bf16_rounding_of_the_exact_latent():
    rec = rand_records(500, 4)
    got = (upconvert_records(rec)[:, :512].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    _, exact = decode_records(rec)
    ulp = np.abs(exact) * 2.0**-7
    assert np.all(np.abs(got - exact) <= ulp + 1e-300)
    direct = bf16_bits(torch.from_numpy(exact).to(torch.bfloat16))  # single rounding of the exact value
    assert np.mean(upconvert_records(rec)[:, :512] == direct) > 0.999


def brute_force(pool, bs, table, cu, starts, num_tokens):
    out = np.zeros((num_tokens, 576), np.uint16)
    ups = upconvert_records(pool)
    for row in range(num_tokens):
        r = None
        for cand in range(len(cu) - 1):
            if cu[cand] <= row < cu[cand + 1]:
                r = cand
        if r is None:
            continue
        p = (0 if starts is None else starts[r]) + row - cu[r]
        if p // bs >= table.shape[1]:
            continue
        blk = table[r, p // bs]
        if blk < 0 or blk * bs + p % bs >= pool.shape[0]:
            continue
        out[row] = ups[blk * bs + p % bs]
    return out


def test_addressing_against_brute_force():
    rng = np.random.default_rng(5)
    bs, nblk = 16, 30
    pool = rand_records(bs * nblk, 6)
    table = rng.permutation(nblk).astype(np.int64)[:24].reshape(4, 6)
    table[1, 3:] = -1
    table[2, 2] = nblk + 4  # outside the pool
    counts = np.array([40, 70, 0, 50])
    starts = np.array([5, 0, 3, 40])
    cu = np.concatenate([[0], np.cumsum(counts)])
    n = int(cu[-1]) + 7  # rows past the chunk stay zero
    got = gather_upconvert(pool, bs, table, cu, starts, n)
    np.testing.assert_array_equal(got, brute_force(pool, bs, table, cu, starts, n))
    assert np.all(got[cu[-1]:] == 0)
    assert np.all(got[40 + 48:40 + 70] == 0)  # request 1, positions 48.. read block -1
    assert np.any(got[:40] != 0)
    # no starts: every chunk begins at position 0
    np.testing.assert_array_equal(gather_upconvert(pool, bs, table, cu, None, n),
                                  brute_force(pool, bs, table, cu, None, n))
