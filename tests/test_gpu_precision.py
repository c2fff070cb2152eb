"""GPU precision tests at the edges of the value range the pages allow, and
an exhaustive pin of the device E4M3 encoder.

* Queries with outlier channels (x30, x100, x300) and with 32-element
  groups spanning 2^14 of range, at a softmax scale that keeps the logits
  realistic (standard deviation 3): out and lse must meet the forward's bar
  against the oracle.  Such queries put products of very different size
  into one dot product; the forward's bf16 dot products with float32
  accumulation keep them (an fp8 block-scaled contraction, which sums each
  32-element block with ~14 bits below its largest product, did not).
* The FlyDSL slice accepts per-tile scales that are powers of two up to
  2^7 (|value| <= 448 * 2^7 = 57344; flydsl_sparse_mla page,
  flydsl_sparse_mla_fp8ds_supported docstring).  Records with such scales
  are checked with lse at the forward's bar and out against a bar that adds
  the bf16 rounding of the softmax weights (2^-9 relative each, taken as
  2^-8 of the largest |value| in the column of the row's keys) to the
  forward's bar; the measured errors are printed.
* The insert's encoder, on every bf16 value in [-448, 448] at tile scale
  exactly 1 (each tile holds +-448), and on tiles whose maximum steps
  through every bf16 exponent, bit-exact against the oracle writer.
"""

import numpy as np
import pytest
import torch

import head_latent_attention_sparse_amd as mla
from head_latent_attention_sparse_amd.workloads import bf16_bits
from oracle import decode_records, sparse_fwd as oracle_fwd
from tests.helpers import LSE_ATOL, OUT_ATOL, OUT_RTOL, assert_fwd_close, oracle_encode, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
HEADS = 16


def _csr(rng, lengths, n_rec):
    rows = [rng.permutation(n_rec)[:n] for n in lengths]
    indptr = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    indices = np.concatenate(rows).astype(np.int32) if rows else np.zeros(0, np.int32)
    return indptr, indices


def _scale_for_logit_std(q, keys, std=3.0):
    """A softmax scale at which q . k over these keys has the given standard
    deviation (q bf16 [T, H, 576], keys float64 [n, 576])."""
    z = q.float().numpy().astype(np.float64).reshape(-1, 576) @ keys.T
    return float(std / np.std(z))


def _outlier_query(seed, t, mult, spread):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((t, HEADS, 576), generator=g)
    if mult > 1:
        channels = torch.randperm(512, generator=g)[:8]
        q[:, :, channels] *= mult
    if spread:
        # each latent element scaled by 2^u, u uniform in [-14, 0]
        q[:, :, :512] *= torch.pow(2.0, -14.0 * torch.rand((t, HEADS, 512), generator=g))
    return q.to(torch.bfloat16)


@pytest.mark.parametrize("mult,spread", [(30, False), (100, False), (300, False), (1, True), (100, True)])
def test_outlier_queries_and_wide_groups(mult, spread):
    say(f"precision: outlier channels x{mult}, groups spanning 2^14: {spread}")
    n_rec = 4096
    g = torch.Generator().manual_seed(1234)
    kv_c = torch.randn((n_rec, 512), generator=g).to(torch.bfloat16)
    k_pe = torch.randn((n_rec, 64), generator=g).to(torch.bfloat16)
    ref_pool = oracle_encode(kv_c, k_pe)
    pool = torch.zeros((n_rec, 656), dtype=torch.uint8, device=DEV)
    mla.cache_insert(kv_c.to(DEV), k_pe.to(DEV), torch.arange(n_rec, dtype=torch.int64, device=DEV), pool)
    torch.cuda.synchronize()
    assert np.array_equal(pool.cpu().numpy(), ref_pool)

    rng = np.random.default_rng(mult * 10 + spread)
    lengths = [2048, 1000, 130, 64, 1, 700, 257, 3000]
    indptr, indices = _csr(rng, lengths, n_rec)
    q = _outlier_query(77 + mult, len(lengths), mult, spread)
    keys, _ = decode_records(ref_pool[rng.permutation(n_rec)[:512]])
    scale = _scale_for_logit_std(q, keys)
    ref_out, ref_lse = oracle_fwd(bf16_bits(q), ref_pool, indptr, indices, scale)
    for chunk_tiles in (0, 5):
        out, lse = mla.sparse_fwd(q.to(DEV), pool, torch.from_numpy(indptr).to(DEV),
                                  torch.from_numpy(indices).to(DEV), scale, return_lse=True,
                                  chunk_tiles=chunk_tiles)
        torch.cuda.synchronize()
        o = out.float().cpu().numpy()
        say(f"  chunk_tiles={chunk_tiles}: max |out err| {np.max(np.abs(o - ref_out)):.3e}, "
            f"max |lse err| {np.max(np.abs(lse.cpu().numpy() - ref_lse)):.3e}")
        assert_fwd_close(out, lse, ref_out, ref_lse, f"outliers x{mult} spread={spread} chunks={chunk_tiles}")


def _top_scale_records(seed, n_rec):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, (n_rec, 512), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x7E  # no NaN codes; the largest finite code instead
    exps = rng.integers(-9, 8, (n_rec, 4))
    exps[rng.random((n_rec, 4)) < 0.25] = 7  # a quarter of the tiles at the top scale 2^7
    scales = np.ldexp(1.0, exps).astype("<f4")
    rope = torch.randn((n_rec, 64), generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16)
    rec = np.zeros((n_rec, 656), np.uint8)
    rec[:, :512] = codes
    rec[:, 512:528] = scales.view(np.uint8).reshape(n_rec, 16)
    rec[:, 528:] = bf16_bits(rope).view(np.uint8).reshape(n_rec, 128)
    return rec


def test_raw_records_top_scale():
    say("precision: raw records with power-of-two scales up to 2^7 (|value| <= 57344)")
    n_rec = 2048
    rec = _top_scale_records(901, n_rec)
    rng = np.random.default_rng(902)
    lengths = [700, 300, 129, 64, 1, 0, 1500, 2048]
    indptr, indices = _csr(rng, lengths, n_rec)
    q = torch.randn((len(lengths), HEADS, 576), generator=torch.Generator().manual_seed(903)).to(torch.bfloat16)
    keys, values = decode_records(rec)
    assert np.max(np.abs(values)) == 448.0 * 2 ** 7
    scale = _scale_for_logit_std(q, keys[rng.permutation(n_rec)[:512]])
    ref_out, ref_lse = oracle_fwd(bf16_bits(q), rec, indptr, indices, scale)
    rec_d = torch.from_numpy(rec).to(DEV)
    ptr_d, idx_d = torch.from_numpy(indptr).to(DEV), torch.from_numpy(indices).to(DEV)
    for chunk_tiles in (0, 3):
        out, lse = mla.sparse_fwd(q.to(DEV), rec_d, ptr_d, idx_d, scale, return_lse=True, chunk_tiles=chunk_tiles)
        torch.cuda.synchronize()
        o = out.float().cpu().numpy().astype(np.float64)
        l = lse.cpu().numpy().astype(np.float64)
        assert np.array_equal(np.isneginf(l), np.isneginf(ref_lse))
        fin = np.isfinite(ref_lse)
        lse_err = np.max(np.abs(l[fin] - ref_lse[fin]))
        err = np.abs(o - ref_out)
        plain = OUT_ATOL + OUT_RTOL * np.abs(ref_out)
        # largest |value| per column over each row's keys
        vmax = np.zeros((len(lengths), 1, 512))
        for t in range(len(lengths)):
            ids = indices[indptr[t]:indptr[t + 1]]
            if ids.size:
                vmax[t, 0] = np.max(np.abs(values[ids]), axis=0)
        bar = plain + 2.0 ** -8 * vmax
        say(f"  chunk_tiles={chunk_tiles}: lse max err {lse_err:.3e}; out max err {err.max():.3e} "
            f"(max |ref| {np.abs(ref_out).max():.1f}); max err / column max |v| "
            f"{np.max(err / np.maximum(vmax, 1e-30)):.3e}; elements over the plain bar "
            f"{int(np.sum(err > plain))} of {err.size}")
        assert lse_err <= LSE_ATOL, f"lse off by {lse_err}"
        assert np.all(err <= bar), f"out off: worst excess {np.max(err - bar)}"


# ------------------------------------------------------------- the encoder

def _bits_to_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def _tokens_from_tiles(tiles, seed):
    """[n_tiles, 128] bf16 bit patterns -> (kv_c bf16 [tokens, 512], k_pe) with
    4 tiles per token (a last partial token padded with tiles of 1.0)."""
    n = tiles.shape[0]
    pad = (-n) % 4
    if pad:
        tiles = np.concatenate([tiles, np.full((pad, 128), 0x3F80, np.uint16)])
    kv = tiles.reshape(-1, 512)
    pe = torch.randn((kv.shape[0], 64), generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16)
    return _bits_to_bf16(kv), pe


def _insert_and_compare(kv_c, k_pe, what):
    n = kv_c.shape[0]
    pool = torch.full((n + 5, 656), 0xA5, dtype=torch.uint8, device=DEV)
    mla.cache_insert(kv_c.to(DEV), k_pe.to(DEV), torch.arange(n, dtype=torch.int64, device=DEV), pool)
    torch.cuda.synchronize()
    want = oracle_encode(kv_c, k_pe)
    got = pool.cpu().numpy()
    assert np.all(got[n:] == 0xA5), f"{what}: bytes past the inserted slots changed"
    bad = np.nonzero(np.any(got[:n] != want, axis=1))[0]
    assert bad.size == 0, f"{what}: {bad.size} records differ, first tokens {bad[:5]}"
    return want


def test_encoder_every_bf16_value_at_scale_one():
    """All 2 * 17377 bf16 patterns of magnitude <= 448 (both zeros and the
    subnormals included) in tiles whose maximum is 448, so the tile scale is
    448 / 448 = 1 and each code is the saturating RNE E4M3 of the value."""
    say("encoder: every bf16 value in [-448, 448] at scale 1")
    mags = np.arange(0, 0x43E0 + 1, dtype=np.uint16)  # +0 .. 448
    vals = np.concatenate([mags, mags | 0x8000])
    rng = np.random.default_rng(31)
    vals = vals[rng.permutation(vals.size)]
    n_tiles = -(-vals.size // 127)
    vals = np.concatenate([vals, np.zeros(n_tiles * 127 - vals.size, np.uint16)]).reshape(n_tiles, 127)
    tiles = np.empty((n_tiles, 128), np.uint16)
    pos = rng.integers(0, 128, n_tiles)
    top = np.where(rng.random(n_tiles) < 0.5, 0x43E0, 0xC3E0).astype(np.uint16)  # +448 or -448
    for i in range(n_tiles):
        tiles[i] = np.insert(vals[i], pos[i], top[i])
    kv_c, k_pe = _tokens_from_tiles(tiles, 32)
    want = _insert_and_compare(kv_c, k_pe, "scale-1 sweep")
    scales = np.ascontiguousarray(want[:, 512:528]).view("<f4")
    real = n_tiles  # the padded tiles of 1.0 have scale 1/448
    assert np.all(scales.reshape(-1)[:real] == 1.0)


def test_encoder_every_bf16_value_under_chosen_tile_maxima():
    """For a set of tile maxima, every bf16 value of magnitude at most that
    maximum (both signs, zeros and subnormals included) in tiles led by the
    maximum.  The maxima: the smallest subnormals and the smallest normal,
    two neighbours on either side of 0x15DF / 0x15E0 (about 1.75 * 2^-84),
    where the scale max / 448 crosses 2^-92 and the writer switches from
    dividing to multiplying by the rounded reciprocal with one correction
    step, the same around 2^-125 (0x055F / 0x0560), all-ones and zero
    mantissas across the exponent range, and random ones.  Each code must
    equal the oracle's, whose quotient is numpy's IEEE float32 division."""
    say("encoder: every bf16 value under chosen tile maxima")
    rng = np.random.default_rng(47)
    tops = [0x0001, 0x0002, 0x007F, 0x0080, 0x055E, 0x055F, 0x0560, 0x0561, 0x15DE, 0x15DF, 0x15E0, 0x15E1]
    for e in (-120, -64, -20, -7, -1, 0, 1, 3, 8, 9, 20, 64, 127):
        tops += [((e + 127) << 7) | 0x7F, ((e + 127) << 7), ((e + 127) << 7) | int(rng.integers(1, 0x7F))]
    tops = [t for t in tops if t <= 0x7F7F]  # finite
    tops += [int(t) for t in rng.integers(0x0080, 0x7F7F, 8)]
    tiles = []
    for t in tops:
        mags = np.arange(0, t + 1, dtype=np.uint16)
        vals = np.concatenate([mags, mags | 0x8000])
        vals = vals[rng.permutation(vals.size)]
        n = -(-vals.size // 127)
        vals = np.concatenate([vals, np.zeros(n * 127 - vals.size, np.uint16)]).reshape(n, 127)
        lead = np.where(rng.random(n) < 0.5, t, t | 0x8000).astype(np.uint16)[:, None]
        tiles.append(np.concatenate([lead, vals], axis=1))
    tiles = np.concatenate(tiles)
    kv_c, k_pe = _tokens_from_tiles(tiles, 43)
    _insert_and_compare(kv_c, k_pe, "maxima sweep")


def test_encoder_tile_maximum_through_every_bf16_exponent():
    """Tiles whose maximum magnitude is m * 2^e for every bf16 exponent e
    (subnormal maxima 2^-133 .. 2^-127 included, up to the largest finite
    bf16), three mantissas each, the other 127 values uniform in
    [-max, max]: the scale max / 448 and the quotients x / scale then run
    over the whole float32 range the writer can meet."""
    say("encoder: tile maxima through every bf16 exponent")
    rng = np.random.default_rng(41)
    tops = []
    for e in range(-133, 128):
        for mant in (0, 0x7F, int(rng.integers(1, 0x7F))):
            if e >= -126:
                tops.append(((e + 127) << 7) | mant)
            else:
                lead = 1 << (e + 133)  # subnormal: value = bits * 2^-133
                tops.append(lead | (mant & (lead - 1)))
    tops = np.array(tops, np.uint16)
    amax = (tops.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rest = rng.uniform(-1.0, 1.0, (tops.size, 127)) * amax[:, None]
    rest_bits = bf16_bits(torch.from_numpy(rest.astype(np.float32)).to(torch.bfloat16))
    # bf16 rounding may carry a value past the maximum: pull it back to +-max
    over = (rest_bits & 0x7FFF) > tops[:, None]
    rest_bits = np.where(over, (rest_bits & 0x8000) | tops[:, None], rest_bits).astype(np.uint16)
    tiles = np.empty((tops.size, 128), np.uint16)
    pos = rng.integers(0, 128, tops.size)
    sign = np.where(rng.random(tops.size) < 0.5, 0, 0x8000).astype(np.uint16)
    for i in range(tops.size):
        tiles[i] = np.insert(rest_bits[i], pos[i], tops[i] | sign[i])
    kv_c, k_pe = _tokens_from_tiles(tiles, 42)
    _insert_and_compare(kv_c, k_pe, "exponent sweep")
