"""Pins for the oracle's sparse attention forward and LSE merge (no GPU).

* brute force on tiny inputs: a separate formulation per (row, head) with
  torch's float8 view for the dequant and torch.softmax / torch.logsumexp in
  float64 (library routines);
* invariants the definition fixes: one key gives out = v and lse = z; q = 0
  gives the mean of the values and lse = ln n; permuting a row or dropping its
  masked entries changes nothing; a key listed m times adds ln m to the lse;
  sigma = 0 gives the mean; two keys give the logaddexp closed form; an empty
  or all-masked row gives out 0 and lse -inf;
* the one-token warmup problem (tests/golden/warmup_problem.json);
* the merge: any split of a row's list merged by LSE equals the unsplit row.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import decode_records, encode_records, merge_partials, sparse_fwd
from head_latent_attention_sparse_amd.workloads import bf16_bits


def make_case(seed, t_count, heads, n_rec, max_len, p_invalid=0.2, latent_std=1.0):
    g = torch.Generator().manual_seed(seed)
    kv_c = (torch.randn((n_rec, 512), generator=g) * latent_std).to(torch.bfloat16)
    k_pe = torch.randn((n_rec, 64), generator=g).to(torch.bfloat16)
    rec = encode_records(bf16_bits(kv_c), bf16_bits(k_pe))
    q = torch.randn((t_count, heads, 576), generator=g).to(torch.bfloat16)
    lens = torch.randint(0, max_len + 1, (t_count,), generator=g)
    indptr = np.concatenate([[0], np.cumsum(lens.numpy())]).astype(np.int64)
    nnz = int(indptr[-1])
    ind = torch.randint(0, n_rec, (nnz,), generator=g).numpy().astype(np.int64)
    ind[torch.rand(nnz, generator=g).numpy() < p_invalid] = -1
    return bf16_bits(q), rec, indptr, ind


def brute_force(q_bits, rec, indptr, indices, scale):
    t = torch.from_numpy(rec)
    lat = t[:, :512].view(torch.float8_e4m3fn).to(torch.float64)
    sc = t[:, 512:528].contiguous().view(torch.float32).to(torch.float64)
    lat = lat * sc.repeat_interleave(128, dim=1)
    rope = t[:, 528:].contiguous().view(torch.bfloat16).to(torch.float64)
    keys = torch.cat([lat, rope], 1)
    q = torch.from_numpy(q_bits.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    sigma = float(np.float32(scale))
    t_count, heads, _ = q.shape
    out = torch.zeros((t_count, heads, 512), dtype=torch.float64)
    lse = torch.full((t_count, heads), -math.inf, dtype=torch.float64)
    for r in range(t_count):
        entries = [int(i) for i in indices[indptr[r] : indptr[r + 1]] if 0 <= i < rec.shape[0]]
        if not entries:
            continue
        for h in range(heads):
            logits = torch.stack([sigma * torch.dot(q[r, h], keys[j]) for j in entries])
            w = torch.softmax(logits, 0)
            lse[r, h] = torch.logsumexp(logits, 0)
            out[r, h] = sum(w[i] * lat[j] for i, j in enumerate(entries))
    return out.numpy(), lse.numpy()


@pytest.mark.parametrize("seed,t_count,heads,n_rec,max_len", [
    (0, 3, 2, 6, 6), (1, 4, 1, 9, 5), (2, 2, 3, 4, 8), (3, 5, 2, 12, 3)])
def test_brute_force(seed, t_count, heads, n_rec, max_len):
    q, rec, indptr, ind = make_case(seed, t_count, heads, n_rec, max_len)
    scale = 192**-0.5
    out, lse = sparse_fwd(q, rec, indptr, ind, scale)
    ref_out, ref_lse = brute_force(q, rec, indptr, ind, scale)
    assert np.array_equal(np.isneginf(lse), np.isneginf(ref_lse))
    fin = np.isfinite(ref_lse)
    np.testing.assert_allclose(lse[fin], ref_lse[fin], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out, ref_out, rtol=1e-10, atol=1e-12)


def _one_row(q_bits, rec, ids, scale):
    ids = np.asarray(ids, dtype=np.int64)
    return sparse_fwd(q_bits[:1], rec, np.array([0, ids.size]), ids, scale)


def test_single_key_gives_its_value_and_logit():
    q, rec, _, _ = make_case(10, 1, 4, 8, 1)
    k, v = decode_records(rec)
    qf = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    sigma = float(np.float32(0.3))
    out, lse = _one_row(q, rec, [5], 0.3)
    np.testing.assert_allclose(out[0], np.broadcast_to(v[5], (4, 512)), rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0], sigma * (qf[0] @ k[5]), rtol=1e-13)


def test_zero_query_gives_mean_and_log_n():
    q, rec, _, _ = make_case(11, 1, 3, 10, 1)
    q = np.zeros_like(q)
    ids = [1, 4, 7, 2]
    out, lse = _one_row(q, rec, ids, 0.7)
    _, v = decode_records(rec)
    np.testing.assert_allclose(out[0], np.broadcast_to(v[ids].mean(0), (3, 512)), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse[0], math.log(len(ids)), rtol=1e-14)


def test_zero_scale_gives_mean():
    q, rec, _, _ = make_case(12, 1, 2, 10, 1)
    ids = [0, 3, 9]
    out, lse = _one_row(q, rec, ids, 0.0)
    _, v = decode_records(rec)
    np.testing.assert_allclose(out[0], np.broadcast_to(v[ids].mean(0), (2, 512)), rtol=1e-13, atol=1e-15)


def test_permutation_and_masked_entries_do_not_matter():
    q, rec, _, _ = make_case(13, 1, 4, 20, 1)
    ids = np.array([3, 17, 5, 0, 12, 8])
    base = _one_row(q, rec, ids, 0.2)
    perm = _one_row(q, rec, ids[[4, 2, 0, 5, 1, 3]], 0.2)
    holes = _one_row(q, rec, [-1, 3, 17, -5, 5, 0, -1, 12, 8, -1], 0.2)
    for other in (perm, holes):
        np.testing.assert_allclose(other[0], base[0], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(other[1], base[1], rtol=1e-13)


def test_duplicated_key_adds_log_multiplicity():
    q, rec, _, _ = make_case(14, 1, 2, 6, 1)
    one = _one_row(q, rec, [4], 0.5)
    three = _one_row(q, rec, [4, 4, 4], 0.5)
    np.testing.assert_allclose(three[1], one[1] + math.log(3), rtol=1e-13)
    np.testing.assert_allclose(three[0], one[0], rtol=1e-13, atol=1e-15)


def test_two_keys_closed_form():
    q, rec, _, _ = make_case(15, 1, 3, 6, 1)
    k, v = decode_records(rec)
    qf = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()[0]
    sigma = float(np.float32(0.9))
    z1, z2 = sigma * (qf @ k[1]), sigma * (qf @ k[2])
    out, lse = _one_row(q, rec, [1, 2], 0.9)
    np.testing.assert_allclose(lse[0], np.logaddexp(z1, z2), rtol=1e-13)
    w1 = 1.0 / (1.0 + np.exp(z2 - z1))
    np.testing.assert_allclose(out[0], w1[:, None] * v[1] + (1 - w1)[:, None] * v[2], rtol=1e-11, atol=1e-14)


def test_empty_and_all_masked_rows():
    q, rec, _, _ = make_case(16, 3, 2, 6, 1)
    indptr = np.array([0, 0, 3, 3])
    ind = np.array([-1, -1, -7])
    out, lse = sparse_fwd(q, rec, indptr, ind, 1.0)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_out_of_range_slot_is_masked():
    q, rec, _, _ = make_case(17, 1, 2, 6, 1)
    base = _one_row(q, rec, [1, 2], 1.0)
    extra = _one_row(q, rec, [1, 6, 2, 1 << 30], 1.0)
    np.testing.assert_allclose(extra[0], base[0], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(extra[1], base[1], rtol=1e-13)


def test_warmup_problem(golden_dir):
    with open(os.path.join(golden_dir, "warmup_problem.json")) as f:
        fx = json.load(f)
    rec = np.zeros((fx["records"], 656), dtype=np.uint8)
    for heads in fx["heads"]:
        q = np.zeros((1, heads, 576), dtype=np.uint16)
        out, lse = sparse_fwd(q, rec, np.array(fx["indptr"]), np.array(fx["indices"]), fx["softmax_scale"])
        assert np.all(out == fx["expected_out"])
        assert np.all(lse == fx["expected_lse"])


@pytest.mark.parametrize("pieces", [2, 3, 7])
def test_merge_of_any_split_equals_unsplit(pieces):
    q, rec, indptr, ind = make_case(20, 4, 3, 40, 30, p_invalid=0.3, latent_std=2.0)
    out, lse = sparse_fwd(q, rec, indptr, ind, 192**-0.5)
    rng = np.random.default_rng(pieces)
    parts_out, parts_lse = [], []
    cuts = [np.sort(rng.integers(indptr[t], indptr[t + 1] + 1, pieces - 1)) for t in range(4)]
    for p in range(pieces):
        sub_ptr, sub_ind = [0], []
        for t in range(4):
            bounds = [indptr[t], *cuts[t], indptr[t + 1]]
            sub_ind.extend(ind[bounds[p] : bounds[p + 1]])
            sub_ptr.append(len(sub_ind))
        o, l = sparse_fwd(q, rec, np.array(sub_ptr), np.array(sub_ind, dtype=np.int64), 192**-0.5)
        parts_out.append(o)
        parts_lse.append(l)
    m_out, m_lse = merge_partials(parts_out, parts_lse)
    assert np.array_equal(np.isneginf(m_lse), np.isneginf(lse))
    fin = np.isfinite(lse)
    np.testing.assert_allclose(m_lse[fin], lse[fin], rtol=1e-12)
    np.testing.assert_allclose(m_out, out, rtol=1e-12, atol=1e-13)


def test_merge_all_empty_partials():
    o = np.zeros((2, 512))
    l = np.full(2, -np.inf)
    out, lse = merge_partials([o, o, o], [l, l, l])
    assert np.all(out == 0) and np.all(np.isneginf(lse))


# ---- the sink and the second segment (readings: a sink is one more logit
# with a zero value; the extra segment's keys join the same softmax)

def bits_of(x):
    return bf16_bits(torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16))


def _records(rng, n):
    return encode_records(bits_of(rng.standard_normal((n, 512))), bits_of(rng.standard_normal((n, 64))))


def _small_problem(seed, t=5, h=3, n=40, n2=30):
    rng = np.random.default_rng(seed)
    q = bits_of(rng.standard_normal((t, h, 576)))
    rec = _records(rng, n)
    rec2 = _records(rng, n2)
    lens = rng.integers(0, 9, t)
    lens[1] = 0
    indptr = np.concatenate([[0], np.cumsum(lens)])
    indices = rng.integers(-2, n + 3, indptr[-1])
    lens2 = rng.integers(0, 7, t)
    lens2[2] = 0
    indptr2 = np.concatenate([[0], np.cumsum(lens2)])
    indices2 = rng.integers(-2, n2 + 3, indptr2[-1])
    return q, rec, indptr, indices, rec2, indptr2, indices2


def test_extra_segment_is_one_pool_with_both_lists():
    q, rec, ip, ix, rec2, ip2, ix2 = _small_problem(11)
    got_out, got_lse = sparse_fwd(q, rec, ip, ix, 0.07, extra=(rec2, ip2, ix2))
    # the same attention over one pool holding both: extra slot s -> N + s
    pool = np.concatenate([rec, rec2])
    n = rec.shape[0]
    rows = []
    for t in range(q.shape[0]):
        a = ix[ip[t]:ip[t + 1]]
        a = np.where((a >= 0) & (a < n), a, -1)
        b = ix2[ip2[t]:ip2[t + 1]]
        b = np.where((b >= 0) & (b < rec2.shape[0]), b + n, -1)
        rows.append(np.concatenate([a, b]))
    ptr = np.concatenate([[0], np.cumsum([len(r) for r in rows])])
    want_out, want_lse = sparse_fwd(q, pool, ptr, np.concatenate(rows), 0.07)
    np.testing.assert_allclose(got_out, want_out, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(got_lse), np.isneginf(want_lse))
    fin = np.isfinite(want_lse)
    np.testing.assert_allclose(got_lse[fin], want_lse[fin], rtol=0, atol=1e-12)


def test_sink_closed_form():
    q, rec, ip, ix, rec2, ip2, ix2 = _small_problem(12)
    sink = np.array([0.5, -3.0, 2.25], dtype=np.float32)
    base_out, base_lse = sparse_fwd(q, rec, ip, ix, 0.07, extra=(rec2, ip2, ix2))
    out, lse = sparse_fwd(q, rec, ip, ix, 0.07, extra=(rec2, ip2, ix2), sink=sink)
    want_lse = np.logaddexp(base_lse, sink.astype(np.float64)[None, :])
    np.testing.assert_allclose(lse, want_lse, rtol=0, atol=1e-12)
    w = np.exp(np.where(np.isneginf(base_lse), -np.inf, base_lse - want_lse))
    np.testing.assert_allclose(out, base_out * w[..., None], rtol=0, atol=1e-12)
    # row 1 has no primary keys; where it has no extra keys either, lse = sink and out = 0
    empty = [t for t in range(q.shape[0]) if np.isneginf(base_lse[t, 0])]
    for t in empty:
        np.testing.assert_array_equal(lse[t], sink.astype(np.float64))
        assert np.all(out[t] == 0)
    # a -inf sink is no sink
    out_n, lse_n = sparse_fwd(q, rec, ip, ix, 0.07, extra=(rec2, ip2, ix2), sink=np.full(3, -np.inf, np.float32))
    np.testing.assert_array_equal(out_n, base_out)
    np.testing.assert_array_equal(lse_n, base_lse)
