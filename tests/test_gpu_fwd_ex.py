"""GPU parity of mla_sparse_fwd_ex (attention sink and a second KV segment)
against the oracle, with the forward's bar (|out - ref| <= 1e-2 + 1e-2|ref|,
|lse - ref| <= 2e-3, -inf exactly where the oracle has it).

Covers the sink alone, the second segment alone and both, without split,
with forced chunks (which then run across the two lists of a row) and with
the library's own split plan; rows empty in one or both lists; masked and
out-of-pool entries in both lists; int32 and int64 indices; sinks of -inf
and sinks that dominate the row.
"""

import numpy as np
import pytest
import torch

import head_latent_attention_sparse_amd as mla
from oracle import encode_records, sparse_fwd as oracle_fwd
from head_latent_attention_sparse_amd.workloads import bf16_bits
from tests.helpers import assert_fwd_close, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCALE = 192 ** -0.5


def pool(g, n):
    kv_c = torch.randn((n, 512), generator=g).to(torch.bfloat16)
    k_pe = torch.randn((n, 64), generator=g).to(torch.bfloat16)
    return encode_records(bf16_bits(kv_c), bf16_bits(k_pe))  # the oracle's writer (pinned bit-exact to the GPU insert)


def csr(g, lengths, n, p_bad):
    lengths = np.asarray(lengths, dtype=np.int64)
    ptr = np.concatenate([[0], np.cumsum(lengths)])
    idx = torch.randint(0, n, (int(ptr[-1]),), generator=g).numpy().astype(np.int64)
    r = torch.rand(int(ptr[-1]), generator=g).numpy()
    idx[r < p_bad / 2] = -1
    idx[(r >= p_bad / 2) & (r < p_bad)] = n + 7  # outside the pool
    return ptr, idx


def run(q, rec, ptr, idx, rec2=None, ptr2=None, idx2=None, sink=None, dtype=torch.int32, chunk_tiles=0):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    extra = {}
    if rec2 is not None:
        extra = dict(extra_kv=t(rec2), extra_indptr=t(ptr2).to(dtype), extra_indices=t(idx2).to(dtype))
    out, lse = mla.sparse_fwd(t(bf16_bits(q)).view(torch.bfloat16), t(rec), t(ptr).to(dtype), t(idx).to(dtype),
                              SCALE, has_invalid=True, return_lse=True, chunk_tiles=chunk_tiles,
                              attn_sink=t(sink) if sink is not None else None, **extra)
    torch.cuda.synchronize()
    want = oracle_fwd(bf16_bits(q), rec, ptr, idx, SCALE,
                      extra=(rec2, ptr2, idx2) if rec2 is not None else None, sink=sink)
    return out, lse, want


def problem(seed, t=37, h=16, n=700, n2=500, max1=300, max2=200):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((t, h, 576), generator=g).to(torch.bfloat16)
    rec, rec2 = pool(g, n), pool(g, n2)
    l1 = torch.randint(0, max1 + 1, (t,), generator=g).numpy()
    l2 = torch.randint(0, max2 + 1, (t,), generator=g).numpy()
    l1[0], l2[0] = 0, 0       # empty in both lists
    l1[1], l2[2] = 0, 0       # empty in one list
    l1[3], l2[3] = 64, 64     # tile-aligned
    ptr, idx = csr(g, l1, n, 0.15)
    ptr2, idx2 = csr(g, l2, n2, 0.15)
    sink = (torch.randn((h,), generator=g) * 2).numpy().astype(np.float32)
    sink[1] = -np.inf
    sink[2] = 30.0  # dominates every row
    return q, rec, ptr, idx, rec2, ptr2, idx2, sink


@pytest.mark.parametrize("chunk_tiles", [0, 1, 3])
def test_sink_only(chunk_tiles):
    say(f"fwd_ex sink chunk_tiles={chunk_tiles}")
    q, rec, ptr, idx, _, _, _, sink = problem(1)
    out, lse, (ro, rl) = run(q, rec, ptr, idx, sink=sink, chunk_tiles=chunk_tiles)
    assert_fwd_close(out, lse, ro, rl, "sink")


@pytest.mark.parametrize("chunk_tiles", [0, 1, 3])
@pytest.mark.parametrize("dtype", [torch.int32, torch.int64])
def test_extra_segment(chunk_tiles, dtype):
    say(f"fwd_ex extra chunk_tiles={chunk_tiles} dtype={dtype}")
    q, rec, ptr, idx, rec2, ptr2, idx2, _ = problem(2)
    out, lse, (ro, rl) = run(q, rec, ptr, idx, rec2, ptr2, idx2, dtype=dtype, chunk_tiles=chunk_tiles)
    assert_fwd_close(out, lse, ro, rl, "extra")


@pytest.mark.parametrize("chunk_tiles", [0, 2])
def test_sink_and_extra_segment(chunk_tiles):
    say(f"fwd_ex sink+extra chunk_tiles={chunk_tiles}")
    q, rec, ptr, idx, rec2, ptr2, idx2, sink = problem(3, h=12)
    out, lse, (ro, rl) = run(q, rec, ptr, idx, rec2, ptr2, idx2, sink=sink, chunk_tiles=chunk_tiles)
    assert_fwd_close(out, lse, ro, rl, "sink+extra")


def test_library_split_plan_over_both_lists():
    """8 long rows: the library splits them; chunks straddle the two lists."""
    say("fwd_ex auto split, 8 rows")
    q, rec, ptr, idx, rec2, ptr2, idx2, sink = problem(4, t=8, n=3000, n2=2000, max1=9000, max2=3000)
    assert mla.split_workgroups(8, idx.size + idx2.size, torch.cuda.get_device_properties(0).multi_processor_count) > 0
    out, lse, (ro, rl) = run(q, rec, ptr, idx, rec2, ptr2, idx2, sink=sink)
    assert_fwd_close(out, lse, ro, rl, "auto split")


def test_empty_extra_list_matches_plain_forward():
    say("fwd_ex empty extra list")
    q, rec, ptr, idx, rec2, _, _, _ = problem(5, t=20)
    ptr2 = np.zeros(21, np.int64)
    out, lse, (ro, rl) = run(q, rec, ptr, idx, rec2, ptr2, np.zeros(0, np.int64))
    assert_fwd_close(out, lse, ro, rl, "empty extra")
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    plain, plain_lse = mla.sparse_fwd(t(bf16_bits(q)).view(torch.bfloat16), t(rec), t(ptr).to(torch.int32),
                                      t(idx).to(torch.int32), SCALE, has_invalid=True, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(plain, out) and torch.equal(plain_lse, lse)


def test_binding_rejections():
    q = torch.zeros((2, 4, 576), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((8, 656), dtype=torch.uint8, device=DEV)
    ip = torch.zeros(3, dtype=torch.int32, device=DEV)
    ix = torch.zeros(0, dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        mla.sparse_fwd(q, kv, ip, ix, 1.0, extra_kv=kv, extra_indptr=ip)  # no extra_indices
    with pytest.raises(ValueError):
        mla.sparse_fwd(q, kv, ip, ix, 1.0, extra_kv=kv, extra_indptr=ip, extra_indices=ix.to(torch.int64))
    with pytest.raises(ValueError):
        mla.sparse_fwd(q, kv, ip, ix, 1.0, attn_sink=torch.zeros(3, device=DEV))


def test_sparse_prefill_full_with_sink_and_extra_sampled():
    """The measured variant (bench.py --with-sink-extra): the sparse prefill
    workload at full size plus sinks and a 256-slot second segment per row;
    sampled rows against the oracle, properties on all rows."""
    from head_latent_attention_sparse_amd import workloads
    from tests.helpers import oracle_subpool, remap_rows

    say("fwd_ex sparse prefill full + sink + extra, sampled rows")
    w = workloads.sparse_prefill()
    seg = workloads.extra_segment(w.num_tokens, w.num_heads)
    pool = torch.zeros((w.num_records, 656), dtype=torch.uint8, device=DEV)
    for b in w.setup_inserts:
        mla.cache_insert(b.kv_c.to(DEV), b.k_pe.to(DEV), b.slots.to(DEV), pool)
    pool2 = torch.zeros((seg.num_records, 656), dtype=torch.uint8, device=DEV)
    mla.cache_insert(seg.insert.kv_c.to(DEV), seg.insert.k_pe.to(DEV), seg.insert.slots.to(DEV), pool2)
    out, lse = mla.sparse_fwd(w.q.to(DEV), pool, w.indptr.to(DEV), w.indices.to(DEV), w.softmax_scale,
                              has_invalid=True, return_lse=True, attn_sink=seg.sink.to(DEV), extra_kv=pool2,
                              extra_indptr=seg.indptr.to(DEV), extra_indices=seg.indices.to(DEV))
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()  # every row has extra keys
    rec2 = encode_records(bf16_bits(seg.insert.kv_c), bf16_bits(seg.insert.k_pe))
    assert np.array_equal(pool2.cpu().numpy(), rec2), "second pool differs from the oracle writer"
    indptr, indices = w.indptr.numpy(), w.indices.numpy()
    empty = [t for t in range(w.num_tokens) if np.all(indices[indptr[t]:indptr[t + 1]] < 0)]
    rows = sorted(set([0, 1, 2047, 4095] + empty[:2]))
    needed = np.concatenate([indices[indptr[t]:indptr[t + 1]] for t in rows])
    uniq, sub = oracle_subpool(w.num_records, w.setup_inserts, needed)
    ptr, ind = remap_rows(indptr, indices, rows, uniq, w.num_records)
    eptr_full, eind_full = seg.indptr.numpy().astype(np.int64), seg.indices.numpy().astype(np.int64)
    eptr = np.concatenate([[0], np.cumsum([eptr_full[t + 1] - eptr_full[t] for t in rows])])
    eind = np.concatenate([eind_full[eptr_full[t]:eptr_full[t + 1]] for t in rows])
    ref_out, ref_lse = oracle_fwd(bf16_bits(w.q)[rows], sub, ptr, ind, w.softmax_scale,
                                  extra=(rec2, eptr, eind), sink=seg.sink.numpy())
    sel = torch.tensor(rows, dtype=torch.long, device=DEV)
    assert_fwd_close(out[sel], lse[sel], ref_out, ref_lse, "prefill+sink+extra")
