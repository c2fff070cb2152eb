"""A record pool past 4 GiB: slot * 656 no longer fits 32 bits, so every
kernel that addresses records must do it in 64 bits.  The pool has 7,000,000
records (4.59 GB); only the slots the test uses are written, by the GPU
insert and by the decode epilogue, and the forward, the sink / second-segment
forward and the gather read them back.  Compared with the oracle on a
sub-pool of exactly those slots."""

import numpy as np
import pytest
import torch

import head_latent_attention_sparse_amd as mla
from oracle import encode_records, gather_upconvert, sparse_fwd as oracle_fwd
from head_latent_attention_sparse_amd.workloads import bf16_bits
from tests.helpers import assert_fwd_close, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
N = 7_000_000  # 7e6 * 656 B = 4.59 GB > 2^32


def test_pool_past_4gib():
    say("large pool: 7,000,000 records (4.59 GB)")
    g = torch.Generator().manual_seed(77)
    pool = torch.zeros((N, 656), dtype=torch.uint8, device=DEV)
    n_used = 600
    slots = torch.cat([torch.arange(N - 300, N), torch.randint(6_540_000, N - 300, (300,), generator=g)])
    slots = torch.unique(slots)[:n_used].to(torch.int64)
    n_used = slots.numel()
    kv_c = torch.randn((n_used, 512), generator=g).to(torch.bfloat16)
    k_pe = torch.randn((n_used, 64), generator=g).to(torch.bfloat16)
    mla.cache_insert(kv_c.to(DEV), k_pe.to(DEV), slots.to(DEV), pool)
    torch.cuda.synchronize()
    want = encode_records(bf16_bits(kv_c), bf16_bits(k_pe))
    got = pool[slots.to(DEV)].cpu().numpy()
    assert np.array_equal(got, want), "insert past 4 GiB differs"

    # forward over rows that list the high slots (and one past the end)
    t_count, heads = 12, 16
    q = torch.randn((t_count, heads, 576), generator=g).to(torch.bfloat16)
    rows = [slots[torch.randint(0, n_used, (int(torch.randint(1, 400, (1,), generator=g)),), generator=g)]
            for _ in range(t_count)]
    rows[3] = torch.cat([rows[3], torch.tensor([N, N + 5, -1])])  # outside the pool: masked
    indptr = torch.tensor([0] + [int(r.numel()) for r in rows]).cumsum(0).to(torch.int32)
    indices = torch.cat(rows).to(torch.int32)
    out, lse = mla.sparse_fwd(q.to(DEV), pool, indptr.to(DEV), indices.to(DEV), 192 ** -0.5, has_invalid=True,
                              return_lse=True)
    torch.cuda.synchronize()
    # oracle on the sub-pool: slot s -> its position in `slots`
    lut = {int(s): i for i, s in enumerate(slots.tolist())}
    sub_idx = np.array([lut.get(int(x), -1) for x in indices.tolist()], dtype=np.int64)
    ref_out, ref_lse = oracle_fwd(bf16_bits(q), want, indptr.numpy(), sub_idx, 192 ** -0.5)
    assert_fwd_close(out, lse, ref_out, ref_lse, "fwd past 4 GiB")

    # the same rows as a second segment over the big pool (sink on), primary lists empty
    empty_ptr = torch.zeros(t_count + 1, dtype=torch.int32, device=DEV)
    sink = torch.randn((heads,), generator=g)
    small = torch.zeros((4, 656), dtype=torch.uint8, device=DEV)
    out2, lse2 = mla.sparse_fwd(q.to(DEV), small, empty_ptr, torch.zeros(0, dtype=torch.int32, device=DEV),
                                192 ** -0.5, return_lse=True, attn_sink=sink.to(DEV), extra_kv=pool,
                                extra_indptr=indptr.to(DEV), extra_indices=indices.to(DEV))
    torch.cuda.synchronize()
    ref2 = oracle_fwd(bf16_bits(q), np.zeros((4, 656), np.uint8), np.zeros(t_count + 1, np.int64),
                      np.zeros(0, np.int64), 192 ** -0.5, extra=(want, indptr.numpy(), sub_idx), sink=sink.numpy())
    assert_fwd_close(out2, lse2, ref2[0], ref2[1], "second segment past 4 GiB")

    # gather through a block table whose blocks lie past 4 GiB (block size 100)
    bs = 100
    blocks = torch.tensor([69_999, 69_990, 65_500], dtype=torch.int32)
    table = blocks.view(1, 3)
    cu = torch.tensor([0, 250], dtype=torch.int32)
    ws = mla.gather_upconvert(pool, table.to(DEV), cu.to(DEV), 250, block_size=bs)
    torch.cuda.synchronize()
    rec_ids = [int(blocks[p // bs]) * bs + p % bs for p in range(250)]
    # the oracle's records for those slots: its own encoding where the test inserted, zero bytes elsewhere
    recs = np.stack([want[lut[r]] if r in lut else np.zeros(656, np.uint8) for r in rec_ids])
    want_ws = gather_upconvert(recs, 1, np.arange(250).reshape(1, 250), np.array([0, 250]), None, 250)
    assert np.array_equal(bf16_bits(ws), want_ws), "gather past 4 GiB differs"
    del pool
    torch.cuda.empty_cache()
