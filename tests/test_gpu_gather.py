"""GPU parity of mla_gather_upconvert against the oracle: the bf16 workspace
rows must be bit-exact (one float32 product per value, then the same bf16
rounding on both sides; rope bits copied)."""

import numpy as np
import pytest
import torch

import head_latent_attention_sparse_amd as mla
from head_latent_attention_sparse_amd import workloads
from head_latent_attention_sparse_amd.workloads import bf16_bits
from oracle import gather_upconvert as oracle_gather
from tests.helpers import oracle_pool, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def build(w):
    """device pool [nb, bs, 656] and the oracle's pool; checks they are equal."""
    pool = torch.zeros((w.num_records // w.block_size, w.block_size, 656), dtype=torch.uint8, device=DEV)
    for b in w.setup_inserts:
        mla.cache_insert(b.kv_c.to(DEV), b.k_pe.to(DEV), b.slots.to(DEV), pool)
    want = oracle_pool(w.num_records, w.setup_inserts)
    assert np.array_equal(pool.cpu().numpy().reshape(-1, 656), want), "pool bytes differ"
    return pool, want


def compare(got, want):
    bad = np.nonzero(np.any(got != want, axis=1))[0]
    assert bad.size == 0, f"{bad.size} rows differ, first {bad[:5]}"


@pytest.mark.parametrize("bs,frac,starts", [(16, 0.5, True), (64, 0.0, False), (1, 0.3, True), (128, 0.9, True)])
def test_gather_bit_exact(bs, frac, starts):
    say(f"gather bs={bs} frac={frac} starts={starts}")
    w = workloads.context_gather(batch=9, len_lo=1, len_hi=700, block_size=bs, start_frac=frac)
    pool, want_pool = build(w)
    table, cu = w.block_table.clone(), w.cu_seq_lens
    table[2, 1] = -1                                       # a hole
    table[3, 0] = w.num_records // bs + 3                  # a block outside the pool
    n = w.num_tokens + 5                                   # rows past the chunk: zero
    st = w.seq_starts if starts else None
    got = mla.gather_upconvert(pool, table.to(DEV), cu.to(DEV), n, seq_starts=st.to(DEV) if starts else None)
    torch.cuda.synchronize()
    compare(bf16_bits(got), oracle_gather(want_pool, bs, table.numpy(), cu.numpy(),
                                          st.numpy() if starts else None, n))


def test_gather_into_a_wider_workspace_and_flat_pool():
    say("gather wide workspace")
    w = workloads.context_gather(batch=4, len_lo=50, len_hi=300, block_size=32, start_frac=0.2)
    pool, want_pool = build(w)
    n = w.num_tokens
    ws = torch.full((n + 3, 640), -3.0, dtype=torch.bfloat16, device=DEV)
    flat = pool.view(-1, 656)
    mla.gather_upconvert(flat, w.block_table.to(DEV), w.cu_seq_lens.to(DEV), n,
                         seq_starts=w.seq_starts.to(DEV), block_size=32, dst=ws[:n, :576])
    torch.cuda.synchronize()
    compare(bf16_bits(ws[:n, :576]), oracle_gather(want_pool, 32, w.block_table.numpy(), w.cu_seq_lens.numpy(),
                                                   w.seq_starts.numpy(), n))
    assert torch.all(ws[:, 576:].cpu() == -3.0) and torch.all(ws[n:].cpu() == -3.0), "wrote outside dst"


def test_gather_full_chunk():
    """The measured shape: 64 requests, contexts of 1024..8192 tokens, blocks of 64."""
    say("gather full chunk")
    w = workloads.context_gather()
    pool, want_pool = build(w)
    got = mla.gather_upconvert(pool, w.block_table.to(DEV), w.cu_seq_lens.to(DEV), w.num_tokens,
                               seq_starts=w.seq_starts.to(DEV))
    torch.cuda.synchronize()
    compare(bf16_bits(got), oracle_gather(want_pool, w.block_size, w.block_table.numpy(), w.cu_seq_lens.numpy(),
                                          w.seq_starts.numpy(), w.num_tokens))


def test_gather_empty_and_rejections():
    say("gather empty / rejections")
    pool = torch.zeros((4, 16, 656), dtype=torch.uint8, device=DEV)
    table = torch.zeros((2, 4), dtype=torch.int32, device=DEV)
    cu = torch.tensor([0, 3, 5], dtype=torch.int32, device=DEV)
    assert mla.gather_upconvert(pool, table, cu, 0).shape == (0, 576)
    with pytest.raises(ValueError):
        mla.gather_upconvert(pool, table.to(torch.int64), cu, 5)
    with pytest.raises(ValueError):
        mla.gather_upconvert(pool, table, cu[:2], 5)
    odd = torch.empty((5 * 580 + 4,), dtype=torch.bfloat16, device=DEV)[4:].view(5, 580)[:, :576]
    with pytest.raises(ValueError):
        mla.gather_upconvert(pool, table, cu, 5, dst=odd)  # misaligned rows
