"""GPU parity of mla_cache_insert: records must equal the oracle writer's bytes.

Bar: bit-exact (the record is an integer byte string); untouched slots keep
their bytes.
"""

import numpy as np
import pytest
import torch

import head_latent_attention_sparse_amd as mla
from head_latent_attention_sparse_amd import workloads
from tests.helpers import oracle_encode, oracle_pool, say
from tests.test_oracle_records import _random_tokens

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def gpu_insert(pool_t, kv_c, k_pe, slots):
    mla.cache_insert(kv_c.to(DEV), k_pe.to(DEV), slots.to(DEV), pool_t)
    torch.cuda.synchronize()


@pytest.mark.parametrize("kind", ["std1", "std2", "heavy", "tiny", "huge", "zero_tiles", "ties"])
def test_insert_bit_exact(kind):
    say(f"insert kind={kind}")
    kv_c, k_pe = _random_tokens(101, 1000, kind)
    n_rec = 1200
    g = torch.Generator().manual_seed(5)
    slots = torch.randperm(n_rec, generator=g)[:1000].to(torch.int64)
    slots[torch.rand(1000, generator=g) < 0.1] = -1
    slots[::97] = n_rec + 3  # outside the pool: skipped
    pool = torch.full((n_rec, 656), 0xA5, dtype=torch.uint8, device=DEV)
    gpu_insert(pool, kv_c, k_pe, slots)
    want = np.full((n_rec, 656), 0xA5, dtype=np.uint8)
    keep = ((slots >= 0) & (slots < n_rec)).numpy()
    want[slots.numpy()[keep]] = oracle_encode(kv_c, k_pe)[keep]
    got = pool.cpu().numpy()
    bad = np.nonzero(np.any(got != want, axis=1))[0]
    assert bad.size == 0, f"{bad.size} records differ, first slot {bad[:5]}"


@pytest.mark.parametrize("view", ["flat", "paged", "n11", "n1"])
def test_insert_pool_views_and_strided_inputs(view):
    say(f"insert view={view}")
    g = torch.Generator().manual_seed(9)
    n = 300
    wide = torch.randn((n, 1024), generator=g).to(torch.bfloat16)
    kv_c = wide[:, 256:768]  # row stride 1024
    k_pe = torch.randn((n, 1, 64), generator=g).to(torch.bfloat16)
    slots = torch.randperm(512, generator=g)[:n].to(torch.int64)
    base = torch.zeros(512 * 656, dtype=torch.uint8, device=DEV)
    pool = {"flat": base.view(512, 656), "paged": base.view(8, 64, 656),
            "n11": base.view(512, 1, 1, 656), "n1": base.view(512, 1, 656)}[view]
    mla.cache_insert(kv_c.to(DEV), k_pe.to(DEV), slots.to(DEV), pool)
    torch.cuda.synchronize()
    want = np.zeros((512, 656), np.uint8)
    want[slots.numpy()] = oracle_encode(kv_c.contiguous(), k_pe)
    assert np.array_equal(base.view(512, 656).cpu().numpy(), want)


def test_insert_attend_pool_bit_exact():
    say("insert: the insert + attend workload's full pool")
    w = workloads.insert_attend()
    pool = torch.zeros((w.num_records, 656), dtype=torch.uint8, device=DEV)
    for b in w.setup_inserts + w.step_inserts:
        mla.cache_insert(b.kv_c.to(DEV), b.k_pe.to(DEV), b.slots.to(DEV), pool)
    torch.cuda.synchronize()
    want = oracle_pool(w.num_records, w.setup_inserts + w.step_inserts)
    got = pool.cpu().numpy()
    bad = np.nonzero(np.any(got != want, axis=1))[0]
    assert bad.size == 0, f"{bad.size} records differ, first slots {bad[:5]}"


def test_insert_zero_tokens():
    pool = torch.full((4, 656), 7, dtype=torch.uint8, device=DEV)
    e = torch.zeros((0, 512), dtype=torch.bfloat16, device=DEV)
    mla.cache_insert(e, torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV),
                     torch.zeros(0, dtype=torch.int64, device=DEV), pool)
    torch.cuda.synchronize()
    assert torch.all(pool == 7)


def test_insert_rejects_padded_pages():
    base = torch.zeros(4 * 70 * 656, dtype=torch.uint8, device=DEV).view(4, 70, 656)[:, :64]
    with pytest.raises(ValueError):
        mla.cache_insert(torch.zeros((1, 512), dtype=torch.bfloat16, device=DEV),
                         torch.zeros((1, 64), dtype=torch.bfloat16, device=DEV),
                         torch.zeros(1, dtype=torch.int64, device=DEV), base)
