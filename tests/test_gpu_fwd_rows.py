"""The forward over many rows of mixed lengths, against the oracle on all
rows (bar as for the forward).  Without split: more rows than the chip
holds workgroups at once, with empty rows, rows of 1 and 2 key tiles,
tile-aligned and ragged long rows, and a long row that is all masked,
interleaved with a period coprime to any power-of-two grid.  With split:
row counts that take each shape of the partial merge, and 130 long rows
whose chunks take the alternating sizes across the plan's 64-row slots."""

import numpy as np
import pytest
import torch

import head_latent_attention_sparse_amd as mla
from oracle import encode_records, sparse_fwd as oracle_fwd
from head_latent_attention_sparse_amd.workloads import bf16_bits
from tests.helpers import assert_fwd_close, plan_chunk_sizes, plan_first_chunks, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCALE = 192 ** -0.5
# period 11: coprime to any power-of-two grid, so neighbouring workgroups see every kind
PATTERN = [0, 1, 64, 65, 700, 128, 2, 200, 0, 191, 300]


def make(seed, t, n, p_bad, heads=16):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((t, heads, 576), generator=g).to(torch.bfloat16)
    kv_c = torch.randn((n, 512), generator=g).to(torch.bfloat16)
    k_pe = torch.randn((n, 64), generator=g).to(torch.bfloat16)
    rec = encode_records(bf16_bits(kv_c), bf16_bits(k_pe))
    lens = np.array([PATTERN[i % len(PATTERN)] for i in range(t)], dtype=np.int64)
    ptr = np.concatenate([[0], np.cumsum(lens)])
    idx = torch.randint(0, n, (int(ptr[-1]),), generator=g).numpy().astype(np.int64)
    r = torch.rand(int(ptr[-1]), generator=g).numpy()
    idx[r < p_bad] = -1
    # one long row entirely masked
    idx[ptr[4]:ptr[5]] = -1
    return q, rec, ptr, idx


def run(q, rec, ptr, idx, dtype, **kw):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    out, lse = mla.sparse_fwd(t(bf16_bits(q)).view(torch.bfloat16), t(rec), t(ptr).to(dtype), t(idx).to(dtype),
                              SCALE, has_invalid=True, return_lse=True, **kw)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("dtype", [torch.int32, torch.int64])
def test_many_mixed_rows(dtype):
    say(f"mixed rows T=1500 dtype={dtype}")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    t = max(1500, 2 * cus + 301)
    q, rec, ptr, idx = make(21, t, 3000, 0.2)
    assert mla.split_workgroups(t, idx.size, cus) == 0
    out, lse = run(q, rec, ptr, idx, dtype)
    ref_out, ref_lse = oracle_fwd(bf16_bits(q), rec, ptr, idx, SCALE)
    assert_fwd_close(out, lse, ref_out, ref_lse, "mixed rows")


def test_many_mixed_rows_with_sink_and_extra_segment():
    say("mixed rows + sink + extra")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    t = max(1200, 2 * cus + 177)
    q, rec, ptr, idx = make(22, t, 2000, 0.1, heads=12)
    g = torch.Generator().manual_seed(23)
    kv2 = torch.randn((900, 512), generator=g).to(torch.bfloat16)
    pe2 = torch.randn((900, 64), generator=g).to(torch.bfloat16)
    rec2 = encode_records(bf16_bits(kv2), bf16_bits(pe2))
    lens2 = np.array([[0, 40, 3, 130][i % 4] for i in range(t)], dtype=np.int64)
    ptr2 = np.concatenate([[0], np.cumsum(lens2)])
    idx2 = torch.randint(-3, 905, (int(ptr2[-1]),), generator=g).numpy().astype(np.int64)
    sink = (torch.randn((12,), generator=g) * 2).numpy().astype(np.float32)
    tt = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    out, lse = run(q, rec, ptr, idx, torch.int32, attn_sink=tt(sink), extra_kv=tt(rec2),
                   extra_indptr=tt(ptr2).to(torch.int32), extra_indices=tt(idx2).to(torch.int32))
    ref_out, ref_lse = oracle_fwd(bf16_bits(q), rec, ptr, idx, SCALE, extra=(rec2, ptr2, idx2), sink=sink)
    assert_fwd_close(out, lse, ref_out, ref_lse, "mixed rows + sink + extra")


@pytest.mark.parametrize("t", [8, 20, 64, 300])
def test_split_merge_shapes(t):
    """Rows the library splits on its own, at row counts whose average chunk
    count per row picks each merge shape (many chunks per row: 8 chunk lanes
    per workgroup; fewer: 4; few: 2); one row empty, one all masked."""
    say(f"split merge shape T={t}")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    g = torch.Generator().manual_seed(30 + t)
    n = 4096
    q = torch.randn((t, 16, 576), generator=g).to(torch.bfloat16)
    kv_c = torch.randn((n, 512), generator=g).to(torch.bfloat16)
    k_pe = torch.randn((n, 64), generator=g).to(torch.bfloat16)
    rec = encode_records(bf16_bits(kv_c), bf16_bits(k_pe))
    lens = torch.randint(520, 1500 if t < 64 else 700, (t,), generator=g).numpy().astype(np.int64)
    lens[t // 2] = 0
    ptr = np.concatenate([[0], np.cumsum(lens)])
    idx = torch.randint(0, n, (int(ptr[-1]),), generator=g).numpy().astype(np.int64)
    idx[torch.rand(int(ptr[-1]), generator=g).numpy() < 0.1] = -1
    idx[ptr[1]:ptr[2]] = -1
    assert mla.split_workgroups(t, idx.size, cus) > 0
    out, lse = run(q, rec, ptr, idx, torch.int32)
    ref_out, ref_lse = oracle_fwd(bf16_bits(q), rec, ptr, idx, SCALE)
    assert_fwd_close(out, lse, ref_out, ref_lse, f"split T={t}")


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("layout", ["equal", "alternating", "two_shifted", "equal_int64"])
def test_row_start_guess(layout, split):
    """nnz a multiple of T makes each one-row workgroup guess that row t
    starts at t * nnz / T and fetch its first entries there before indptr
    arrives; workgroups whose guess indptr confirms use it, the others fetch
    again.  Layouts: all rows equal; lengths alternating L + 5, L - 5 (even
    rows start at the guess, odd rows elsewhere); two rows shifted by 7
    entries inside an otherwise equal layout.  Without split: 600 rows of
    150; the same layouts also go through the library's split pass (16 rows
    of 2000), which takes no guess.  Against the oracle on all rows."""
    say(f"row start guess: {layout} split={split}")
    t, length, n = (16, 2000, 3000) if split else (600, 150, 3000)
    g = torch.Generator().manual_seed(50)
    q = torch.randn((t, 16, 576), generator=g).to(torch.bfloat16)
    kv_c = torch.randn((n, 512), generator=g).to(torch.bfloat16)
    k_pe = torch.randn((n, 64), generator=g).to(torch.bfloat16)
    rec = encode_records(bf16_bits(kv_c), bf16_bits(k_pe))
    ptr = np.arange(t + 1, dtype=np.int64) * length
    if layout == "alternating":
        ptr[1:-1:2] += 5
    elif layout == "two_shifted":
        ptr[t // 50 + 1] += 7
        ptr[t // 2] -= 7
    idx = torch.randint(0, n, (t * length,), generator=g).numpy().astype(np.int64)
    idx[torch.rand(t * length, generator=g).numpy() < 0.1] = -1
    dtype = torch.int64 if layout == "equal_int64" else torch.int32
    wgs = mla.split_workgroups(t, idx.size, torch.cuda.get_device_properties(0).multi_processor_count)
    assert (wgs > 0) == split
    out, lse = run(q, rec, ptr, idx, dtype)
    ref_out, ref_lse = oracle_fwd(bf16_bits(q), rec, ptr, idx, SCALE)
    assert_fwd_close(out, lse, ref_out, ref_lse, f"guess {layout} split={split}")


@pytest.mark.parametrize("t", [8, 20, 64])
@pytest.mark.parametrize("with_sink", [False, True])
def test_split_without_lse(t, with_sink):
    """The split pass and merge when no LSE is asked for (the merge then
    writes out only), with and without a sink, at the three merge shapes the
    row counts pick; out against the oracle."""
    say(f"split without lse T={t} sink={with_sink}")
    g = torch.Generator().manual_seed(80 + t)
    n = 4096
    q = torch.randn((t, 16, 576), generator=g).to(torch.bfloat16)
    kv_c = torch.randn((n, 512), generator=g).to(torch.bfloat16)
    k_pe = torch.randn((n, 64), generator=g).to(torch.bfloat16)
    rec = encode_records(bf16_bits(kv_c), bf16_bits(k_pe))
    lens = torch.randint(600, 3000, (t,), generator=g).numpy().astype(np.int64)
    ptr = np.concatenate([[0], np.cumsum(lens)])
    idx = torch.randint(-1, n, (int(ptr[-1]),), generator=g).numpy().astype(np.int64)
    sink = (torch.randn((16,), generator=g) * 2).numpy().astype(np.float32) if with_sink else None
    assert mla.split_workgroups(t, idx.size, torch.cuda.get_device_properties(0).multi_processor_count) > 0
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    out, lse = mla.sparse_fwd(dev(bf16_bits(q)).view(torch.bfloat16), dev(rec), dev(ptr).to(torch.int32),
                              dev(idx).to(torch.int32), SCALE, has_invalid=True, return_lse=False,
                              attn_sink=dev(sink) if with_sink else None)
    torch.cuda.synchronize()
    assert lse is None
    ref_out, ref_lse = oracle_fwd(bf16_bits(q), rec, ptr, idx, SCALE, sink=sink)
    assert_fwd_close(out, None, ref_out, ref_lse, f"split without lse T={t}")


def test_split_many_rows_alternating_chunks():
    """130 split rows (three 64-row slots of the plan's scans) of 3000-9000
    entries, where the alternating chunk sizes fit the bound (the plan's rule
    restated in tests.helpers says so): rows start on even and odd chunks
    across the slots, so the parity carried between slots decides every
    later row's chunks.  One row empty, one all masked, 10% of entries
    masked; all rows against the oracle."""
    t = 130
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    g = torch.Generator().manual_seed(61)
    n = 8192
    q = torch.randn((t, 16, 576), generator=g).to(torch.bfloat16)
    kv_c = torch.randn((n, 512), generator=g).to(torch.bfloat16)
    k_pe = torch.randn((n, 64), generator=g).to(torch.bfloat16)
    rec = encode_records(bf16_bits(kv_c), bf16_bits(k_pe))
    lens = torch.randint(3000, 9001, (t,), generator=g).numpy().astype(np.int64)
    lens[70] = 0
    ptr = np.concatenate([[0], np.cumsum(lens)])
    idx = torch.randint(0, n, (int(ptr[-1]),), generator=g).numpy().astype(np.int64)
    idx[torch.rand(int(ptr[-1]), generator=g).numpy() < 0.1] = -1
    idx[ptr[100]:ptr[101]] = -1
    bound = mla.split_workgroups(t, idx.size, cus)
    assert bound > 0
    big, small = plan_chunk_sizes(lens, bound)
    first = plan_first_chunks(lens, big, small)
    assert big > small, "the alternating sizes must fit for this test to reach them"
    parities = [x % 2 for x in first[64:t]]
    assert 0 < sum(parities) < t - 64, "later slots must hold rows starting on both parities"
    say(f"split T={t}, bound {bound}: chunks of {big} / {small} entries, {first[-1]} in all")
    out, lse = run(q, rec, ptr, idx, torch.int32)
    ref_out, ref_lse = oracle_fwd(bf16_bits(q), rec, ptr, idx, SCALE)
    assert_fwd_close(out, lse, ref_out, ref_lse, f"split T={t} alternating chunks")


@pytest.mark.parametrize("t", [63, 64, 65, 127, 128, 129, 255, 256, 257, 511])
def test_split_row_counts_across_plan_slots(t):
    """Row counts on both sides of the plan's 64-row slots (lane l holds rows
    l, l + 64, ...; a slot past the last row reads indptr[T]), up to the
    split pass's 512-row limit, rows of 520-2600 entries, one empty: all
    rows against the oracle, whichever chunk sizes the rule picks."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    g = torch.Generator().manual_seed(70 + t)
    n = 4096
    q = torch.randn((t, 16, 576), generator=g).to(torch.bfloat16)
    kv_c = torch.randn((n, 512), generator=g).to(torch.bfloat16)
    k_pe = torch.randn((n, 64), generator=g).to(torch.bfloat16)
    rec = encode_records(bf16_bits(kv_c), bf16_bits(k_pe))
    lens = torch.randint(520, 2601, (t,), generator=g).numpy().astype(np.int64)
    lens[t - 1 if t % 2 else t // 2] = 0
    ptr = np.concatenate([[0], np.cumsum(lens)])
    idx = torch.randint(0, n, (int(ptr[-1]),), generator=g).numpy().astype(np.int64)
    idx[torch.rand(int(ptr[-1]), generator=g).numpy() < 0.05] = -1
    bound = mla.split_workgroups(t, idx.size, cus)
    assert bound > 0
    big, small = plan_chunk_sizes(lens, bound)
    say(f"split T={t}, bound {bound}: chunks of {big} / {small} entries")
    out, lse = run(q, rec, ptr, idx, torch.int32)
    ref_out, ref_lse = oracle_fwd(bf16_bits(q), rec, ptr, idx, SCALE)
    assert_fwd_close(out, lse, ref_out, ref_lse, f"split T={t} across plan slots")
