"""The forward at the index-count limit: just under 2^29 CSR entries (the
most the C ABI accepts), int32 indices, once with one workgroup per row
(4096 rows of 131,071 entries) and once through the split pass (511 rows of
1,050,623 entries, the last one entry shorter: rows of one length above
CU-many rows take one workgroup each).  The entries are drawn on the device by torch's seeded
generator over a 4096-record pool (5% masked); the oracle checks sampled
rows from the same index values.  A 1M-entry row is too big for the oracle
in one piece, so it is computed in 8 slices and the slices are combined by
the oracle's LSE merge (pinned against the unsplit row on the CPU).
"""

import numpy as np
import pytest
import torch

import head_latent_attention_sparse_amd as mla
from oracle import encode_records, merge_partials, sparse_fwd as oracle_fwd
from head_latent_attention_sparse_amd.workloads import bf16_bits
from tests.helpers import assert_fwd_close, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCALE = 192 ** -0.5
MAX_INDICES = 1 << 29
N = 4096


def problem(t, per_row, seed, short_last=False):
    assert t * per_row < MAX_INDICES
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((t, 16, 576), generator=g).to(torch.bfloat16)
    kv_c = torch.randn((N, 512), generator=g).to(torch.bfloat16)
    k_pe = torch.randn((N, 64), generator=g).to(torch.bfloat16)
    rec = encode_records(bf16_bits(kv_c), bf16_bits(k_pe))
    gd = torch.Generator(device=DEV).manual_seed(seed)
    nnz = t * per_row - (1 if short_last else 0)
    idx = torch.randint(0, N, (nnz,), generator=gd, device=DEV, dtype=torch.int32)
    mask = torch.rand((nnz,), generator=gd, device=DEV) < 0.05
    idx.masked_fill_(mask, -1)
    del mask
    ptr = torch.arange(t + 1, dtype=torch.int64) * per_row
    ptr[-1] = nnz
    return q, rec, ptr, idx


def oracle_row(q, rec, idx_row, slices):
    """Oracle result of one row, computed over `slices` pieces and merged."""
    q1 = bf16_bits(q)[None]
    outs, lses = [], []
    for piece in np.array_split(idx_row, slices):
        o, l = oracle_fwd(q1, rec, np.array([0, piece.size]), piece, SCALE)
        outs.append(o[0])
        lses.append(l[0])
    o, l = merge_partials(outs, lses)
    return o[None], l[None]


@pytest.mark.parametrize("t,per_row,rows,slices", [
    (4096, 131071, [0, 2047, 4095], 2),
    (511, 1050623, [510], 8),
])
def test_forward_at_the_index_limit(t, per_row, rows, slices):
    say(f"max nnz: T={t} x {per_row} = {t * per_row} entries")
    q, rec, ptr, idx = problem(t, per_row, 60 + t, short_last=t < 512)
    split = mla.split_workgroups(t, idx.numel(), torch.cuda.get_device_properties(0).multi_processor_count)
    assert (split > 0) == (t < 512)
    out, lse = mla.sparse_fwd(q.to(DEV), torch.from_numpy(rec).to(DEV), ptr.to(torch.int32).to(DEV), idx,
                              SCALE, has_invalid=True, return_lse=True)
    torch.cuda.synchronize()
    say("forward done; checking sampled rows")
    for r in rows:
        idx_row = idx[int(ptr[r]):int(ptr[r + 1])].cpu().numpy().astype(np.int64)
        ref_out, ref_lse = oracle_row(q[r], rec, idx_row, slices)
        assert_fwd_close(out[r:r + 1], lse[r:r + 1], ref_out, ref_lse, f"row {r}")
        say(f"row {r} ok")
