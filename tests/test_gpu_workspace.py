"""The library-owned split-KV workspace: mla_sparse_fwd called through the C
ABI with workspace NULL after mla_workspace_reserve of a small size, so the
library grows its buffer (a new hipMalloc; the old buffer is retired, not
freed) on the first split call and again for a call that needs more; each
result must equal, bit for bit, the same call with a caller-provided
workspace (the binding's path).  A graph captured on the library's buffer
must still replay correctly after the buffer has been replaced by a larger
one."""


import ctypes

import pytest
import torch

import head_latent_attention_sparse_amd as mla
from head_latent_attention_sparse_amd import ops
from oracle import encode_records
from head_latent_attention_sparse_amd.workloads import bf16_bits
from tests.helpers import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCALE = 192 ** -0.5


def problem(seed, t, heads, n, length):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((t, heads, 576), generator=g).to(torch.bfloat16).to(DEV)
    kv = torch.randn((n, 512), generator=g).to(torch.bfloat16)
    pe = torch.randn((n, 64), generator=g).to(torch.bfloat16)
    pool = torch.from_numpy(encode_records(bf16_bits(kv), bf16_bits(pe))).to(DEV)
    ptr = torch.arange(t + 1, dtype=torch.int32) * length
    idx = torch.randint(-1, n, (t * length,), generator=g, dtype=torch.int32)
    return q, pool, ptr.to(DEV), idx.to(DEV)


def fwd_library_workspace(q, pool, ptr, idx, chunk_tiles=0):
    t, heads = q.shape[0], q.shape[1]
    out = torch.empty((t, heads, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((t, heads), dtype=torch.float32, device=DEV)
    L = mla.lib()
    st = L.mla_sparse_fwd(q.data_ptr(), t, heads, q.stride(0), q.stride(1), pool.data_ptr(), pool.shape[0], 656,
                          ptr.data_ptr(), idx.data_ptr(), idx.numel(), SCALE,
                          ops.FLAG_HAS_INVALID | ops.FLAG_RETURN_LSE | (chunk_tiles << ops.CHUNK_SHIFT),
                          out.data_ptr(), out.stride(0), out.stride(1),
                          lse.data_ptr(), None, 0, ops._stream(q.device))
    assert st == 0, L.mla_last_error().decode()
    return out, lse


@pytest.mark.parametrize("order", [(4, 16), (16, 4)])
def test_library_workspace_grows_and_matches_caller_workspace(order):
    say(f"library-owned workspace, heads {order}")
    L = mla.lib()
    assert L.mla_workspace_reserve(0, 1 << 20) == 0, L.mla_last_error().decode()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for k, heads in enumerate(order):
        q, pool, ptr, idx = problem(70 + k, 8, heads, 3000, 4000)
        assert mla.split_workgroups(8, idx.numel(), cus) > 0
        need = L.mla_sparse_fwd_workspace_size(8, heads, idx.numel(), 0, 0)
        assert need > (1 << 20)
        got_out, got_lse = fwd_library_workspace(q, pool, ptr, idx)
        want_out, want_lse = mla.sparse_fwd(q, pool, ptr, idx, SCALE, has_invalid=True, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(got_out.view(torch.int16), want_out.view(torch.int16)), f"out differs (H={heads})"
        assert torch.equal(got_lse.view(torch.int32), want_lse.view(torch.int32)), f"lse differs (H={heads})"


def test_graph_on_library_workspace_survives_growth():
    """Capture a NULL-workspace split call in a graph, then make a call that
    needs a far larger workspace (so the library replaces its buffer) and
    fill fresh device memory with 0xFF; replaying the graph must still give
    the eager result bit for bit, since the captured buffer stays allocated."""
    say("library-owned workspace: graph replay after growth")
    L = mla.lib()
    q, pool, ptr, idx = problem(90, 8, 8, 3000, 4000)
    flags = ops.FLAG_HAS_INVALID | ops.FLAG_RETURN_LSE | (8 << ops.CHUNK_SHIFT)
    need = L.mla_sparse_fwd_workspace_size(8, 8, idx.numel(), flags, 0)
    assert 0 < need != ctypes.c_size_t(-1).value
    assert L.mla_workspace_reserve(0, need) == 0, L.mla_last_error().decode()
    want_out, want_lse = fwd_library_workspace(q, pool, ptr, idx, chunk_tiles=8)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        got_out, got_lse = fwd_library_workspace(q, pool, ptr, idx, chunk_tiles=8)
    torch.cuda.synchronize()
    # 64 rows of 4000 entries in chunks of one tile: ~4064 partials of 16 heads
    # (about 133 MB), more than any other call in this process needs
    bq, bpool, bptr, bidx = problem(91, 64, 16, 3000, 4000)
    big = L.mla_sparse_fwd_workspace_size(64, 16, bidx.numel(), 1 << ops.CHUNK_SHIFT, 0)
    assert big > 50 * need
    fwd_library_workspace(bq, bpool, bptr, bidx, chunk_tiles=1)
    torch.cuda.synchronize()
    junk = torch.full((4 * need,), 255, dtype=torch.uint8, device=DEV)
    torch.cuda.synchronize()
    for _ in range(2):
        got_out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(got_out.view(torch.int16), want_out.view(torch.int16)), "replay out differs"
        assert torch.equal(got_lse.view(torch.int32), want_lse.view(torch.int32)), "replay lse differs"
    del junk
