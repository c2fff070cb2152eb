"""mla_sparse_fwd_noalloc (the forward for callers that cannot allocate)
against mla_sparse_fwd with a caller workspace: two split calls in a row, the
second smaller, must each equal the existing entry point's out and lse bit
for bit (the same kernels, the split workspace in the library's fixed
scratch array instead); a call that does not split uses no scratch; a call
whose split workspace exceeds the scratch is refused before anything is
queued."""

import ctypes

import pytest
import torch

import head_latent_attention_sparse_amd as mla
from head_latent_attention_sparse_amd import ops
from head_latent_attention_sparse_amd.workloads import bf16_bits
from oracle import encode_records
from tests.helpers import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCALE = 192 ** -0.5
SCRATCH = 32 << 20


def problem(seed, t, heads, n, lo, hi):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((t, heads, 576), generator=g).to(torch.bfloat16).to(DEV)
    kv = torch.randn((n, 512), generator=g).to(torch.bfloat16)
    pe = torch.randn((n, 64), generator=g).to(torch.bfloat16)
    pool = torch.from_numpy(encode_records(bf16_bits(kv), bf16_bits(pe))).to(DEV)
    lens = torch.randint(lo, hi + 1, (t,), generator=g)
    ptr = torch.cat([torch.zeros(1, dtype=torch.int64), torch.cumsum(lens, 0)]).to(torch.int32)
    idx = torch.randint(-1, n, (int(ptr[-1]),), generator=g, dtype=torch.int32)
    return q, pool, ptr.to(DEV), idx.to(DEV)


def noalloc(q, pool, ptr, idx, chunk_tiles=0, out=None, lse=None):
    t, heads = q.shape[0], q.shape[1]
    out = torch.empty((t, heads, 512), dtype=torch.bfloat16, device=DEV) if out is None else out
    lse = torch.empty((t, heads), dtype=torch.float32, device=DEV) if lse is None else lse
    L = mla.lib()
    st = L.mla_sparse_fwd_noalloc(q.data_ptr(), t, heads, q.stride(0), q.stride(1), pool.data_ptr(), pool.shape[0],
                                  656, ptr.data_ptr(), idx.data_ptr(), idx.numel(), SCALE,
                                  ops.FLAG_HAS_INVALID | ops.FLAG_RETURN_LSE | (chunk_tiles << ops.CHUNK_SHIFT),
                                  out.data_ptr(), out.stride(0), out.stride(1), lse.data_ptr(),
                                  ops._stream(q.device))
    return st, out, lse


def same(a, b, what):
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)), f"{what}: out differs"
    assert torch.equal(a[1].view(torch.int32), b[1].view(torch.int32)), f"{what}: lse differs"


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    say("no-alloc forward: a split call, then a smaller one, against mla_sparse_fwd")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    L = mla.lib()
    cases = [problem(11, 64, 16, 8192, 1024, 8192), problem(12, 8, 8, 3000, 600, 4000)]
    for k, (q, pool, ptr, idx) in enumerate(cases):
        t, heads = q.shape[0], q.shape[1]
        assert mla.split_workgroups(t, idx.numel(), cus) > 0
        need = L.mla_sparse_fwd_workspace_size(t, heads, idx.numel(), 0, 0)
        assert 0 < need <= SCRATCH
        st, out, lse = noalloc(q, pool, ptr, idx)
        assert st == 0, L.mla_last_error().decode()
        want = mla.sparse_fwd(q, pool, ptr, idx, SCALE, has_invalid=True, return_lse=True)
        torch.cuda.synchronize()
        same((out, lse), want, f"call {k} (T={t}, H={heads})")


def test_noalloc_forced_chunks_and_one_workgroup_per_row():
    say("no-alloc forward: forced chunks, and a call that does not split")
    L = mla.lib()
    q, pool, ptr, idx = problem(13, 5, 12, 2000, 0, 2500)
    st, out, lse = noalloc(q, pool, ptr, idx, chunk_tiles=3)
    assert st == 0, L.mla_last_error().decode()
    want = mla.sparse_fwd(q, pool, ptr, idx, SCALE, has_invalid=True, return_lse=True, chunk_tiles=3)
    torch.cuda.synchronize()
    same((out, lse), want, "forced chunks")
    q, pool, ptr, idx = problem(14, 600, 16, 2000, 0, 300)  # 600 rows: one workgroup per row
    assert mla.lib().mla_sparse_fwd_workspace_size(600, 16, idx.numel(), 0, 0) == 0
    st, out, lse = noalloc(q, pool, ptr, idx)
    assert st == 0, L.mla_last_error().decode()
    want = mla.sparse_fwd(q, pool, ptr, idx, SCALE, has_invalid=True, return_lse=True)
    torch.cuda.synchronize()
    same((out, lse), want, "no split")


def test_noalloc_refuses_a_split_larger_than_the_scratch():
    say("no-alloc forward: a split workspace beyond the scratch is refused")
    L = mla.lib()
    q, pool, ptr, idx = problem(15, 64, 16, 3000, 4000, 4000)
    need = L.mla_sparse_fwd_workspace_size(64, 16, idx.numel(), 1 << ops.CHUNK_SHIFT, 0)
    assert need != ctypes.c_size_t(-1).value and need > SCRATCH
    out = torch.full((64, 16, 512), 3.0, dtype=torch.bfloat16, device=DEV)
    lse = torch.full((64, 16), 7.0, dtype=torch.float32, device=DEV)
    st, _, _ = noalloc(q, pool, ptr, idx, chunk_tiles=1, out=out, lse=lse)
    assert st == 2, f"status {st}: {L.mla_last_error().decode()}"  # MLA_ERR_UNSUPPORTED
    assert "scratch" in L.mla_last_error().decode()
    torch.cuda.synchronize()
    assert torch.all(out == 3.0) and torch.all(lse == 7.0)
    # the scratch is still usable afterwards
    q, pool, ptr, idx = problem(16, 8, 16, 3000, 2000, 3000)
    st, out, lse = noalloc(q, pool, ptr, idx)
    assert st == 0, L.mla_last_error().decode()
    want = mla.sparse_fwd(q, pool, ptr, idx, SCALE, has_invalid=True, return_lse=True)
    torch.cuda.synchronize()
    same((out, lse), want, "after a refused call")


def test_noalloc_under_graph_capture():
    """The callers the entry point is for: a split forward captured in a HIP
    graph with no workspace argument and no allocation, replayed three times
    with new queries and slot ids written into the captured buffers (other
    eager work and synchronizations between the replays).  Each replay must
    equal the workspace entry point, run eagerly on the same inputs, bit for
    bit."""
    say("no-alloc forward: captured in a graph, replayed three times")
    L = mla.lib()
    q, pool, ptr, idx = problem(17, 32, 16, 6000, 1500, 6000)
    t, heads = q.shape[0], q.shape[1]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert mla.split_workgroups(t, idx.numel(), cus) > 0
    out = torch.empty((t, heads, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((t, heads), dtype=torch.float32, device=DEV)
    st, _, _ = noalloc(q, pool, ptr, idx, out=out, lse=lse)  # first call on the device: eager
    assert st == 0, L.mla_last_error().decode()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st, _, _ = noalloc(q, pool, ptr, idx, out=out, lse=lse)
    assert st == 0, L.mla_last_error().decode()
    g = torch.Generator().manual_seed(18)
    for rep in range(3):
        q.copy_(torch.randn(q.shape, generator=g).to(torch.bfloat16))
        idx.copy_(torch.randint(-1, pool.shape[0], idx.shape, generator=g, dtype=torch.int32))
        noise = torch.randn((1 << 20,), device=DEV).abs().sum()  # unrelated eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        want = mla.sparse_fwd(q, pool, ptr, idx, SCALE, has_invalid=True, return_lse=True)
        torch.cuda.synchronize()
        assert torch.isfinite(noise)
        same((out, lse), want, f"replay {rep}")
