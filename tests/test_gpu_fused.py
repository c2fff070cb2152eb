"""mla_sparse_fwd_v_up_proj: the forward followed by the gated W_UV
up-projection, fused into the split-KV merge when the call splits.

It must equal, bit for bit, mla_sparse_fwd followed by
mla_v_up_proj_prepared on the same arguments (out, lse and the projected
v_out), at every merge shape (2, 4 and 8 chunk lanes), with forced chunks
over ragged, empty and masked rows, with row counts that do not fill the
last row block, on the path that does not split, with padded output views,
and with and without the gate and the LSE; and v_out must match the oracle
end to end (the oracle forward, rounded to bf16, then its up-projection),
within the up-projection's bar plus the forward's carried through it.
"""

import numpy as np
import pytest
import torch

import head_latent_attention_sparse_amd as mla
from head_latent_attention_sparse_amd.workloads import bf16_bits
from oracle import encode_records
from oracle import sparse_fwd as oracle_sparse_fwd
from oracle.epilogue import f32_to_bf16_bits
from oracle.records import bf16_bits_to_f32
from oracle.value import v_up_proj as oracle_v_up_proj
from tests.helpers import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCALE = 192 ** -0.5


def problem(seed, t, heads, n, lo, hi, masked=0.0, empty_rows=()):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((t, heads, 576), generator=g).to(torch.bfloat16).to(DEV)
    kv = torch.randn((n, 512), generator=g).to(torch.bfloat16)
    pe = torch.randn((n, 64), generator=g).to(torch.bfloat16)
    pool = torch.from_numpy(encode_records(bf16_bits(kv), bf16_bits(pe))).to(DEV)
    lens = torch.randint(lo, hi + 1, (t,), generator=g)
    for r in empty_rows:
        lens[r] = 0
    ptr = torch.cat([torch.zeros(1, dtype=torch.int64), torch.cumsum(lens, 0)]).to(torch.int32)
    idx = torch.randint(0, n, (int(ptr[-1]),), generator=g, dtype=torch.int32)
    if masked:
        idx[torch.rand(idx.shape, generator=g) < masked] = -1
    w = (torch.randn((heads, 512, 128), generator=g) * 512 ** -0.5).to(torch.bfloat16).to(DEV)
    gate = torch.randn((t, heads * 128), generator=g).to(torch.bfloat16).to(DEV)
    return q, pool, ptr.to(DEV), idx.to(DEV), w, gate


def two_calls(q, pool, ptr, idx, wp, gate, return_lse, chunk_tiles=0):
    out, lse = mla.sparse_fwd(q, pool, ptr, idx, SCALE, has_invalid=True, return_lse=return_lse,
                              chunk_tiles=chunk_tiles)
    v = mla.v_up_proj(out, wp, gate=gate, prepared=True)
    return v, out, lse


def same(a, b, what):
    for x, y, name in zip(a, b, ("v_out", "out", "lse")):
        if x is None and y is None:
            continue
        assert torch.equal(x.contiguous().view(torch.int16 if x.dtype == torch.bfloat16 else torch.int32),
                           y.contiguous().view(torch.int16 if y.dtype == torch.bfloat16 else torch.int32)), \
            f"{what}: {name} differs"


CASES = [
    # (seed, T, H, records, len lo, len hi, chunk_tiles, gate, lse, what)
    (21, 64, 16, 8192, 1024, 8192, 0, True, True, "paged-decode shape, library plan (2 chunk lanes)"),
    (22, 20, 16, 8192, 4000, 9000, 0, True, False, "library plan at 4 chunk lanes"),
    (23, 8, 16, 8192, 20000, 30000, 0, False, True, "library plan at 8 chunk lanes"),
    (24, 7, 12, 3000, 0, 2500, 3, True, True, "forced 3-tile chunks, 7 rows (a partial row block), 12 heads"),
    (25, 33, 1, 3000, 0, 900, 1, False, False, "forced 1-tile chunks, one head"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[-1] for c in CASES])
def test_fused_equals_forward_then_projection(case):
    seed, t, heads, n, lo, hi, chunk_tiles, use_gate, return_lse, what = case
    say(f"fused forward + up-projection: {what}")
    q, pool, ptr, idx, w, gate = problem(seed, t, heads, n, lo, hi, masked=0.1, empty_rows=(0,) if t > 4 else ())
    wp = mla.prepare_w_uv(w)
    g = gate if use_gate else None
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert chunk_tiles or mla.split_workgroups(t, idx.numel(), cus) > 0, "the case must split"
    got = mla.sparse_fwd_v_up_proj(q, pool, ptr, idx, SCALE, wp, gate=g, has_invalid=True, return_lse=return_lse,
                                   chunk_tiles=chunk_tiles)
    want = two_calls(q, pool, ptr, idx, wp, g, return_lse, chunk_tiles)
    torch.cuda.synchronize()
    same(got, want, what)


def test_fused_without_split_and_with_padded_views():
    say("fused forward + up-projection: a call that does not split, padded out / v_out views")
    q, pool, ptr, idx, w, gate = problem(26, 600, 16, 2000, 0, 300, masked=0.1)
    wp = mla.prepare_w_uv(w)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert mla.split_workgroups(600, idx.numel(), cus) == 0
    out_buf = torch.full((600, 16, 520), 7.0, dtype=torch.bfloat16, device=DEV)
    v_buf = torch.full((600, 16, 136), 5.0, dtype=torch.bfloat16, device=DEV)
    got = mla.sparse_fwd_v_up_proj(q, pool, ptr, idx, SCALE, wp, gate=gate, has_invalid=True, return_lse=True,
                                   out=out_buf, v_out=v_buf)
    want = two_calls(q, pool, ptr, idx, wp, gate, True)
    torch.cuda.synchronize()
    same((got[0][:, :, :128], got[1][:, :, :512], got[2]), want, "no split")
    assert torch.all(out_buf[:, :, 512:] == 7.0) and torch.all(v_buf[:, :, 128:] == 5.0), "padding columns changed"
    # the same with a padded view on the split path
    q, pool, ptr, idx, w, gate = problem(27, 64, 16, 8192, 1024, 8192)
    wp = mla.prepare_w_uv(w)
    out_buf = torch.full((64, 16, 520), 7.0, dtype=torch.bfloat16, device=DEV)
    v_buf = torch.full((64, 16, 136), 5.0, dtype=torch.bfloat16, device=DEV)
    got = mla.sparse_fwd_v_up_proj(q, pool, ptr, idx, SCALE, wp, gate=gate, has_invalid=True, return_lse=True,
                                   out=out_buf, v_out=v_buf)
    want = two_calls(q, pool, ptr, idx, wp, gate, True)
    torch.cuda.synchronize()
    same((got[0][:, :, :128], got[1][:, :, :512], got[2]), want, "split, padded views")
    assert torch.all(out_buf[:, :, 512:] == 7.0) and torch.all(v_buf[:, :, 128:] == 5.0), "padding columns changed"


def test_fused_projection_against_the_oracle():
    """v_out against the oracle end to end: the oracle forward on the same
    query, records (the oracle writer's) and lists, its output rounded to
    bf16 (the forward's output dtype), then the oracle's gated up-projection.
    The bar is the up-projection's own (4e-3 |ref| + 1e-4) plus the
    forward's bar on out (1e-2 + 1e-2 |out|) carried through the linear map:
    sigmoid(gate) * sum_l |W[h, l, v]| * (1e-2 + 1e-2 |out_ref[t, h, l]|)."""
    say("fused forward + up-projection: v_out against the oracle, end to end")
    q, pool, ptr, idx, w, gate = problem(28, 64, 16, 8192, 1024, 8192, masked=0.1)
    wp = mla.prepare_w_uv(w)
    v, _, _ = mla.sparse_fwd_v_up_proj(q, pool, ptr, idx, SCALE, wp, gate=gate, has_invalid=True)
    torch.cuda.synchronize()
    # inputs (not outputs) back on the host for the oracle
    q_bits, w_bits, g_bits = bf16_bits(q.cpu()), bf16_bits(w.cpu()), bf16_bits(gate.cpu())
    out_ref, _ = oracle_sparse_fwd(q_bits, pool.cpu().numpy(), ptr.cpu().numpy(), idx.cpu().numpy(), SCALE)
    out_ref_bits = f32_to_bf16_bits(out_ref.astype(np.float32))
    v_ref = oracle_v_up_proj(out_ref_bits, w_bits, g_bits)
    w_abs = np.abs(bf16_bits_to_f32(w_bits).astype(np.float64))                    # [H, 512, 128]
    sig = 1.0 / (1.0 + np.exp(-bf16_bits_to_f32(g_bits).astype(np.float64)))      # [T, H * 128]
    carried = np.einsum("thl,hlv->thv", 1e-2 + 1e-2 * np.abs(out_ref), w_abs) * sig.reshape(v_ref.shape)
    bound = 4e-3 * np.abs(v_ref) + 1e-4 + carried
    err = np.abs(v.float().cpu().numpy() - v_ref)
    assert np.all(err <= bound), f"max err / bound {np.max(err / bound):.3f}"
    say(f"  max err {err.max():.3e}, max err / bound {np.max(err / bound):.3f}")


def test_fused_zero_tokens_and_rejections():
    q, pool, ptr, idx, w, gate = problem(29, 4, 16, 100, 10, 20)
    wp = mla.prepare_w_uv(w)
    empty_q = q[:0]
    v, out, lse = mla.sparse_fwd_v_up_proj(empty_q, pool, ptr[:1], idx[:0], SCALE, wp[:16], return_lse=True)
    assert v.shape == (0, 16, 128) and out.shape == (0, 16, 512)
    with pytest.raises(ValueError):
        mla.sparse_fwd_v_up_proj(q, pool, ptr, idx, SCALE, w[:8])  # weights for another head count
    with pytest.raises(ValueError):
        mla.sparse_fwd_v_up_proj(q, pool, ptr, idx, SCALE, wp, gate=gate[:, :100])


@pytest.mark.parametrize("return_lse", [True, False])
def test_single_chunk_rows_written_directly_equal_the_merge(return_lse):
    """With forced 2-tile chunks, rows of at most 128 entries have one chunk:
    the plain forward writes their out / lse from the partial pass (the merge
    skips them) while the fused call merges them; the two must agree bit for
    bit on every row, one-chunk rows (some empty, some all masked) mixed with
    rows of several chunks."""
    say(f"one-chunk rows written directly (return_lse={return_lse})")
    g = torch.Generator().manual_seed(31)
    t, heads, n = 40, 16, 3000
    q = torch.randn((t, heads, 576), generator=g).to(torch.bfloat16).to(DEV)
    kv = torch.randn((n, 512), generator=g).to(torch.bfloat16)
    pe = torch.randn((n, 64), generator=g).to(torch.bfloat16)
    pool = torch.from_numpy(encode_records(bf16_bits(kv), bf16_bits(pe))).to(DEV)
    lens = torch.tensor([[0, 1, 64, 100, 128][i % 5] if i % 2 == 0 else 129 + 97 * i for i in range(t)])
    ptr = torch.cat([torch.zeros(1, dtype=torch.int64), torch.cumsum(lens, 0)]).to(torch.int32)
    idx = torch.randint(0, n, (int(ptr[-1]),), generator=g, dtype=torch.int32)
    idx[torch.rand(idx.shape, generator=g) < 0.1] = -1
    idx[int(ptr[6]):int(ptr[7])] = -1  # a one-chunk row with every entry masked
    w = (torch.randn((heads, 512, 128), generator=g) * 512 ** -0.5).to(torch.bfloat16).to(DEV)
    wp = mla.prepare_w_uv(w)
    ptr, idx = ptr.to(DEV), idx.to(DEV)
    plain = mla.sparse_fwd(q, pool, ptr, idx, SCALE, has_invalid=True, return_lse=return_lse, chunk_tiles=2)
    _, out_f, lse_f = mla.sparse_fwd_v_up_proj(q, pool, ptr, idx, SCALE, wp, has_invalid=True,
                                               return_lse=return_lse, chunk_tiles=2)
    torch.cuda.synchronize()
    assert torch.equal(plain[0].view(torch.int16), out_f.view(torch.int16)), "out differs"
    if return_lse:
        assert torch.equal(plain[1].view(torch.int32), lse_f.view(torch.int32)), "lse differs"
        assert torch.isneginf(plain[1][0]).all() and torch.isneginf(plain[1][6]).all()
