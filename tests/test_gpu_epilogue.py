"""GPU parity of the decode epilogue (mla_decode_q_concat_insert) and the
prefill epilogue (mla_prefill_key_concat_insert) against the oracle: mqa_q,
the rotated q, k_out and the pool bytes must be bit-exact (bf16 values and
record bytes are integer patterns, and both sides round the same float32
RoPE arithmetic to bf16 to nearest even).
"""

import numpy as np
import pytest
import torch

import head_latent_attention_sparse_amd as mla
from head_latent_attention_sparse_amd import workloads
from head_latent_attention_sparse_amd.workloads import bf16_bits
from oracle import decode_q_concat_insert as oracle_epilogue
from tests.helpers import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
FILL = 0x5A


def run_both(ql, qp, kv, kp, slots, n_rec, positions=None, table=None, mqa_q=None):
    """The GPU epilogue and the oracle on the same inputs; returns
    (device mqa bits, device pool, oracle mqa bits, oracle pool)."""
    pool = torch.full((n_rec, 656), FILL, dtype=torch.uint8, device=DEV)
    out = mla.decode_q_concat_insert(
        ql.to(DEV), qp.to(DEV), kv.to(DEV), kp.to(DEV), pool, slots.to(DEV),
        positions=positions.to(DEV) if positions is not None else None,
        cos_sin_cache=table.to(DEV) if table is not None else None,
        mqa_q=mqa_q)
    torch.cuda.synchronize()
    want_q, want_pool = oracle_epilogue(
        bf16_bits(ql), bf16_bits(qp), bf16_bits(kv), bf16_bits(kp.reshape(kp.shape[0], 64)), slots.numpy(),
        np.full((n_rec, 656), FILL, dtype=np.uint8),
        positions.numpy() if positions is not None else None,
        table.numpy() if table is not None else None)
    return bf16_bits(out), pool.cpu().numpy(), want_q, want_pool


def check(got_q, got_pool, want_q, want_pool):
    bad_q = np.argwhere(got_q != want_q)
    assert bad_q.size == 0, f"{len(bad_q)} mqa_q values differ, first (b, h, d) {bad_q[:3].tolist()}"
    bad = np.nonzero(np.any(got_pool != want_pool, axis=1))[0]
    assert bad.size == 0, f"{bad.size} records differ, first slots {bad[:5]}"


@pytest.mark.parametrize("b,h", [(1, 1), (5, 16), (64, 16), (300, 12), (33, 128), (7, 1024)])
@pytest.mark.parametrize("rope", [False, True])
def test_epilogue_bit_exact(b, h, rope):
    say(f"epilogue B={b} H={h} rope={rope}")
    w = workloads.decode_epilogue(batch=b, heads=h, pool=4 * b + 16, max_position=2048)
    check(*run_both(w.ql_nope, w.q_pe, w.kv_c, w.k_pe, w.slots, w.num_records,
                    w.positions if rope else None, w.cos_sin_cache if rope else None))


def test_epilogue_strided_views_and_out_of_range():
    say("epilogue strided views")
    g = torch.Generator().manual_seed(11)
    b, h = 40, 8
    # ql_nope as the transposed output of a per-head batched product [H, B, 512]
    ql = torch.randn((h, b, 512), generator=g).to(torch.bfloat16).transpose(0, 1)
    qp = torch.randn((b, h, 96), generator=g).to(torch.bfloat16)[:, :, 16:80]  # head stride 96
    kv = torch.randn((b, 640), generator=g).to(torch.bfloat16)[:, 64:576]
    kp = torch.randn((b, 1, 64), generator=g).to(torch.bfloat16)
    slots = torch.randperm(64, generator=g)[:b].to(torch.int64)
    slots[::5] = -1
    slots[1] = 64  # == num_records: skipped
    slots[2] = 1 << 40
    pos = torch.randint(-100, 3000, (b,), generator=g, dtype=torch.int64)  # clamped into [0, 2048)
    table = workloads.rope_table(2048)
    out = torch.full((b, h, 600), -7.0, dtype=torch.bfloat16, device=DEV)
    got_q, got_pool, want_q, want_pool = run_both(ql, qp, kv, kp, slots, 64, pos, table, mqa_q=out[:, :, :576])
    check(got_q, got_pool, want_q, want_pool)
    assert torch.all(out[:, :, 576:].cpu() == -7.0), "columns past 576 were written"


def test_epilogue_full_batch():
    """The measured shape: 4096 tokens, 16 heads, RoPE, a 131072-record pool."""
    say("epilogue B=4096 H=16 full")
    w = workloads.decode_epilogue()
    check(*run_both(w.ql_nope, w.q_pe, w.kv_c, w.k_pe, w.slots, w.num_records, w.positions, w.cos_sin_cache))


def test_epilogue_empty_and_rejections():
    say("epilogue empty / rejections")
    z = torch.zeros
    pool = torch.zeros((8, 656), dtype=torch.uint8, device=DEV)
    out = mla.decode_q_concat_insert(z((0, 4, 512), dtype=torch.bfloat16, device=DEV),
                                     z((0, 4, 64), dtype=torch.bfloat16, device=DEV),
                                     z((0, 512), dtype=torch.bfloat16, device=DEV),
                                     z((0, 64), dtype=torch.bfloat16, device=DEV), pool,
                                     z((0,), dtype=torch.int64, device=DEV))
    assert out.shape == (0, 4, 576)
    args = [z((2, 4, 512), dtype=torch.bfloat16, device=DEV), z((2, 4, 64), dtype=torch.bfloat16, device=DEV),
            z((2, 512), dtype=torch.bfloat16, device=DEV), z((2, 64), dtype=torch.bfloat16, device=DEV), pool,
            z((2,), dtype=torch.int64, device=DEV)]
    with pytest.raises(ValueError):
        mla.decode_q_concat_insert(*args, positions=z((2,), dtype=torch.int64, device=DEV))
    with pytest.raises(ValueError):
        mla.decode_q_concat_insert(*args, positions=z((2,), dtype=torch.int64, device=DEV),
                                   cos_sin_cache=z((4, 64), dtype=torch.float16, device=DEV))
    assert torch.all(pool == 0)


# ---- prefill epilogue (mla_prefill_key_concat_insert)

def run_prefill(w, rope, q_view=None, k_out=None):
    from oracle import key_concat_insert as oracle_prefill
    pool = torch.full((w.num_records, 656), FILL, dtype=torch.uint8, device=DEV)
    q = (q_view if q_view is not None else w.q.to(DEV).clone())
    ko = mla.key_concat_insert(q, w.k_nope.to(DEV), w.k_pe.to(DEV), w.kv_c.to(DEV), pool, w.slots.to(DEV),
                               positions=w.positions.to(DEV) if rope else None,
                               cos_sin_cache=w.cos_sin_cache.to(DEV) if rope else None, k_out=k_out)
    torch.cuda.synchronize()
    want_q, want_k, want_pool = oracle_prefill(
        bf16_bits(w.q), bf16_bits(w.k_nope), bf16_bits(w.kv_c), bf16_bits(w.k_pe), w.slots.numpy(),
        np.full((w.num_records, 656), FILL, dtype=np.uint8),
        w.positions.numpy() if rope else None, w.cos_sin_cache.numpy() if rope else None)
    return bf16_bits(q), bf16_bits(ko), pool.cpu().numpy(), want_q, want_k, want_pool


@pytest.mark.parametrize("tp,h,nope", [(1, 1, 128), (7, 16, 128), (300, 16, 128), (33, 4, 64), (20, 128, 128)])
@pytest.mark.parametrize("rope", [False, True])
def test_prefill_epilogue_bit_exact(tp, h, nope, rope):
    say(f"prefill epilogue Tp={tp} H={h} nope={nope} rope={rope}")
    w = workloads.prefill_epilogue(tokens=tp, heads=h, nope=nope, pool=4 * tp + 16, max_position=4096)
    got_q, got_k, got_pool, want_q, want_k, want_pool = run_prefill(w, rope)
    check(got_q, got_pool, want_q, want_pool)
    bad = np.argwhere(got_k != want_k)
    assert bad.size == 0, f"{len(bad)} k_out values differ, first {bad[:3].tolist()}"


def test_prefill_epilogue_strided_and_full():
    say("prefill epilogue strided views, Tp=4096 full")
    w = workloads.prefill_epilogue()
    tp, h = w.q.shape[0], w.q.shape[1]
    qbuf = torch.full((tp, h, 200), -9.0, dtype=torch.bfloat16, device=DEV)
    qbuf[:, :, :192] = w.q.to(DEV)
    kbuf = torch.full((tp, h, 200), -9.0, dtype=torch.bfloat16, device=DEV)
    got_q, got_k, got_pool, want_q, want_k, want_pool = run_prefill(w, True, q_view=qbuf[:, :, :192],
                                                                    k_out=kbuf[:, :, :192])
    check(got_q, got_pool, want_q, want_pool)
    assert np.array_equal(got_k, want_k), "k_out differs"
    assert torch.all(qbuf[:, :, 192:].cpu() == -9.0) and torch.all(kbuf[:, :, 192:].cpu() == -9.0)


def test_prefill_epilogue_rejects_k_out_of_another_token_count():
    """A caller's k_out with fewer (or more) tokens than the inputs is refused
    before any launch: the pool and the buffers stay untouched."""
    say("prefill epilogue: k_out with the wrong token count")
    w = workloads.prefill_epilogue(tokens=6, heads=2, nope=128, pool=64, max_position=64)
    pool = torch.full((w.num_records, 656), FILL, dtype=torch.uint8, device=DEV)
    for rows in (5, 7):
        k_out = torch.full((rows, 2, 192), -3.0, dtype=torch.bfloat16, device=DEV)
        with pytest.raises(ValueError, match="k_out"):
            mla.key_concat_insert(w.q.to(DEV), w.k_nope.to(DEV), w.k_pe.to(DEV), w.kv_c.to(DEV), pool,
                                  w.slots.to(DEV), k_out=k_out)
        torch.cuda.synchronize()
        assert torch.all(k_out == -3.0)
    assert torch.all(pool == FILL)
