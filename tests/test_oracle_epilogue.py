"""Pins for the oracle's decode epilogue (no GPU).

* bf16 rounding against torch's float32 -> bfloat16 cast (a library
  routine), ties included;
* GPT-J RoPE: hand-worked pairs (tests/golden/rope_worked.json), the
  special angles that reduce it to identity, negation and a quarter turn,
  and complex multiplication (x[2i] + i x[2i+1]) * (c + i s) in float64,
  which fixes the adjacent-pair layout and the signs; a NeoX-style (half
  split) rotation differs from it;
* the epilogue: the latent query columns copied bit for bit, the rope
  columns rotated per token position, records equal to the writer applied
  to the rotated k_pe, skipped and out-of-pool slots untouched, positions
  clamped into the table.
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import decode_q_concat_insert, encode_records, f32_to_bf16_bits, rope_gptj_bits
from head_latent_attention_sparse_amd.workloads import bf16_bits, rope_table


def bits_of(x):
    return bf16_bits(torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16))


def f32_of(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(200000).astype(np.float32) * np.float32(3.0)
    # exact midpoints between neighbouring bf16 values, both parities
    mids = (f32_of(rng.integers(0, 0x7F00, 5000, dtype=np.uint16)).view(np.uint32) | 0x8000).view(np.float32)
    big = np.array([3.3895314e38, -3.3895314e38, 1e-40, -0.0, 0.0], dtype=np.float32)
    for v in (x, mids, -mids, big):
        want = bf16_bits(torch.from_numpy(v).to(torch.bfloat16))
        np.testing.assert_array_equal(f32_to_bf16_bits(v), want)


def test_rope_worked_pairs(golden_dir):
    with open(os.path.join(golden_dir, "rope_worked.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        x = np.zeros(64, dtype=np.float32)
        x[10:12] = case["x"]  # pair 5
        cs = np.zeros(64, dtype=np.float32)
        cs[:32] = 1.0  # other pairs: identity
        cs[5], cs[32 + 5] = case["c"], case["s"]
        y = f32_of(rope_gptj_bits(bits_of(x), cs))
        assert y[10:12].tolist() == case["y"], case["why"]
        np.testing.assert_array_equal(np.delete(y, [10, 11]), np.delete(f32_of(bits_of(x)), [10, 11]))


@pytest.mark.parametrize("c,s,kind", [(1.0, 0.0, "identity"), (-1.0, 0.0, "negate"), (0.0, 1.0, "quarter")])
def test_rope_special_angles(c, s, kind):
    rng = np.random.default_rng(2)
    xb = bits_of(rng.standard_normal((50, 64)))
    cs = np.concatenate([np.full(32, c), np.full(32, s)]).astype(np.float32)
    y = f32_of(rope_gptj_bits(xb, cs))
    x = f32_of(xb)
    if kind == "identity":
        want = x
    elif kind == "negate":
        want = -x
    else:
        want = np.empty_like(x)
        want[:, 0::2], want[:, 1::2] = -x[:, 1::2], x[:, 0::2]
    np.testing.assert_array_equal(y, want)


def test_rope_is_complex_multiplication_of_adjacent_pairs():
    rng = np.random.default_rng(3)
    xb = bits_of(rng.standard_normal((400, 64)) * 2.0)
    table = rope_table(4096).numpy()
    pos = rng.integers(0, 4096, 400)
    got = f32_of(rope_gptj_bits(xb, table[pos])).astype(np.float64)
    x = f32_of(xb).astype(np.float64)
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * (table[pos, :32].astype(np.float64) + 1j * table[pos, 32:].astype(np.float64))
    ref = np.empty_like(x)
    ref[:, 0::2], ref[:, 1::2] = z.real, z.imag
    # float32 rounding of two products and a sum, then bf16: within one bf16
    # ulp of the exact value (plus a float32 cancellation term).
    ulp = np.maximum(np.abs(ref), 1e-30) * 2.0**-7
    err = np.abs(got - ref)
    assert np.all(err <= ulp + 4 * 2.0**-24 * (np.abs(x).max(axis=1, keepdims=True) + 1e-30)), err.max()
    assert np.mean(got == f32_of(f32_to_bf16_bits(ref.astype(np.float32)))) > 0.99
    # the half-split (NeoX) pairing is a different rotation
    neox = np.empty_like(x)
    h = (x[:, :32] + 1j * x[:, 32:]) * (table[pos, :32] + 1j * table[pos, 32:])
    neox[:, :32], neox[:, 32:] = h.real, h.imag
    assert np.mean(np.abs(got - neox) > 1e-2) > 0.5


def make_step(b=37, h=3, n=200, seed=4, rope=True):
    rng = np.random.default_rng(seed)
    ql = bits_of(rng.standard_normal((b, h, 512)))
    qp = bits_of(rng.standard_normal((b, h, 64)))
    kv = bits_of(rng.standard_normal((b, 512)))
    kp = bits_of(rng.standard_normal((b, 64)))
    slots = rng.permutation(n)[:b].astype(np.int64)
    slots[::7] = -1
    slots[3] = n + 5  # outside the pool: skipped
    table = rope_table(100).numpy() if rope else None
    pos = rng.integers(-20, 130, b).astype(np.int64) if rope else None  # some outside [0, 100)
    return ql, qp, kv, kp, slots, table, pos


@pytest.mark.parametrize("rope", [False, True])
def test_epilogue_concat_rope_and_insert(rope):
    ql, qp, kv, kp, slots, table, pos = make_step(rope=rope)
    pool0 = np.random.default_rng(5).integers(0, 256, (200, 656), dtype=np.uint8)
    mqa, pool = decode_q_concat_insert(ql, qp, kv, kp, slots, pool0.copy(), positions=pos, cos_sin_cache=table)
    np.testing.assert_array_equal(mqa[:, :, :512], ql)
    if rope:
        rows = table[np.clip(pos, 0, 99)]
        for t in range(ql.shape[0]):
            for hh in range(ql.shape[1]):
                np.testing.assert_array_equal(mqa[t, hh, 512:], rope_gptj_bits(qp[t, hh], rows[t]))
        kp_used = np.stack([rope_gptj_bits(kp[t], rows[t]) for t in range(kp.shape[0])])
    else:
        np.testing.assert_array_equal(mqa[:, :, 512:], qp)
        kp_used = kp
    keep = (slots >= 0) & (slots < 200)
    np.testing.assert_array_equal(pool[slots[keep]], encode_records(kv[keep], kp_used[keep]))
    untouched = np.setdiff1d(np.arange(200), slots[keep])
    np.testing.assert_array_equal(pool[untouched], pool0[untouched])


def test_epilogue_clamps_positions_into_the_table():
    ql, qp, kv, kp, slots, table, pos = make_step(b=4, h=1, rope=True)
    pos[:] = [-5, 0, 99, 1000]
    mqa, _ = decode_q_concat_insert(ql, qp, kv, kp, slots, np.zeros((200, 656), np.uint8), pos, table)
    same, _ = decode_q_concat_insert(ql, qp, kv, kp, slots, np.zeros((200, 656), np.uint8),
                                     np.array([0, 0, 99, 99]), table)
    np.testing.assert_array_equal(mqa, same)


@pytest.mark.parametrize("rope", [False, True])
def test_prefill_key_concat_insert(rope):
    from oracle import key_concat_insert
    rng = np.random.default_rng(9)
    tp, h, nope, n = 11, 3, 128, 50
    q = bits_of(rng.standard_normal((tp, h, nope + 64)))
    kn = bits_of(rng.standard_normal((tp, h, nope)))
    kv = bits_of(rng.standard_normal((tp, 512)))
    kp = bits_of(rng.standard_normal((tp, 64)))
    slots = rng.permutation(n)[:tp].astype(np.int64)
    slots[::4] = -1
    table = rope_table(64).numpy() if rope else None
    pos = rng.integers(0, 64, tp) if rope else None
    pool0 = np.random.default_rng(10).integers(0, 256, (n, 656), dtype=np.uint8)
    q_out, k_out, pool = key_concat_insert(q, kn, kv, kp, slots, pool0.copy(), pos, table)
    np.testing.assert_array_equal(k_out[:, :, :nope], kn)                 # the nope part verbatim
    kp_used = np.stack([rope_gptj_bits(kp[t], table[pos[t]]) for t in range(tp)]) if rope else kp
    for hh in range(h):
        np.testing.assert_array_equal(k_out[:, hh, nope:], kp_used)        # one rope key for every head
    np.testing.assert_array_equal(q_out[:, :, :nope], q[:, :, :nope])      # q's nope part untouched
    if rope:
        for t in range(tp):
            np.testing.assert_array_equal(q_out[t, :, nope:], rope_gptj_bits(q[t, :, nope:], table[pos[t]]))
    else:
        np.testing.assert_array_equal(q_out, q)
    keep = slots >= 0
    np.testing.assert_array_equal(pool[slots[keep]], encode_records(kv[keep], kp_used[keep]))
    untouched = np.setdiff1d(np.arange(n), slots[keep])
    np.testing.assert_array_equal(pool[untouched], pool0[untouched])
