"""Seeded random forward problems against the oracle, every row checked
with the forward's bar.  Each seed draws a whole problem: rows T in [1, 700],
heads H in [1, 16], a pool of up to 4096 records, row lengths from one of
four mixes (short, long, mixed with empty rows, equal rows back to back),
masked and out-of-pool entries, int32 or int64 indices, the library's plan
or forced chunks, with or without the LSE, padded strides for q and out,
and (for some seeds) a sink and a second segment.  The draws combine cases the targeted tests cover one
at a time; the seeds are fixed, so a failure names a reproducible problem.
"""

import numpy as np
import pytest
import torch

import head_latent_attention_sparse_amd as mla
from oracle import encode_records, sparse_fwd as oracle_fwd
from head_latent_attention_sparse_amd.workloads import bf16_bits
from tests.helpers import assert_fwd_close, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SEEDS = list(range(24))


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    g = torch.Generator().manual_seed(1000 + seed)
    mix = ["short", "long", "mixed", "equal"][seed % 4]
    t = int(rng.integers(1, 701)) if mix != "long" else int(rng.integers(1, 40))
    h = int(rng.integers(1, 17))
    n = int(rng.integers(1, 4097))
    if mix == "short":
        lens = rng.integers(0, 200, t)
    elif mix == "long":
        lens = rng.integers(500, 6000, t)
    elif mix == "mixed":
        lens = rng.choice([0, 1, 63, 64, 65, 130, 700, 1500], t)
    else:
        lens = np.full(t, int(rng.integers(1, 400)))
    ptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    nnz = int(ptr[-1])
    idx = rng.integers(0, n, nnz).astype(np.int64)
    r = rng.random(nnz)
    p_bad = float(rng.choice([0.0, 0.05, 0.3]))
    idx[r < p_bad / 2] = -1
    idx[(r >= p_bad / 2) & (r < p_bad)] = n + int(rng.integers(0, 100))  # outside the pool
    kv_c = torch.randn((n, 512), generator=g).to(torch.bfloat16)
    k_pe = torch.randn((n, 64), generator=g).to(torch.bfloat16)
    rec = encode_records(bf16_bits(kv_c), bf16_bits(k_pe))
    q = torch.randn((t, h, 576), generator=g).to(torch.bfloat16)
    p = dict(mix=mix, t=t, h=h, n=n, ptr=ptr, idx=idx, rec=rec, q=q,
             dtype=torch.int64 if rng.random() < 0.5 else torch.int32,
             chunk_tiles=int(rng.choice([0, 0, 1, 3, 8])) if t <= 512 else 0,
             scale=float(rng.choice([192 ** -0.5, 0.02, 0.2])),
             q_pad=int(rng.choice([0, 8, 64])), o_pad=int(rng.choice([0, 8, 100])))
    p["return_lse"] = bool(rng.random() < 0.7)  # drawn after the rest: earlier draws are unchanged
    if seed % 3 == 2:  # sink and second segment
        n2 = int(rng.integers(1, 1025))
        kv2 = torch.randn((n2, 512), generator=g).to(torch.bfloat16)
        pe2 = torch.randn((n2, 64), generator=g).to(torch.bfloat16)
        lens2 = rng.integers(0, 120, t)
        ptr2 = np.concatenate([[0], np.cumsum(lens2)]).astype(np.int64)
        idx2 = rng.integers(-2, n2 + 3, int(ptr2[-1])).astype(np.int64)
        p.update(rec2=encode_records(bf16_bits(kv2), bf16_bits(pe2)), ptr2=ptr2, idx2=idx2,
                 sink=(rng.standard_normal(h) * 2).astype(np.float32))
    return p


@pytest.mark.parametrize("seed", SEEDS)
def test_random_problem(seed):
    p = draw(seed)
    say(f"random seed {seed}: {p['mix']} T={p['t']} H={p['h']} N={p['n']} nnz={p['idx'].size} "
        f"{p['dtype']} chunk_tiles={p['chunk_tiles']} extra={'rec2' in p} lse={p['return_lse']}")
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    t, h = p["t"], p["h"]
    qbuf = torch.zeros((t, h, 576 + p["q_pad"]), dtype=torch.bfloat16, device=DEV)
    qbuf[:, :, :576] = p["q"].to(DEV)
    obuf = torch.full((t, h, 512 + p["o_pad"]), -3.0, dtype=torch.bfloat16, device=DEV)
    extra = {}
    if "rec2" in p:
        extra = dict(extra_kv=dev(p["rec2"]), extra_indptr=dev(p["ptr2"]).to(p["dtype"]),
                     extra_indices=dev(p["idx2"]).to(p["dtype"]), attn_sink=dev(p["sink"]))
    out, lse = mla.sparse_fwd(qbuf[:, :, :576], dev(p["rec"]), dev(p["ptr"]).to(p["dtype"]),
                              dev(p["idx"]).to(p["dtype"]), p["scale"], has_invalid=True,
                              out=obuf[:, :, :512], return_lse=p["return_lse"], chunk_tiles=p["chunk_tiles"],
                              **extra)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_fwd(bf16_bits(p["q"]), p["rec"], p["ptr"], p["idx"], p["scale"],
                                  extra=(p["rec2"], p["ptr2"], p["idx2"]) if "rec2" in p else None,
                                  sink=p.get("sink"))
    assert (lse is None) == (not p["return_lse"])
    assert_fwd_close(out, lse, ref_out, ref_lse, f"seed {seed}")
    if p["o_pad"]:
        assert torch.all(obuf[:, :, 512:].cpu() == -3.0), "columns past 512 were written"
