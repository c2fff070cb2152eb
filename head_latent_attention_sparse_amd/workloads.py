"""Seeded synthetic inputs for the five sparse-MLA workloads and the decode epilogue.

This module only draws random numbers and lays them out (CSR lists, block
tables, slot mappings).  It holds none of the method's arithmetic, so the
HIP path and the CPU oracle can both take their inputs from it.

Every tensor is drawn on the CPU from ``torch.Generator().manual_seed(seed)``
in the order written below; float values are drawn as float32 and rounded to
bf16 (round to nearest even).  "N(0, s)" means standard deviation s.

The shapes follow the workloads the pages serve: DeepSeek-V3.2 / Kimi-K3
sparse prefill over the fp8_ds_mla cache with at most 16 heads per rank
(flydsl_sparse_mla page, module docstring), paged decode over a block table
(fused_mla_key_concat_kv_cache page; kimi_k3 nvidia mla page), 12 heads per
rank at TP8 (mono/attention/mla page, module docstring), a 576-wide absorbed
query [ql_nope | q_pe] and a 192^-0.5 softmax scale (qk_nope 128 + qk_rope 64;
kimi_k3 nvidia mla page, ``__init__``).
"""

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import torch

SEED_BASE = 20261202
QK_HEAD_DIM = 192  # qk_nope_head_dim 128 + qk_rope_head_dim 64
SOFTMAX_SCALE = QK_HEAD_DIM**-0.5
D_QK = 576
LATENT = 512
ROPE = 64


@dataclass
class InsertBatch:
    kv_c: torch.Tensor  # bf16 [n, 512]
    k_pe: torch.Tensor  # bf16 [n, 64]
    slots: torch.Tensor  # int64 [n], -1 = skip


@dataclass
class Workload:
    name: str
    num_records: int
    q: torch.Tensor  # bf16 [T, H, 576]
    indptr: torch.Tensor  # int32 [T + 1]
    indices: torch.Tensor  # int32 [nnz]
    softmax_scale: float
    has_invalid: bool
    return_lse: bool
    # Insert batches that build the pool from zero bytes, applied in order.
    setup_inserts: List[InsertBatch] = field(default_factory=list)
    # Insert batches that belong to the timed step (before the forward).
    step_inserts: List[InsertBatch] = field(default_factory=list)
    block_size: Optional[int] = None  # pool viewed as [nb, block_size, 656]

    @property
    def num_tokens(self) -> int:
        return self.q.shape[0]

    @property
    def num_heads(self) -> int:
        return self.q.shape[1]

    @property
    def nnz(self) -> int:
        return int(self.indices.numel())

    def nnz_valid(self) -> int:
        ok = (self.indices >= 0) & (self.indices < self.num_records)
        return int(ok.sum())


def _bf16(g: torch.Generator, shape, std: float = 1.0) -> torch.Tensor:
    x = torch.randn(shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(torch.bfloat16)


def _csr(rows: List[torch.Tensor]) -> Tuple[torch.Tensor, torch.Tensor]:
    lengths = torch.tensor([0] + [int(r.numel()) for r in rows], dtype=torch.int64)
    indptr = torch.cumsum(lengths, 0).to(torch.int32)
    if rows:
        indices = torch.cat([r.to(torch.int32) for r in rows])
    else:
        indices = torch.zeros(0, dtype=torch.int32)
    return indptr, indices


def _pool_fill(g: torch.Generator, n: int, latent_std: float = 1.0) -> InsertBatch:
    kv_c = _bf16(g, (n, LATENT), latent_std)
    k_pe = _bf16(g, (n, ROPE))
    return InsertBatch(kv_c, k_pe, torch.arange(n, dtype=torch.int64))


def tiny(tokens: int = 4, heads: int = 16, records: int = 2048, per_row: int = 128) -> Workload:
    """Tiny: 4 rows x 128 distinct random slots over a 2048-record cache."""
    g = torch.Generator().manual_seed(SEED_BASE + 1)
    fill = _pool_fill(g, records)
    q = _bf16(g, (tokens, heads, D_QK))
    rows = [torch.randperm(records, generator=g)[:per_row] for _ in range(tokens)]
    indptr, indices = _csr(rows)
    return Workload("tiny", records, q, indptr, indices, SOFTMAX_SCALE,
                    has_invalid=False, return_lse=True, setup_inserts=[fill])


def paged_decode(batch: int = 64, heads: int = 16, len_lo: int = 1024, len_hi: int = 8192,
                 block_size: int = 64) -> Workload:
    """Paged decode: one query row per request over a paged pool and a random block table.

    Context lengths are uniform on [len_lo, len_hi] (inclusive).  The pool holds
    exactly the blocks the requests need; a random permutation of the blocks is
    dealt to the requests in order, and position j of request b reads slot
    ``table[b][j // block_size] * block_size + j % block_size``.
    """
    g = torch.Generator().manual_seed(SEED_BASE + 2)
    lengths = torch.randint(len_lo, len_hi + 1, (batch,), generator=g)
    blocks_per = [(int(n) + block_size - 1) // block_size for n in lengths]
    num_blocks = sum(blocks_per)
    fill = _pool_fill(g, num_blocks * block_size)
    q = _bf16(g, (batch, heads, D_QK))
    perm = torch.randperm(num_blocks, generator=g)
    rows, start = [], 0
    for n, nb in zip(lengths.tolist(), blocks_per):
        table = perm[start : start + nb]
        start += nb
        pos = torch.arange(n, dtype=torch.int64)
        rows.append(table[pos // block_size] * block_size + pos % block_size)
    indptr, indices = _csr(rows)
    return Workload("paged_decode", num_blocks * block_size, q, indptr, indices, SOFTMAX_SCALE,
                    has_invalid=False, return_lse=True, setup_inserts=[fill],
                    block_size=block_size)


def sparse_prefill(tokens: int = 4096, heads: int = 16, records: int = 131072,
                   per_row: int = 2048, p_invalid: float = 0.10,
                   frac_empty: float = 0.01) -> Workload:
    """Sparse top-k prefill.

    Each row lists ``per_row`` distinct uniform slots; then round(frac_empty * T)
    random rows are set entirely to -1, and every other entry is set to -1
    independently with probability ``p_invalid``.
    """
    g = torch.Generator().manual_seed(SEED_BASE + 3)
    fill = _pool_fill(g, records)
    q = _bf16(g, (tokens, heads, D_QK))
    idx = torch.stack([torch.randperm(records, generator=g)[:per_row] for _ in range(tokens)])
    n_empty = int(round(frac_empty * tokens))
    empty_rows = torch.randperm(tokens, generator=g)[:n_empty]
    drop = torch.rand((tokens, per_row), generator=g) < p_invalid
    idx[drop] = -1
    idx[empty_rows] = -1
    indptr = torch.arange(0, tokens * per_row + 1, per_row, dtype=torch.int64).to(torch.int32)
    return Workload("sparse_prefill", records, q, indptr, idx.reshape(-1).to(torch.int32),
                    SOFTMAX_SCALE, has_invalid=True, return_lse=True, setup_inserts=[fill])


def long_context(tokens: int = 8, heads: int = 16, records: int = 131072,
                 latent_std: float = 2.0) -> Workload:
    """Long context: few rows, each a random permutation of the whole cache."""
    g = torch.Generator().manual_seed(SEED_BASE + 4)
    fill = _pool_fill(g, records, latent_std)
    q = _bf16(g, (tokens, heads, D_QK))
    rows = [torch.randperm(records, generator=g) for _ in range(tokens)]
    indptr, indices = _csr(rows)
    return Workload("long_context", records, q, indptr, indices, SOFTMAX_SCALE,
                    has_invalid=False, return_lse=True, setup_inserts=[fill])


def insert_attend(pool: int = 65536, new_tokens: int = 4096, p_skip: float = 0.05,
                  tokens: int = 1024, heads: int = 12, per_row: int = 1024) -> Workload:
    """Insert + attend: insert new tokens into a filled pool, then attend over it.

    The pool is first filled at every slot; the step inserts ``new_tokens``
    tokens at distinct random slots, each slot set to -1 (skipped) with
    probability ``p_skip``, then runs the forward with ``per_row`` distinct
    random slots per row.
    """
    g = torch.Generator().manual_seed(SEED_BASE + 5)
    fill = _pool_fill(g, pool)
    kv_c = _bf16(g, (new_tokens, LATENT))
    k_pe = _bf16(g, (new_tokens, ROPE))
    slots = torch.randperm(pool, generator=g)[:new_tokens].to(torch.int64)
    slots[torch.rand(new_tokens, generator=g) < p_skip] = -1
    q = _bf16(g, (tokens, heads, D_QK))
    rows = [torch.randperm(pool, generator=g)[:per_row] for _ in range(tokens)]
    indptr, indices = _csr(rows)
    return Workload("insert_attend", pool, q, indptr, indices, SOFTMAX_SCALE,
                    has_invalid=False, return_lse=True, setup_inserts=[fill],
                    step_inserts=[InsertBatch(kv_c, k_pe, slots)])


@dataclass
class DecodeEpilogueBatch:
    """Inputs of one decode epilogue call (query concat + RoPE + insert)."""
    ql_nope: torch.Tensor         # bf16 [B, H, 512]
    q_pe: torch.Tensor            # bf16 [B, H, 64]
    kv_c: torch.Tensor            # bf16 [B, 512]
    k_pe: torch.Tensor            # bf16 [B, 64]
    slots: torch.Tensor           # int64 [B], -1 = skip
    positions: torch.Tensor       # int64 [B]
    cos_sin_cache: torch.Tensor   # float32 [max_position, 64]
    num_records: int


@dataclass
class PrefillEpilogueBatch:
    """Inputs of one prefill epilogue call (RoPE on q, key concat, insert)."""
    q: torch.Tensor               # bf16 [Tp, H, nope + 64]
    k_nope: torch.Tensor          # bf16 [Tp, H, nope]
    kv_c: torch.Tensor            # bf16 [Tp, 512]
    k_pe: torch.Tensor            # bf16 [Tp, 64]
    slots: torch.Tensor           # int64 [Tp], -1 = skip
    positions: torch.Tensor       # int64 [Tp]
    cos_sin_cache: torch.Tensor   # float32 [max_position, 64]
    num_records: int


def prefill_epilogue(tokens: int = 4096, heads: int = 16, nope: int = 128, pool: int = 131072,
                     max_position: int = 65536, p_skip: float = 0.05, seed_offset: int = 10) -> PrefillEpilogueBatch:
    """A prefill epilogue call: Tp tokens with H heads of q [nope | rope] and
    k_nope, all N(0,1), their latent and rope N(0,1), at distinct random
    slots (each -1 with probability p_skip), at consecutive positions from a
    random start, with a standard rotary table."""
    g = torch.Generator().manual_seed(SEED_BASE + seed_offset)
    q = _bf16(g, (tokens, heads, nope + ROPE))
    k_nope = _bf16(g, (tokens, heads, nope))
    kv_c = _bf16(g, (tokens, LATENT))
    k_pe = _bf16(g, (tokens, ROPE))
    slots = torch.randperm(pool, generator=g)[:tokens].to(torch.int64)
    slots[torch.rand(tokens, generator=g) < p_skip] = -1
    start = int(torch.randint(0, max(max_position - tokens, 1), (1,), generator=g))
    positions = torch.arange(start, start + tokens, dtype=torch.int64)
    return PrefillEpilogueBatch(q, k_nope, kv_c, k_pe, slots, positions, rope_table(max_position), pool)


def rope_table(max_position: int, dim: int = ROPE, base: float = 10000.0) -> torch.Tensor:
    """A rotary table as a model builds one: row p holds cos(p * f_i) for the
    dim/2 frequencies f_i = base^(-2i/dim), then sin(p * f_i); computed in
    float64 and stored as float32.  (Input data: the epilogue only reads it.)"""
    inv_freq = base ** (-torch.arange(0, dim, 2, dtype=torch.float64) / dim)
    ang = torch.arange(max_position, dtype=torch.float64)[:, None] * inv_freq[None, :]
    return torch.cat([torch.cos(ang), torch.sin(ang)], dim=1).to(torch.float32)


def decode_epilogue(batch: int = 4096, heads: int = 16, pool: int = 131072, max_position: int = 65536,
                    p_skip: float = 0.05, seed_offset: int = 6) -> DecodeEpilogueBatch:
    """A decode epilogue call: B tokens with H heads of absorbed query
    (ql_nope N(0,1), q_pe N(0,1)), their latent N(0,1) and rope N(0,1), at
    distinct random slots of a pool (each -1 with probability p_skip), at
    random positions below max_position, with a standard rotary table."""
    g = torch.Generator().manual_seed(SEED_BASE + seed_offset)
    ql_nope = _bf16(g, (batch, heads, LATENT))
    q_pe = _bf16(g, (batch, heads, ROPE))
    kv_c = _bf16(g, (batch, LATENT))
    k_pe = _bf16(g, (batch, ROPE))
    slots = torch.randperm(pool, generator=g)[:batch].to(torch.int64)
    slots[torch.rand(batch, generator=g) < p_skip] = -1
    positions = torch.randint(0, max_position, (batch,), generator=g, dtype=torch.int64)
    return DecodeEpilogueBatch(ql_nope, q_pe, kv_c, k_pe, slots, positions, rope_table(max_position), pool)


@dataclass
class ContextGatherBatch:
    """Inputs of one context-chunk gather: a paged pool and its requests."""
    setup_inserts: List[InsertBatch]  # build the pool from zero bytes
    num_records: int
    block_size: int
    block_table: torch.Tensor   # int32 [B, W]; unused entries -1
    cu_seq_lens: torch.Tensor   # int32 [B + 1]
    seq_starts: torch.Tensor    # int32 [B]

    @property
    def num_tokens(self) -> int:
        return int(self.cu_seq_lens[-1])


def context_gather(batch: int = 64, len_lo: int = 1024, len_hi: int = 8192, block_size: int = 64,
                   start_frac: float = 0.0, seed_offset: int = 7) -> ContextGatherBatch:
    """A context chunk over a paged pool: context lengths uniform on
    [len_lo, len_hi], a random permutation of the pool's blocks dealt to the
    requests in order (as in the paged decode workload); the chunk of request
    b starts at a uniform position below start_frac * length and runs to the
    end of its context."""
    g = torch.Generator().manual_seed(SEED_BASE + seed_offset)
    lengths = torch.randint(len_lo, len_hi + 1, (batch,), generator=g)
    blocks_per = [(int(n) + block_size - 1) // block_size for n in lengths]
    num_blocks = sum(blocks_per)
    fill = _pool_fill(g, num_blocks * block_size)
    perm = torch.randperm(num_blocks, generator=g).to(torch.int32)
    width = max(blocks_per) if blocks_per else 0
    table = torch.full((batch, width), -1, dtype=torch.int32)
    start = 0
    for b, nb in enumerate(blocks_per):
        table[b, :nb] = perm[start:start + nb]
        start += nb
    hi = (lengths.to(torch.float64) * start_frac).to(torch.int64) + 1
    starts = (torch.rand(batch, generator=g, dtype=torch.float64) * hi).to(torch.int64).clamp(max=lengths - 1)
    counts = lengths - starts
    cu = torch.cat([torch.zeros(1, dtype=torch.int64), torch.cumsum(counts, 0)]).to(torch.int32)
    return ContextGatherBatch([fill], num_blocks * block_size, block_size, table, cu, starts.to(torch.int32))


@dataclass
class VUpProjBatch:
    latent: torch.Tensor  # bf16 [T, H, 512]
    w_uv: torch.Tensor    # bf16 [H, 512, 128]
    gate: torch.Tensor    # bf16 [T, H * 128]


def v_up_proj_inputs(tokens: int = 4096, heads: int = 16, seed_offset: int = 8) -> VUpProjBatch:
    """Latent attention output N(0,1), a random-init W_UV N(0, 512^-1/2)
    (so the projection has unit scale), and a gate N(0,1); all bf16."""
    g = torch.Generator().manual_seed(SEED_BASE + seed_offset)
    latent = _bf16(g, (tokens, heads, LATENT))
    w_uv = _bf16(g, (heads, LATENT, 128), std=LATENT**-0.5)
    gate = _bf16(g, (tokens, heads * 128))
    return VUpProjBatch(latent, w_uv, gate)


@dataclass
class ExtraSegment:
    """A second record pool with its own CSR list, and per-head sink logits."""
    insert: InsertBatch         # fills the second pool from zero bytes
    num_records: int
    indptr: torch.Tensor        # int32 [T + 1]
    indices: torch.Tensor       # int32 [T * per_row]
    sink: torch.Tensor          # float32 [H]


def extra_segment(tokens: int, heads: int, per_row: int = 256, records: int = 16384,
                  seed_offset: int = 9) -> ExtraSegment:
    """For the sink / second-segment variant of a workload: a second pool of
    `records` records (latent and rope N(0,1)), `per_row` distinct random
    slots of it per row, and sink logits N(0,1)."""
    g = torch.Generator().manual_seed(SEED_BASE + seed_offset)
    fill = _pool_fill(g, records)
    rows = [torch.randperm(records, generator=g)[:per_row] for _ in range(tokens)]
    indptr, indices = _csr(rows)
    sink = torch.randn((heads,), generator=g, dtype=torch.float32)
    return ExtraSegment(fill, records, indptr, indices, sink)


WORKLOADS = {
    1: tiny,
    2: paged_decode,
    3: sparse_prefill,
    4: long_context,
    5: insert_attend,
}


def bf16_bits(t: torch.Tensor):
    """A bf16 tensor's bit patterns as a numpy uint16 array (CPU copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")
