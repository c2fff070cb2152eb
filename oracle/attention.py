"""Sparse absorbed-MLA attention forward over records, and the LSE merge.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The forward is the plain definition of softmax attention, in float64, as the
flydsl_sparse_mla page describes ``flydsl_sparse_mla_fp8ds_fwd``: row ``t``
attends ``kv_indices[kv_indptr[t] : kv_indptr[t + 1]]``; negative entries
are masked; every head of the row uses the same keys (one shared latent KV
head); ``lse`` is the natural-log log-sum-exp of ``softmax_scale * q.k``
over the unmasked keys; a row with no unmasked key gives out = 0 and
lse = -inf.

Readings where the pages are silent (listed in the design doc):
* slot ids >= the number of records are masked like negative ones (the
  pages leave them undefined; the HIP kernel masks them too, so no caller
  error can make it read outside the pool);
* a slot listed twice in a row counts twice (the softmax is a plain sum
  over the list);
* the scale is used as the float32 the caller's float becomes at the
  C boundary.
"""

import numpy as np

from .records import bf16_bits_to_f32, decode_records


def sparse_fwd(q_bits, records, indptr, indices, softmax_scale, rows=None):
    """Reference forward.

    q_bits:  uint16 [T, H, 576] bf16 bit patterns of the absorbed query
             [ql_nope | q_pe].
    records: uint8 [N, 656].
    indptr:  int [T + 1] CSR offsets into ``indices``.
    indices: int [nnz] flat slot ids (negative = masked).
    rows:    optional iterable of row ids to compute (default: all).
    Returns (out float64 [R, H, 512], lse float64 [R, H]) for the R rows.
    """
    q = bf16_bits_to_f32(q_bits).astype(np.float64)  # exact
    records = np.asarray(records, dtype=np.uint8)
    indptr = np.asarray(indptr, dtype=np.int64)
    indices = np.asarray(indices, dtype=np.int64)
    n_records = records.shape[0]
    sigma = np.float64(np.float32(softmax_scale))
    t_count, heads, _ = q.shape
    rows = range(t_count) if rows is None else list(rows)

    out = np.zeros((len(rows), heads, 512), dtype=np.float64)
    lse = np.full((len(rows), heads), -np.inf, dtype=np.float64)
    for r, t in enumerate(rows):
        ids = indices[indptr[t] : indptr[t + 1]]
        ids = ids[(ids >= 0) & (ids < n_records)]
        if ids.size == 0:
            continue  # out 0, lse -inf
        k, v = decode_records(records[ids])  # [n, 576], [n, 512]
        z = sigma * (k @ q[t].T)  # [n, H] logits
        m = z.max(axis=0)
        lse[r] = m + np.log(np.sum(np.exp(z - m), axis=0))
        p = np.exp(z - lse[r])  # softmax weights, columns sum to 1
        out[r] = p.T @ v
    return out, lse


def merge_partials(outs, lses):
    """Combine attention partials over disjoint key sets by their LSEs.

    outs: sequence of float64 [..., 512]; lses: sequence of float64 [...].
    lse = ln sum_s exp(lse_s); out = sum_s exp(lse_s - lse) * out_s.  A
    partial with lse_s = -inf (no keys) has weight 0; if every partial is
    empty the result is out 0, lse -inf (the same convention as an empty
    row).  This is the combination named by ``merge_attn_states`` on the
    kimi_k3 nvidia mla page; the formula is the standard one, since the
    page does not print it.
    """
    lses = np.stack([np.asarray(x, dtype=np.float64) for x in lses])  # [S, ...]
    outs = np.stack([np.asarray(x, dtype=np.float64) for x in outs])  # [S, ..., 512]
    m = np.max(lses, axis=0)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(lses - m_safe)  # exp(-inf) = 0 for empty partials
    total = np.sum(w, axis=0)
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, total)))
    weights = np.where(empty, 0.0, w / np.where(empty, 1.0, total))
    out = np.sum(weights[..., None] * outs, axis=0)
    return out, lse
