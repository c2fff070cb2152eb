"""Sparse absorbed-MLA attention forward over records, and the LSE merge.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The forward is the plain definition of softmax attention, in float64,
following the ``flydsl_sparse_mla_fp8ds_fwd`` docstring on the
flydsl_sparse_mla page: the keys of row ``t`` are the slots listed in
``kv_indices`` between ``kv_indptr[t]`` and ``kv_indptr[t + 1]``, minus the
negative ones; all heads of a row share those keys (the latent cache has a
single KV head); the optional LSE is taken in base e over the scaled logits
of the kept keys; and a row that keeps no key has a zero output with an LSE
of minus infinity.

Readings where the pages are silent:
* slot ids >= the number of records are masked like negative ones (the
  pages leave them undefined; the HIP kernel masks them too, so no caller
  error can make it read outside the pool);
* a slot listed twice in a row counts twice (the softmax is a plain sum
  over the list);
* the scale is used as the float32 the caller's float becomes at the
  C boundary;
* ``attn_sink`` and the ``extra_*`` segment (arguments of ``sparse_mla_fwd``
  that the page's ``..._supported`` docstring lists but does not define):
  the sink of head h is one more logit s_h, in the units of the scaled
  logits, with a zero value vector, so it adds exp(s_h) to the softmax
  denominator and to the LSE (an otherwise empty row gives out 0 and
  lse = s_h); the extra segment is a second record pool with its own CSR
  list whose keys join the row's softmax with the primary ones (masked by
  the same rules against its own pool).
"""

import numpy as np

from .records import bf16_bits_to_f32, decode_records


def sparse_fwd(q_bits, records, indptr, indices, softmax_scale, rows=None, extra=None, sink=None):
    """Reference forward.

    q_bits:  uint16 [T, H, 576] bf16 bit patterns of the absorbed query
             [ql_nope | q_pe].
    records: uint8 [N, 656].
    indptr:  int [T + 1] CSR offsets into ``indices``.
    indices: int [nnz] flat slot ids (negative = masked).
    rows:    optional iterable of row ids to compute (default: all).
    extra:   optional (records2 uint8 [N2, 656], indptr2 [T + 1], indices2):
             a second segment attended jointly with the first.
    sink:    optional float [H] per-head sink logits (natural-log units of
             the scaled logits), taken as the float32 values given.
    Returns (out float64 [R, H, 512], lse float64 [R, H]) for the R rows.
    """
    q = bf16_bits_to_f32(q_bits).astype(np.float64)  # exact
    segs = [(np.asarray(records, dtype=np.uint8), np.asarray(indptr, dtype=np.int64),
             np.asarray(indices, dtype=np.int64))]
    if extra is not None:
        segs.append((np.asarray(extra[0], dtype=np.uint8), np.asarray(extra[1], dtype=np.int64),
                     np.asarray(extra[2], dtype=np.int64)))
    sigma = np.float64(np.float32(softmax_scale))
    t_count, heads, _ = q.shape
    rows = range(t_count) if rows is None else list(rows)
    s_logit = None if sink is None else np.asarray(sink, dtype=np.float32).astype(np.float64)

    out = np.zeros((len(rows), heads, 512), dtype=np.float64)
    lse = np.full((len(rows), heads), -np.inf, dtype=np.float64)
    for r, t in enumerate(rows):
        ks, vs = [], []
        for recs, iptr, idx in segs:
            ids = idx[iptr[t] : iptr[t + 1]]
            ids = ids[(ids >= 0) & (ids < recs.shape[0])]
            if ids.size:
                k, v = decode_records(recs[ids])  # [n, 576], [n, 512]
                ks.append(k)
                vs.append(v)
        if ks:
            k, v = np.concatenate(ks), np.concatenate(vs)
            z = sigma * (k @ q[t].T)  # [n, H] logits
        else:
            k, v = np.zeros((0, 576)), np.zeros((0, 512))
            z = np.zeros((0, heads))
        if s_logit is not None:  # the sink: one more logit per head, value 0
            z = np.concatenate([z, s_logit[None, :]])
            v = np.concatenate([v, np.zeros((1, 512))])
        if z.shape[0] == 0:
            continue  # out 0, lse -inf
        m = z.max(axis=0)
        if np.all(np.isneginf(m)):
            continue
        dead = np.isneginf(m)  # a head with no key and a -inf sink: out 0, lse -inf
        m_safe = np.where(dead, 0.0, m)
        total = np.sum(np.exp(z - m_safe), axis=0)
        lse[r] = np.where(dead, -np.inf, m_safe + np.log(np.where(dead, 1.0, total)))
        p = np.where(dead, 0.0, np.exp(z - np.where(dead, 0.0, lse[r])))  # softmax weights, columns sum to 1
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
