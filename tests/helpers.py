"""Shared test helpers: oracle-side pool building and the parity check.

The oracle side never consumes a value produced by the HIP path: its
records come from the oracle's own writer applied to the generated tokens.
"""

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch
from threadpoolctl import threadpool_limits

from oracle import encode_records, sparse_fwd as oracle_fwd
from head_latent_attention_sparse_amd.workloads import bf16_bits

# Parity bar for the forward: |out - ref| <= 1e-2 + 1e-2 |ref| elementwise,
# |lse - ref| <= 2e-3, and -inf (empty row) exactly where the oracle has it.
OUT_ATOL = 1e-2
OUT_RTOL = 1e-2
LSE_ATOL = 2e-3

CHUNK = 8192


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_encode(kv_c, k_pe):
    """Oracle records of bf16 token tensors, in chunks of CHUNK tokens."""
    kv_bits, pe_bits = bf16_bits(kv_c), bf16_bits(k_pe.reshape(k_pe.shape[0], -1))
    parts = [encode_records(kv_bits[i : i + CHUNK], pe_bits[i : i + CHUNK]) for i in range(0, kv_bits.shape[0], CHUNK)]
    return np.concatenate(parts) if parts else np.zeros((0, 656), np.uint8)


def oracle_threads():
    """Threads for oracle work: the CPUs this process may use, at most 16
    (a GPU machine's CPU share).  numpy releases the GIL in the oracle's array
    work, so threads share it without extra processes."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _parallel(fn, items):
    """fn over items on oracle_threads() threads (BLAS pinned to one thread
    each), results in item order."""
    with threadpool_limits(limits=1), ThreadPoolExecutor(oracle_threads()) as ex:
        return list(ex.map(fn, items))


def oracle_encode_parallel(kv_c, k_pe):
    """oracle_encode over CHUNK-token blocks on oracle_threads() threads."""
    kv_bits, pe_bits = bf16_bits(kv_c), bf16_bits(k_pe.reshape(k_pe.shape[0], -1))
    parts = _parallel(lambda i: encode_records(kv_bits[i : i + CHUNK], pe_bits[i : i + CHUNK]),
                      range(0, kv_bits.shape[0], CHUNK))
    return np.concatenate(parts) if parts else np.zeros((0, 656), np.uint8)


def oracle_pool(num_records, batches, fill=0):
    """The whole pool after applying insert batches in order (oracle writer)."""
    pool = np.full((num_records, 656), fill, dtype=np.uint8)
    for b in batches:
        slots = b.slots.numpy()
        keep = (slots >= 0) & (slots < num_records)
        if keep.any():
            rec = oracle_encode_parallel(b.kv_c[torch.from_numpy(keep)], b.k_pe[torch.from_numpy(keep)])
            pool[slots[keep]] = rec
    return pool


def oracle_fwd_rows(q_bits, pool, indptr, indices, softmax_scale, rows, block=16):
    """The oracle forward of the listed rows, in blocks of `block` rows run on
    oracle_threads() threads; returns (out [R, H, 512], lse [R, H]) in row order."""
    rows = list(rows)
    blocks = [rows[i : i + block] for i in range(0, len(rows), block)]
    parts = _parallel(lambda r: oracle_fwd(q_bits, pool, indptr, indices, softmax_scale, rows=r), blocks)
    if not parts:
        return np.zeros((0, q_bits.shape[1], 512)), np.zeros((0, q_bits.shape[1]))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def oracle_subpool(num_records, batches, slots_needed):
    """Records of only the listed slots (pool starts as zero bytes).

    Returns (sorted unique slots, their records).  Later batches win.
    """
    uniq = np.unique(np.asarray(slots_needed, dtype=np.int64))
    uniq = uniq[(uniq >= 0) & (uniq < num_records)]
    sub = np.zeros((uniq.size, 656), dtype=np.uint8)
    for b in batches:
        slots = b.slots.numpy()
        hit = np.isin(slots, uniq)
        if hit.any():
            rec = oracle_encode(b.kv_c[torch.from_numpy(hit)], b.k_pe[torch.from_numpy(hit)])
            sub[np.searchsorted(uniq, slots[hit])] = rec
    return uniq, sub


def remap_rows(indptr, indices, rows, uniq, num_records):
    """CSR of the listed rows with slot ids renumbered into the sub-pool."""
    indptr = np.asarray(indptr, dtype=np.int64)
    indices = np.asarray(indices, dtype=np.int64)
    new_ptr, new_ind = [0], []
    for t in rows:
        ids = indices[indptr[t] : indptr[t + 1]]
        ok = (ids >= 0) & (ids < num_records)
        mapped = np.full(ids.shape, -1, dtype=np.int64)
        mapped[ok] = np.searchsorted(uniq, ids[ok])
        new_ind.append(mapped)
        new_ptr.append(new_ptr[-1] + ids.size)
    ind = np.concatenate(new_ind) if new_ind else np.zeros(0, np.int64)
    return np.array(new_ptr, dtype=np.int64), ind


def assert_fwd_close(out, lse, ref_out, ref_lse, what=""):
    """GPU (out bf16, lse f32 or None) against oracle float64 results."""
    o = out.float().cpu().numpy().astype(np.float64)
    assert o.shape == ref_out.shape, (o.shape, ref_out.shape)
    assert np.all(np.isfinite(o)), f"{what}: non-finite out"
    err = np.abs(o - ref_out)
    bound = OUT_ATOL + OUT_RTOL * np.abs(ref_out)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} out elements off; worst at {i}: got {o[i]} want {ref_out[i]}")
    if lse is not None:
        l = lse.cpu().numpy().astype(np.float64)
        assert np.array_equal(np.isneginf(l), np.isneginf(ref_lse)), f"{what}: -inf pattern of lse differs"
        fin = np.isfinite(ref_lse)
        assert np.all(np.isfinite(l[fin])), f"{what}: non-finite lse"
        d = np.abs(l[fin] - ref_lse[fin])
        assert d.size == 0 or d.max() <= LSE_ATOL, f"{what}: lse off by {d.max()}"
