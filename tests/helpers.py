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
    (the host cores that one GPU of the machine is given).  numpy releases the GIL in the oracle's array
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


# ---- The split plan's chunking rule, restated for tests (the kernel's
# split_plan computes it on the device).  Candidate sizes C are multiples of
# 64 between ceil(n / W) and ceil(n / (W - rows)), at least 512; the smallest
# whose chunk total fits W workgroups is kept; then chunk sizes alternate
# C + 128, C - 128 along the chunk order if that fits W too.  With two sizes a
# row's chunk count depends on the parity of its first chunk.
SKEW_ENTRIES = 128


def plan_row_counts(length, big, small):
    """Chunks of a row of `length` entries when its first chunk is even (big
    first) and when it is odd (small first)."""
    q, rem = divmod(int(length), big + small)
    k0 = 2 * q + (0 if rem == 0 else (1 if rem <= big else 2))
    k1 = 2 * q + (0 if rem == 0 else (1 if rem <= small else 2))
    return k0, k1


def plan_chunk_sizes(lens, bound):
    """(big, small): the chunk sizes the plan picks for these row lengths."""
    up64 = lambda x: (min(x, 1 << 29) + 63) // 64 * 64
    cdiv = lambda a, b: -(-a // b)
    n, rows = int(sum(lens)), int(sum(1 for x in lens if x > 0))
    lo = max(512, up64(cdiv(n, bound)))
    hi = min(max(lo, up64(cdiv(n, bound - rows if bound > rows else 1))), 1 << 29)
    step = max(64, up64((hi - lo) // 3))
    c = hi
    for k in range(3, -1, -1):
        ck = min(lo + step * k, hi)
        if sum(cdiv(int(x), ck) for x in lens) <= bound:
            c = ck
    big, small = c + SKEW_ENTRIES, c - SKEW_ENTRIES
    if bound % 2 == 0 and plan_first_chunks(lens, big, small)[-1] <= bound:
        return big, small
    return c, c


def plan_first_chunks(lens, big, small):
    """Each row's first chunk index and, last, the total: a prefix in row
    order, each row's count taken at the parity of its first chunk."""
    f = [0]
    for x in lens:
        k0, k1 = plan_row_counts(x, big, small)
        f.append(f[-1] + (k1 if f[-1] % 2 else k0))
    return f


def plan_chunk_of_workgroup(b, bound, big, small):
    """The chunk index workgroup b takes: even chunks go to the first half of
    the workgroups (longer chunks), odd ones to the second."""
    if big == small:
        return b
    half = bound // 2
    return 2 * b if b < half else 2 * (b - half) + 1


def plan_chunk_range(f_row, i, big, small):
    """[start, start + size) of chunk i of a row whose first chunk is f_row
    (before clipping to the row's length)."""
    even_before = (f_row + i + 1) // 2 - (f_row + 1) // 2
    start = even_before * big + (i - even_before) * small
    return start, (big if (f_row + i) % 2 == 0 else small)
