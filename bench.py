"""Benchmark of the sparse MLA forward on MI355X (one GPU).

python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3]
                [--no-cpu-baseline] [--copy-calibration]
                [--epilogue | --prefill-epilogue | --gather | --vproj | --insert | --decode-step |
                 --with-sink-extra]

A step is one pass of the hot path over the workload: for the sparse top-k
prefill workload (the default) that is one mla_sparse_fwd call over all
4096 rows; for the insert + attend workload it is the insert of the new
tokens followed by the forward.  With --epilogue a step is instead one
decode epilogue call (mla_decode_q_concat_insert: 4096 tokens, 16 heads,
RoPE), and with --gather one context-chunk gather + upconvert
(mla_gather_upconvert: 64 requests of 1024..8192 tokens), and with --vproj
one W_UV up-projection with the sigmoid gate (mla_v_up_proj: 4096 rows x 16
heads); with --insert one cache insert of 131072 tokens.  With --decode-step
a step is one decode step of 64 requests over the paged decode workload
(decode epilogue, split-KV forward, gated up-projection), timed eagerly and
as replayed HIP graphs.  Inputs are synthetic, seeded, and resident in HBM
before timing starts.  Prints ONE JSON line.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
FWD_KERNEL_SOURCE = os.path.join(ROOT, "head_latent_attention_sparse_amd", "csrc", "sparse_fwd.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sparse_fwd_sparse_prefill_traffic.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "sparse_fwd_sparse_prefill_mfma.json")

WORKLOAD_NAMES = {
    1: "tiny: T=4 rows, H=16, 128 distinct slots/row over 2048 records",
    2: "paged decode: B=64 rows, H=16, context U[1024,8192], block 64",
    3: "sparse top-k prefill: T=4096 rows, H=16, 2048 slots/row over 131072 records, 10% -1, 1% empty rows",
    4: "long context: T=8 rows, H=16, 131072 slots/row (split-KV + LSE merge)",
    5: "insert + attend: insert 4096 tokens (5% skipped) into 65536 records, then T=1024, H=12, 1024 slots/row",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4, 5],
                    help="workload: 1 tiny, 2 paged decode, 3 sparse top-k prefill, 4 long context, "
                         "5 insert + attend")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="oracle worker processes for cpu_baseline (default: the usable cores, at most 16)")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="time only the --config workload (default: the other four are timed too)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (counter calibration under rocprofv3 --pmc)")
    ap.add_argument("--epilogue", action="store_true",
                    help="measure the decode epilogue (query concat + RoPE + insert) instead of the forward")
    ap.add_argument("--prefill-epilogue", action="store_true",
                    help="measure the prefill epilogue (q RoPE + key concat + insert) instead of the forward")
    ap.add_argument("--gather", action="store_true",
                    help="measure the context gather + upconvert to bf16 instead of the forward")
    ap.add_argument("--with-sink-extra", action="store_true",
                    help="forward variant: add per-head sink logits and a second segment of 256 entries per row "
                         "over a second 16384-record pool (mla_sparse_fwd_ex)")
    ap.add_argument("--insert", action="store_true",
                    help="measure the cache insert alone: 131072 tokens into random slots of a 131072-record pool")
    ap.add_argument("--decode-step", action="store_true",
                    help="measure one decode step on the paged decode workload (decode epilogue with RoPE and "
                         "insert, split-KV forward, gated up-projection), eager and as a replayed HIP graph")
    ap.add_argument("--vproj", action="store_true",
                    help="measure the W_UV up-projection with the sigmoid gate instead of the forward")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash():
    """Hash of the forward kernel's source with comments and blank space
    removed, so the stored counters stay valid across comment edits and
    lapse with any change to the code."""
    import re

    with open(FWD_KERNEL_SOURCE) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: this library has no multi-GPU path "
              "(rows would shard across GPUs with no exchange).", file=sys.stderr)
        sys.exit(2)
    modes = {"epilogue": "bench_epilogue", "prefill_epilogue": "bench_prefill_epilogue", "gather": "bench_gather",
             "vproj": "bench_vproj", "decode_step": "bench_decode_step", "insert": "bench_insert"}
    for flag, fn in modes.items():
        if getattr(args, flag):
            import torch

            dev = torch.device("cuda:0")
            torch.cuda.set_device(dev)
            globals()[fn](args, dev)
            return
    bench_forward(args)


def input_hash(w, seg=None):
    """SHA-256 of every input of a forward workload as the GPU receives it:
    query, CSR, the insert batches that build (and, for insert + attend,
    update) the pool, the softmax scale and flags, and the sink and second
    segment when given."""
    import numpy as np
    import torch

    h = hashlib.sha256()
    parts = [w.q, w.indptr, w.indices]
    for b in w.setup_inserts + w.step_inserts:
        parts += [b.kv_c, b.k_pe, b.slots]
    if seg is not None:
        parts += [seg.sink, seg.indptr, seg.indices, seg.insert.kv_c, seg.insert.k_pe, seg.insert.slots]
    for x in parts:
        h.update(x.contiguous().view(-1).view(torch.uint8).numpy().tobytes())
    h.update(np.float32(w.softmax_scale).tobytes())
    h.update(bytes([int(w.has_invalid), int(w.return_lse), w.num_heads, w.block_size or 0]))
    return h.hexdigest()


def measure_forward(w, args, dev, seg=None):
    """Resident inputs, W warmup steps, then K timed steps of the workload's
    hot path (the step's inserts, then mla_sparse_fwd), a HIP event pair per
    step on the launch stream.  Returns the timings and sizes."""
    import numpy as np
    import torch

    import head_latent_attention_sparse_amd as mla

    t_count, heads = w.num_tokens, w.num_heads
    nnz, nnz_valid = w.nnz, w.nnz_valid()
    pool = torch.zeros((w.num_records, 656), dtype=torch.uint8, device=dev)
    view = pool.view(-1, w.block_size, 656) if w.block_size else pool
    for b in w.setup_inserts:
        mla.cache_insert(b.kv_c.to(dev), b.k_pe.to(dev), b.slots.to(dev), view)
    step_inserts = [(b.kv_c.to(dev), b.k_pe.to(dev), b.slots.to(dev)) for b in w.step_inserts]
    ex = {}
    if seg is not None:
        pool2 = torch.zeros((seg.num_records, 656), dtype=torch.uint8, device=dev)
        mla.cache_insert(seg.insert.kv_c.to(dev), seg.insert.k_pe.to(dev), seg.insert.slots.to(dev), pool2)
        ex = dict(attn_sink=seg.sink.to(dev), extra_kv=pool2, extra_indptr=seg.indptr.to(dev),
                  extra_indices=seg.indices.to(dev))
        nnz += int(seg.indices.numel())
        nnz_valid += int(seg.indices.numel())
    q = w.q.to(dev)
    indptr, indices = w.indptr.to(dev), w.indices.to(dev)
    out = torch.empty((t_count, heads, 512), dtype=torch.bfloat16, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    split_wgs = mla.split_workgroups(t_count, nnz, cus)
    ws_bytes = mla.lib().mla_sparse_fwd_workspace_size(t_count, heads, nnz, 0, dev.index or 0)
    workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step():
        for kv_c, k_pe, slots in step_inserts:
            mla.cache_insert(kv_c, k_pe, slots, view)
        return mla.sparse_fwd(q, view, indptr, indices, w.softmax_scale, has_invalid=w.has_invalid,
                              out=out, return_lse=w.return_lse, workspace=workspace, **ex)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed region: K steps; a HIP event pair around each step on the stream
    # the kernels are launched on (torch's current stream)
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = np.array([a.elapsed_time(b) for a, b in ev])
    _, lse = step()
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all(), "non-finite output"

    total_bytes = (nnz_valid * 656.0 + q.numel() * 2 + indptr.numel() * indptr.element_size()
                   + indices.numel() * indices.element_size() + out.numel() * 2
                   + (t_count * heads * 4 if w.return_lse else 0))
    if ex:
        total_bytes += (ex["extra_indptr"].numel() * ex["extra_indptr"].element_size()
                        + ex["extra_indices"].numel() * ex["extra_indices"].element_size() + heads * 4)
    for kv_c, k_pe, slots in step_inserts:  # [kv_c | k_pe] and the slot read, a record written
        total_bytes += kv_c.numel() * 2 + k_pe.numel() * 2 + slots.numel() * 8 + int((slots >= 0).sum()) * 656
    return dict(nnz=nnz, nnz_valid=nnz_valid, heads=heads, tokens=t_count, split_wgs=split_wgs,
                ms_per_step=wall * 1e3 / args.steps, dev_ms_mean=float(step_ms.mean()),
                dev_ms_median=float(np.median(step_ms)), total_bytes=total_bytes)


def config_summary(k, w, r, seg=None):
    """Per-workload figures for the JSON line."""
    gathered = r["nnz_valid"] * 656.0
    gbps = gathered / (r["dev_ms_mean"] * 1e-3) / 1e9
    return {
        "workload": WORKLOAD_NAMES[k],
        "rows": r["tokens"],
        "heads": r["heads"],
        "csr_entries": r["nnz"],
        "valid_entries": r["nnz_valid"],
        "split_kv_workgroups": r["split_wgs"],
        "device_us_mean": r["dev_ms_mean"] * 1e3,
        "device_us_median": r["dev_ms_median"] * 1e3,
        "pairs_H_per_s": r["nnz"] * r["heads"] / (r["ms_per_step"] * 1e-3),
        "record_GBps": gbps,
        "hbm_frac": gbps / HBM_PEAK_GBPS,
        "mfma_tflops": r["nnz_valid"] * r["heads"] * 2.0 * (576 + 512) / (r["dev_ms_mean"] * 1e-3) / 1e12,
        "input_sha256": input_hash(w, seg),
    }


def bench_forward(args):
    """The forward workloads: the headline one (--config, default the sparse
    top-k prefill) gives metric / value / roofline; the other four are timed
    the same way and reported under "configs"; the fp64 oracle is timed on
    the headline workload's rows on the host's cores."""
    import torch

    from head_latent_attention_sparse_amd import workloads

    log(f"generating workload {args.config}")
    w = workloads.WORKLOADS[args.config]()
    seg = workloads.extra_segment(w.num_tokens, w.num_heads) if args.with_sink_extra else None
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle's records and worker processes are set up before anything touches the GPU
        cpu = CpuOracle(w, seg, args.cpu_workers)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("headline workload: inputs resident; warmup and timed steps")
    r = measure_forward(w, args, dev, seg)
    head = config_summary(args.config, w, r, seg)
    log(f"timed {args.steps} steps: {r['ms_per_step']:.3f} ms/step (device mean {r['dev_ms_mean']:.3f} ms, "
        f"median {r['dev_ms_median']:.3f} ms)")
    configs = {}
    if not args.no_other_configs and seg is None:
        for k in sorted(WORKLOAD_NAMES):
            if k == args.config:
                continue
            log(f"workload {k}")
            wk = workloads.WORKLOADS[k]()
            configs[str(k)] = config_summary(k, wk, measure_forward(wk, args, dev))
            del wk
            torch.cuda.empty_cache()

    gathered = r["nnz_valid"] * 656.0
    dev_ms = r["dev_ms_mean"]
    achieved_gbps = gathered / (dev_ms * 1e-3) / 1e9
    flops = r["nnz_valid"] * r["heads"] * 2.0 * (576 + 512)
    traffic = None
    if os.path.exists(TRAFFIC_FILE) and args.config == 3 and seg is None:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_source_sha256_16") == source_hash():
            traffic = tr.get("bytes_per_launch")
    mfma = None
    if os.path.exists(MFMA_FILE) and args.config == 3 and seg is None:
        with open(MFMA_FILE) as f:
            mf = json.load(f)
        if mf.get("kernel_source_sha256_16") == source_hash():
            mfma = mf.get("mfma_busy_frac")

    result = {
        "metric": "sparse MLA fwd: (row,key) pairs/s x H and achieved HBM GB/s on 656B records",
        "value": r["nnz"] * r["heads"] / (r["ms_per_step"] * 1e-3),
        "unit": "pairs*H/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "arithmetic": "bf16 MFMA dot products with float32 accumulation for QK^T and PV (E4M3 record codes "
                      "converted exactly to bf16, per-128 tile scales applied in float32), float32 softmax",
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD_NAMES[args.config] + (
                "; + per-head sink and a second segment of 256 slots/row over 16384 more records"
                if seg is not None else ""),
            "rows": r["tokens"],
            "heads": r["heads"],
            "records": w.num_records,
            "csr_entries": r["nnz"],
            "valid_entries": r["nnz_valid"],
            "split_kv_workgroups": r["split_wgs"],
            "input_sha256": head["input_sha256"],
            "parallelism": "single GPU",
        },
        "gathered_record_GBps": gathered / (r["ms_per_step"] * 1e-3) / 1e9,
        "total_algorithmic_bytes": r["total_bytes"],
        "total_algorithmic_GBps": r["total_bytes"] / (dev_ms * 1e-3) / 1e9,
        "valid_pairs_H_per_s": r["nnz_valid"] * r["heads"] / (r["ms_per_step"] * 1e-3),
        "device_ms_per_step": dev_ms,
        "device_ms_per_step_median": r["dev_ms_median"],
        "mfma_tflops": flops / (dev_ms * 1e-3) / 1e12,
        "mfma_frac_algorithmic": flops / (dev_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        "mfma_busy_frac": mfma,
        "roofline": {
            "bound": "hbm",
            "achieved": achieved_gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved_gbps / HBM_PEAK_GBPS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": gathered,
        },
        "configs": configs,
    }
    if cpu is not None:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu.run()
        cpu.close()
    print(json.dumps(result), flush=True)


def time_steps(step, args, stream):
    """W untimed steps, then K steps with a HIP event pair each on `stream`;
    returns (wall ms per step, mean device ms per step)."""
    import numpy as np
    import torch

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall * 1e3 / args.steps, float(np.mean([a.elapsed_time(b) for a, b in ev]))


def bench_epilogue(args, dev):
    """One decode epilogue call per step: mqa_q = [ql_nope | RoPE(q_pe)] and the
    insert of [kv_c | RoPE(k_pe)], 4096 tokens x 16 heads into 131072 records."""
    import numpy as np
    import torch

    import head_latent_attention_sparse_amd as mla
    from head_latent_attention_sparse_amd import workloads

    log("generating the decode epilogue inputs")
    w = workloads.decode_epilogue()
    b, h = w.ql_nope.shape[0], w.ql_nope.shape[1]
    ql, qp, kv, kp = w.ql_nope.to(dev), w.q_pe.to(dev), w.kv_c.to(dev), w.k_pe.to(dev)
    slots, pos, table = w.slots.to(dev), w.positions.to(dev), w.cos_sin_cache.to(dev)
    pool = torch.zeros((w.num_records, 656), dtype=torch.uint8, device=dev)
    mqa = torch.empty((b, h, 576), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def step():
        mla.decode_q_concat_insert(ql, qp, kv, kp, pool, slots, positions=pos, cos_sin_cache=table, mqa_q=mqa)

    ms, dev_ms = time_steps(step, args, torch.cuda.current_stream(dev))
    kept = int(((w.slots >= 0) & (w.slots < w.num_records)).sum())
    # algorithmic bytes: every input once (the token's cos/sin row included),
    # mqa_q once, one record per kept token
    read = b * (h * 576 * 2 + 512 * 2 + 64 * 2 + 8 + 8 + 64 * 4)
    written = b * h * 576 * 2 + kept * 656
    achieved = (read + written) / (dev_ms * 1e-3) / 1e9
    result = {
        "metric": "MLA decode epilogue (query concat + GPT-J RoPE + fp8_ds_mla insert): tokens/s",
        "value": b / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"decode epilogue: B={b} tokens, H={h}, RoPE from a 65536-position fp32 table, "
                               f"{w.num_records} records, 5% slots skipped", "parallelism": "single GPU"},
        "device_ms_per_step": dev_ms,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": None,
                     "algorithmic_bytes_per_launch": read + written},
    }
    log(f"timed {args.steps} steps: {ms:.4f} ms/step (device {dev_ms:.4f} ms)")
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits

        from oracle import decode_q_concat_insert
        from head_latent_attention_sparse_amd.workloads import bf16_bits

        bits = [bf16_bits(x) for x in (w.ql_nope, w.q_pe, w.kv_c, w.k_pe)]
        opool = np.zeros((w.num_records, 656), dtype=np.uint8)
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            decode_q_concat_insert(*bits, w.slots.numpy(), opool, w.positions.numpy(), w.cos_sin_cache.numpy())
            el = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": b / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                                  "sample": f"the whole call ({b} tokens), numpy oracle, one thread, {el:.2f} s"}
    print(json.dumps(result), flush=True)


def bench_prefill_epilogue(args, dev):
    """One prefill epilogue per step: RoPE on q's rope part in place, the full
    key [k_nope | RoPE(k_pe)] for 16 heads, and the insert, 4096 tokens."""
    import numpy as np
    import torch

    import head_latent_attention_sparse_amd as mla
    from head_latent_attention_sparse_amd import workloads

    log("generating the prefill epilogue inputs")
    w = workloads.prefill_epilogue()
    tp, h, nope = w.k_nope.shape
    q, kn, kv, kp = w.q.to(dev), w.k_nope.to(dev), w.kv_c.to(dev), w.k_pe.to(dev)
    slots, pos, table = w.slots.to(dev), w.positions.to(dev), w.cos_sin_cache.to(dev)
    pool = torch.zeros((w.num_records, 656), dtype=torch.uint8, device=dev)
    k_out = torch.empty((tp, h, nope + 64), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def step():  # q is rotated again each step: same traffic, values drift (not checked here)
        mla.key_concat_insert(q, kn, kp, kv, pool, slots, positions=pos, cos_sin_cache=table, k_out=k_out)

    ms, dev_ms = time_steps(step, args, torch.cuda.current_stream(dev))
    kept = int(((w.slots >= 0) & (w.slots < w.num_records)).sum())
    read = tp * (h * 64 * 2 + h * nope * 2 + 512 * 2 + 64 * 2 + 8 + 8 + 64 * 4)
    written = tp * (h * 64 * 2 + h * (nope + 64) * 2) + kept * 656
    achieved = (read + written) / (dev_ms * 1e-3) / 1e9
    result = {
        "metric": "MLA prefill epilogue (q RoPE + full-key concat + fp8_ds_mla insert): tokens/s",
        "value": tp / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"prefill epilogue: Tp={tp} tokens, H={h}, qk_nope {nope} + rope 64, RoPE, "
                               f"{w.num_records} records, 5% slots skipped", "parallelism": "single GPU"},
        "device_ms_per_step": dev_ms,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": None,
                     "algorithmic_bytes_per_launch": read + written},
    }
    log(f"timed {args.steps} steps: {ms:.4f} ms/step (device {dev_ms:.4f} ms)")
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits

        from oracle import key_concat_insert
        from head_latent_attention_sparse_amd.workloads import bf16_bits

        bits = [bf16_bits(x) for x in (w.q, w.k_nope, w.kv_c, w.k_pe)]
        opool = np.zeros((w.num_records, 656), dtype=np.uint8)
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            key_concat_insert(*bits, w.slots.numpy(), opool, w.positions.numpy(), w.cos_sin_cache.numpy())
            el = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": tp / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                                  "sample": f"the whole call ({tp} tokens), numpy oracle, one thread, {el:.2f} s"}
    print(json.dumps(result), flush=True)


def bench_gather(args, dev):
    """One mla_gather_upconvert per step: a context chunk of 64 requests
    (contexts of 1024..8192 tokens, blocks of 64) into a bf16 [toks, 576]
    workspace."""
    import numpy as np
    import torch

    import head_latent_attention_sparse_amd as mla
    from head_latent_attention_sparse_amd import workloads

    log("generating the context gather inputs")
    w = workloads.context_gather()
    pool = torch.zeros((w.num_records // w.block_size, w.block_size, 656), dtype=torch.uint8, device=dev)
    for b in w.setup_inserts:
        mla.cache_insert(b.kv_c.to(dev), b.k_pe.to(dev), b.slots.to(dev), pool)
    table, cu, starts = w.block_table.to(dev), w.cu_seq_lens.to(dev), w.seq_starts.to(dev)
    n = w.num_tokens
    dst = torch.empty((n, 576), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def step():
        mla.gather_upconvert(pool, table, cu, n, seq_starts=starts, dst=dst)

    ms, dev_ms = time_steps(step, args, torch.cuda.current_stream(dev))
    moved = n * (656 + 576 * 2)  # each row: one record read, one bf16 row written
    achieved = moved / (dev_ms * 1e-3) / 1e9
    result = {
        "metric": "context gather + upconvert (fp8_ds_mla records -> bf16 workspace): tokens/s",
        "value": n / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"context gather: 64 requests, contexts U[1024,8192], blocks of 64, {n} tokens",
                   "parallelism": "single GPU"},
        "device_ms_per_step": dev_ms,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": None, "algorithmic_bytes_per_launch": moved},
    }
    log(f"timed {args.steps} steps: {ms:.4f} ms/step (device {dev_ms:.4f} ms)")
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits

        from oracle import encode_records, gather_upconvert
        from head_latent_attention_sparse_amd.workloads import bf16_bits

        with threadpool_limits(limits=1):
            # the pool by the oracle's own writer (untimed setup)
            opool = np.zeros((w.num_records, 656), dtype=np.uint8)
            for b in w.setup_inserts:
                kv, pe, sl = bf16_bits(b.kv_c), bf16_bits(b.k_pe), b.slots.numpy()
                for i in range(0, sl.size, 8192):
                    opool[sl[i:i + 8192]] = encode_records(kv[i:i + 8192], pe[i:i + 8192])
            t0 = time.perf_counter()
            gather_upconvert(opool, w.block_size, w.block_table.numpy(), w.cu_seq_lens.numpy(),
                             w.seq_starts.numpy(), n)
            el = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": n / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                                  "sample": f"the whole chunk ({n} tokens), numpy oracle, one thread, {el:.2f} s"}
    print(json.dumps(result), flush=True)


def bench_vproj(args, dev):
    """One mla_v_up_proj per step: [4096, 16, 512] latent times W_UV [16, 512, 128],
    gated by sigmoid of a [4096, 2048] gate."""
    import torch

    import head_latent_attention_sparse_amd as mla
    from head_latent_attention_sparse_amd import workloads

    log("generating the up-projection inputs")
    w = workloads.v_up_proj_inputs()
    lat, wuv, gate = w.latent.to(dev), w.w_uv.to(dev), w.gate.to(dev)
    t, h = lat.shape[0], lat.shape[1]
    out = torch.empty((t, h, 128), dtype=torch.bfloat16, device=dev)
    prepared = mla.prepare_w_uv(wuv)  # once, as after loading the weights
    torch.cuda.synchronize()

    def step():
        mla.v_up_proj(lat, prepared, gate=gate, out=out, prepared=True)

    def step_plain():
        mla.v_up_proj(lat, wuv, gate=gate, out=out)

    _, plain_dev_ms = time_steps(step_plain, args, torch.cuda.current_stream(dev))
    ms, dev_ms = time_steps(step, args, torch.cuda.current_stream(dev))
    moved = lat.numel() * 2 + wuv.numel() * 2 + gate.numel() * 2 + out.numel() * 2
    flops = 2.0 * t * h * 512 * 128
    achieved = moved / (dev_ms * 1e-3) / 1e9
    result = {
        "metric": "W_UV up-projection + sigmoid gate: rows/s",
        "value": t / (ms * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"v up-projection: T={t} rows, H={h}, latent 512 -> v 128, gated",
                   "parallelism": "single GPU"},
        "device_ms_per_step": dev_ms,
        "weights": "prepared once with mla_v_up_proj_prepare_weights (outside the timed steps)",
        "plain_weights_device_ms_per_step": plain_dev_ms,
        "mfma_tflops": flops / (dev_ms * 1e-3) / 1e12,
        "mfma_frac": flops / (dev_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": None, "algorithmic_bytes_per_launch": moved},
    }
    log(f"timed {args.steps} steps: {ms:.4f} ms/step (device {dev_ms:.4f} ms; plain weights {plain_dev_ms:.4f} ms)")
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits

        from oracle import v_up_proj
        from head_latent_attention_sparse_amd.workloads import bf16_bits

        lb, wb, gb = bf16_bits(w.latent), bf16_bits(w.w_uv), bf16_bits(w.gate)
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            v_up_proj(lb, wb, gb)
            el = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": t / el, "unit": "rows/s", "cores": 1, "kind": "oracle",
                                  "sample": f"the whole call ({t} rows x {h} heads), numpy float64 oracle, "
                                            f"one thread, {el:.2f} s"}
    print(json.dumps(result), flush=True)


def bench_insert(args, dev):
    """One mla_cache_insert per step: 131072 tokens of [kv_c_normed | k_pe]
    (N(0,1) bf16) into distinct random slots of a 131072-record pool, 5% of
    the tokens skipped (slot -1)."""
    import numpy as np
    import torch

    import head_latent_attention_sparse_amd as mla

    log("generating the insert inputs")
    n, records = 131072, 131072
    g = torch.Generator().manual_seed(20261202 + 11)
    kv_c = torch.randn((n, 512), generator=g).to(torch.bfloat16)
    k_pe = torch.randn((n, 64), generator=g).to(torch.bfloat16)
    slots = torch.randperm(records, generator=g)[:n]
    slots[torch.rand(n, generator=g) < 0.05] = -1
    kv, pe, sl = kv_c.to(dev), k_pe.to(dev), slots.to(dev)
    pool = torch.zeros((records, 656), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step():
        mla.cache_insert(kv, pe, sl, pool)

    ms, dev_ms = time_steps(step, args, torch.cuda.current_stream(dev))
    written = int((slots >= 0).sum())
    moved = n * (512 * 2 + 64 * 2 + 8) + written * 656  # tokens and slots read, records written
    achieved = moved / (dev_ms * 1e-3) / 1e9
    result = {
        "metric": "fp8_ds_mla cache insert: tokens/s",
        "value": n / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"cache insert: {n} tokens into random slots of a {records}-record pool, 5% skipped",
                   "parallelism": "single GPU"},
        "device_ms_per_step": dev_ms,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": None, "algorithmic_bytes_per_launch": moved},
    }
    log(f"timed {args.steps} steps: {ms:.4f} ms/step (device {dev_ms:.4f} ms)")
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits

        from oracle import encode_records
        from head_latent_attention_sparse_amd.workloads import bf16_bits

        keep = slots.numpy() >= 0
        kb, pb = bf16_bits(kv_c)[keep], bf16_bits(k_pe)[keep]
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            recs = encode_records(kb, pb)
            el = time.perf_counter() - t0
        assert recs.shape == (int(keep.sum()), 656) and np.isfinite(el)
        result["cpu_baseline"] = {"value": n / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                                  "sample": f"the whole call ({int(keep.sum())} records written, {n} tokens), "
                                            f"numpy oracle writer, one thread, {el:.2f} s"}
    print(json.dumps(result), flush=True)


def bench_decode_step(args, dev):
    """One decode step of 64 requests, H = 16, over the paged decode
    workload's pool and CSR lists: mla_decode_q_concat_insert (mqa_q with
    RoPE, the new tokens' records), then the attention and the gated W_UV
    up-projection, either as mla_sparse_fwd (split-KV pass and merge) plus
    mla_v_up_proj_prepared, or as mla_sparse_fwd_v_up_proj (the projection
    fused into the merge).  Each is timed eagerly, as one captured HIP graph
    replayed per step, and as one graph of ten steps; `value` takes the
    fastest."""
    import torch

    import head_latent_attention_sparse_amd as mla
    from head_latent_attention_sparse_amd import workloads

    log("generating the decode step inputs")
    w = workloads.paged_decode()
    b, h = w.num_tokens, w.num_heads
    pool = torch.zeros((w.num_records, 656), dtype=torch.uint8, device=dev)
    view = pool.view(-1, w.block_size, 656)
    for ins in w.setup_inserts:
        mla.cache_insert(ins.kv_c.to(dev), ins.k_pe.to(dev), ins.slots.to(dev), view)
    e = workloads.decode_epilogue(batch=b, heads=h, pool=w.num_records, max_position=8192)
    ql, qp, kv, kp = e.ql_nope.to(dev), e.q_pe.to(dev), e.kv_c.to(dev), e.k_pe.to(dev)
    slots, pos, table = e.slots.to(dev), e.positions.to(dev), e.cos_sin_cache.to(dev)
    vp = workloads.v_up_proj_inputs(tokens=b, heads=h)
    w_uv, gate = mla.prepare_w_uv(vp.w_uv.to(dev)), vp.gate.to(dev)  # prepared once, as after loading
    indptr, indices = w.indptr.to(dev), w.indices.to(dev)
    mqa = torch.empty((b, h, 576), dtype=torch.bfloat16, device=dev)
    out = torch.empty((b, h, 512), dtype=torch.bfloat16, device=dev)
    vout = torch.empty((b, h, 128), dtype=torch.bfloat16, device=dev)
    ws_bytes = mla.lib().mla_sparse_fwd_workspace_size(b, h, w.nnz, 0, 0)
    workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step_separate():
        mla.decode_q_concat_insert(ql, qp, kv, kp, view, slots, positions=pos, cos_sin_cache=table, mqa_q=mqa)
        mla.sparse_fwd(mqa, view, indptr, indices, w.softmax_scale, out=out, return_lse=True, workspace=workspace)
        mla.v_up_proj(out, w_uv, gate=gate, out=vout, prepared=True)

    def step_fused():
        mla.decode_q_concat_insert(ql, qp, kv, kp, view, slots, positions=pos, cos_sin_cache=table, mqa_q=mqa)
        mla.sparse_fwd_v_up_proj(mqa, view, indptr, indices, w.softmax_scale, w_uv, gate=gate, out=out, v_out=vout,
                                 return_lse=True, workspace=workspace)

    stream = torch.cuda.current_stream(dev)
    timings = {}
    for name, step in (("separate", step_separate), ("fused", step_fused)):
        eager = time_steps(step, args, stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        one = time_steps(graph.replay, args, torch.cuda.current_stream(dev))
        # ten steps in one graph: per-replay costs spread over ten steps
        graph10 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph10):
            for _ in range(10):
                step()
        torch.cuda.synchronize()
        ten = time_steps(graph10.replay, args, torch.cuda.current_stream(dev))
        timings[name] = {"eager": eager, "graph": one, "graph10": (ten[0] / 10, ten[1] / 10)}
        assert torch.isfinite(vout.float()).all(), "non-finite output"

    written = int((e.slots >= 0).sum())
    moved = (w.nnz_valid() * 656.0                      # records gathered
             + b * h * (512 + 64) * 2 + b * (512 + 64) * 2 + written * 656  # epilogue reads, records written
             + b * h * 576 * 2 * 2                      # mqa_q written, then read by the forward
             + b * h * 512 * 2                          # the attention output written
             + w_uv.numel() * 2 + gate.numel() * 2 + vout.numel() * 2)
    best_name, best_mode = min(((n, m) for n in timings for m in timings[n]), key=lambda nm: timings[nm[0]][nm[1]][1])
    best_ms, best_dev = timings[best_name][best_mode]
    eager_ms, eager_dev = timings["fused"]["eager"]
    graph_ms, graph_dev = timings["fused"]["graph"]
    g10_ms, g10_dev = timings["fused"]["graph10"]
    achieved = moved / (best_dev * 1e-3) / 1e9
    result = {
        "metric": "MLA decode step (epilogue + split-KV sparse forward + W_UV up-projection): steps/s",
        "value": 1e3 / best_ms,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": best_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"decode step: B={b} requests, H={h}, contexts U[1024, 8192] over a paged pool "
                               f"of {w.num_records} records, RoPE, gated up-projection",
                   "parallelism": "single GPU"},
        "device_ms_per_step": best_dev,
        "best": f"{best_name}, {best_mode}",
        "eager_ms_per_step": eager_ms,
        "eager_device_ms_per_step": eager_dev,
        "graph_ms_per_step": graph_ms,
        "graph_device_ms_per_step": graph_dev,
        "graph10_ms_per_step": g10_ms,
        "graph10_device_ms_per_step": g10_dev,
        "device_ms_per_step_by_variant": {n: {m: timings[n][m][1] for m in timings[n]} for n in timings},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": None, "algorithmic_bytes_per_launch": moved},
    }
    for n in timings:
        log(f"{n}: device us/step eager {timings[n]['eager'][1] * 1e3:.1f}, graph of one step "
            f"{timings[n]['graph'][1] * 1e3:.1f}, graph of ten steps {timings[n]['graph10'][1] * 1e3:.1f}")
    print(json.dumps(result), flush=True)


# ---- the oracle on the host's cores.  The worker processes are forked
# from this process before it touches the GPU; they inherit the oracle's
# records and the workload (copy on write) and run numpy only.
_CPU = {}


def _cpu_worker_init():
    from threadpoolctl import threadpool_limits

    _CPU["limits"] = threadpool_limits(limits=1)  # one BLAS thread per process


def _cpu_worker_rows(rows):
    from oracle import sparse_fwd

    sparse_fwd(_CPU["q_bits"], _CPU["pool"], _CPU["indptr"], _CPU["indices"], _CPU["scale"], rows=rows,
               extra=_CPU["extra"], sink=_CPU["sink"])
    return len(rows)


class CpuOracle:
    """The fp64 numpy oracle forward over all rows of a workload, in blocks of
    rows on a pool of worker processes (one per core the process may use, at
    most 16, the host cores that one GPU of the machine is given)."""

    def __init__(self, w, seg=None, workers=0):
        import multiprocessing

        import numpy as np

        from oracle import encode_records
        from head_latent_attention_sparse_amd.workloads import bf16_bits

        log("cpu baseline: the oracle's own records (untimed)")
        pool = np.zeros((w.num_records, 656), dtype=np.uint8)
        for b in w.setup_inserts + w.step_inserts:
            slots = b.slots.numpy()
            keep = (slots >= 0) & (slots < w.num_records)
            kv, pe = bf16_bits(b.kv_c)[keep], bf16_bits(b.k_pe)[keep]
            recs = [encode_records(kv[i:i + 8192], pe[i:i + 8192]) for i in range(0, kv.shape[0], 8192)]
            pool[slots[keep]] = np.concatenate(recs)
        _CPU.update(q_bits=bf16_bits(w.q), pool=pool, indptr=w.indptr.numpy().astype(np.int64),
                    indices=w.indices.numpy().astype(np.int64), scale=w.softmax_scale, extra=None, sink=None)
        self.pairs = int(w.nnz)
        if seg is not None:
            pool2 = encode_records(bf16_bits(seg.insert.kv_c), bf16_bits(seg.insert.k_pe))  # slots 0..N2-1 in order
            _CPU.update(extra=(pool2, seg.indptr.numpy().astype(np.int64), seg.indices.numpy().astype(np.int64)),
                        sink=seg.sink.numpy())
            self.pairs += int(seg.indices.numel())
        self.rows, self.heads = w.num_tokens, w.num_heads
        self.workers = workers or max(1, min(16, len(os.sched_getaffinity(0))))
        self.procs = multiprocessing.get_context("fork").Pool(self.workers, initializer=_cpu_worker_init)

    def run(self):
        blocks = [list(range(i, min(i + 8, self.rows))) for i in range(0, self.rows, 8)]
        self.procs.map(_cpu_worker_rows, blocks[: self.workers])  # first touch of the pages in every worker
        t0 = time.perf_counter()
        done = sum(self.procs.map(_cpu_worker_rows, blocks, chunksize=1))
        elapsed = time.perf_counter() - t0
        assert done == self.rows
        return {
            "value": self.pairs * self.heads / elapsed,
            "unit": "pairs*H/s",
            "cores": self.workers,
            "kind": "oracle",
            "sample": f"all {self.rows} rows ({self.pairs} CSR entries) of the same workload, fp64 numpy oracle, "
                      f"{self.workers} worker processes with one BLAS thread each, {elapsed:.2f} s wall",
        }

    def close(self):
        self.procs.close()
        self.procs.join()


if __name__ == "__main__":
    main()
