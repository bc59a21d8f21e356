#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

One step is one whole decode-attention call over one batch: phase 1 (per
partition attention) and phase 2 (log-sum-exp merge) for the split workloads,
the single one-pass kernel for P = 0.  The default workload is the 100K-token
split decode (1 sequence x 100000 tokens, 24 query / 4 KV heads, head size
256, bf16 K/V, partition size 512 -> 196 partitions).

Inputs are generated on the host from a fixed seed, uploaded once, and stay
resident in HBM.  The KV pool is held in several copies and consecutive steps
read different copies, so every step streams its K/V from HBM rather than from
the 256 MB memory-side cache (at least 1.5 GiB of pool copies rotate).

Prints one JSON line (rank 0) with the step time, the KV-read bandwidth
(algorithmic bytes: every K and V element of every sequence read once), the
phase-1 kernel's roofline fraction against 8 TB/s, the oracle's CPU baseline on
the same workload, and the max abs error of the timed output against the oracle.
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode-attn µs/step + achieved KV-read HBM GB/s (% roofline) at 100K ctx"
PREFILL_METRIC = "prefix (chunked prefill) attention TFLOP/s over a paged KV cache"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, published


def kernel_source_hash() -> str:
    """Hash of the sources that determine the decode kernels' code (phase 1, the
    merge, their launchers and shared definitions, and the build script with
    their compiler flags)."""
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "decode_attention_paged_05_amd")
    csrc = os.path.join(pkg, "csrc")
    files = sorted(glob.glob(os.path.join(csrc, "pad_attn*")) +
                   [os.path.join(csrc, n) for n in ("pad_kernels.hip", "pad_internal.h", "pad_lane_ops.h")] +
                   [os.path.join(pkg, "build.py")])
    for f in files:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM bytes per phase-1 launch from the committed rocprofv3 counter runs,
    or None when absent or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def record_traffic(workload: str, fetch_csv: str, write_csv: str, copy_mib: int) -> int:
    """Write profiles/traffic_<workload>.json from two rocprofv3 --pmc runs of this
    script (FETCH_SIZE, then WRITE_SIZE, both with --copy-probe-mib): HBM bytes per
    phase-1 launch, each counter scaled by what it reads for the copy probe, a
    plain device copy of known size."""
    import csv

    def rows(path, counter):
        with open(path) as f:
            return [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]

    fetch, write = rows(fetch_csv, "FETCH_SIZE"), rows(write_csv, "WRITE_SIZE")
    copy_bytes = copy_mib * 2**20
    # the copy probe: the copy kernel whose WRITE_SIZE matches its size; the same dispatch in the fetch run
    probe = min((r for r in write if "copy" in r["Kernel_Name"].lower()),
                key=lambda r: abs(float(r["Counter_Value"]) * 1024 - copy_bytes))
    probe_fetch = next(r for r in fetch if r["Dispatch_Id"] == probe["Dispatch_Id"])
    assert probe_fetch["Kernel_Name"] == probe["Kernel_Name"], "the two runs dispatched different kernels"
    read_scale = copy_bytes / (float(probe_fetch["Counter_Value"]) * 1024)
    write_scale = copy_bytes / (float(probe["Counter_Value"]) * 1024)

    def phase1(rs):
        v = [float(r["Counter_Value"]) for r in rs if "attn_kernel" in r["Kernel_Name"]
             and ", true," in r["Kernel_Name"]]
        assert v, "no phase-1 dispatches in the counter file"
        return sum(v) / len(v), len(v)

    fk, nf = phase1(fetch)
    wk, nw = phase1(write)
    read_b, write_b = fk * 1024 * read_scale, wk * 1024 * write_scale
    out = {
        "workload": workload,
        "kernel_source_hash": kernel_source_hash(),
        "hbm_bytes_per_launch": round(read_b + write_b),
        "read_bytes_per_launch": round(read_b),
        "write_bytes_per_launch": round(write_b),
        "fetch_size_kib_per_dispatch": fk,
        "write_size_kib_per_dispatch": wk,
        "dispatches": [nf, nw],
        "calibration": {"copy_bytes": copy_bytes, "fetch_size_kib": float(probe_fetch["Counter_Value"]),
                        "write_size_kib": float(probe["Counter_Value"]), "read_scale": read_scale,
                        "write_scale": write_scale},
    }
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))
    return 0


def run_prefill(args) -> int:
    """One step = the chunk write into the cache plus the prefix attention of
    every chunk token, for one prefill workload (``--config prefill`` is one
    8192-token chunk over a 32768-token cached prefix, 24 query / 4 KV heads,
    head 256, bf16).  The roofline is the bf16 matrix-core peak against the
    algorithmic flops (4 H D per visible query-key pair)."""
    import numpy as np
    import torch

    import decode_attention_paged_05_amd as pad
    from decode_attention_paged_05_amd import inputs as gen

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    pp = gen.make_prefill_problem(args.config)
    spec, pool = pp.spec, pp.pool
    t0 = time.perf_counter()
    x = 16 // 2
    kc = torch.full((pool.num_blocks, spec.num_kv_heads, spec.head_size // x, 16, x), float("nan"),
                    dtype=torch.bfloat16, device=dev)
    vc = torch.full((pool.num_blocks, spec.num_kv_heads, spec.head_size, 16), float("nan"), dtype=torch.bfloat16,
                    device=dev)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    def sink(ids, kb, vb):
        idx = torch.from_numpy(ids.astype(np.int64)).to(dev)
        kt, vt = gen.to_tiled(kb, vb, "bf16")
        kc.index_copy_(0, idx, up(kt))
        vc.index_copy_(0, idx, up(vt))

    gen.fill_pool(pool, sink)
    key, value = pp.chunk_kv()
    q, kd, vd = up(pp.query), up(key), up(value)
    tables = torch.from_numpy(pool.block_tables).to(dev)
    qs = torch.from_numpy(pp.query_start).to(dev)
    ctx = torch.from_numpy(pp.context_lens).to(dev)
    out = torch.empty(tuple(pp.query.shape), dtype=torch.float32, device=dev)
    form = args.prefill_form
    if form == "auto":
        n_ranges = pad.paged_attention_prefill_split_ranges(spec.head_size, spec.num_heads, spec.num_kv_heads)
        form = "split" if pad.paged_attention_prefill_choose_split(
            pp.context_lens, pp.query_lens, spec.num_heads, spec.num_kv_heads, spec.head_size, n_ranges) else "grid"
    split = form == "split"
    ws = (pad.alloc_prefill_split_workspace(pp.num_seqs, spec.num_heads, spec.num_kv_heads, spec.head_size,
                                            pp.max_query_len, tables.shape[1], dev) if split else None)
    torch.cuda.synchronize()
    flops = pp.flops()
    desc = (f"{args.config}: {pp.num_seqs} seq, context {list(map(int, pp.context_lens))}, chunk "
            f"{list(map(int, pp.query_lens))} tokens, {spec.num_heads} q / {spec.num_kv_heads} KV heads, head "
            f"{spec.head_size}, bf16, block 16, tiled layout, "
            f"{'split launch' if split else 'one walk per workgroup'}")
    print(f"[bench] {desc}; inputs ready in {time.perf_counter() - t0:.1f}s", file=sys.stderr, flush=True)

    def step(ev=None):
        pad.paged_attention_prefill_write_kv(kc, vc, kd, vd, tables, qs, ctx, spec.num_kv_heads, 16,
                                             pp.max_query_len)
        if ev:
            ev[0].record()
        if split:
            pad.paged_attention_prefill_split(out, q, kc, vc, tables, qs, ctx, pp.scale, spec.num_kv_heads, 16,
                                              pp.max_query_len, ws)
        else:
            pad.paged_attention_prefill(out, q, kc, vc, tables, qs, ctx, pp.scale, spec.num_kv_heads, 16,
                                        pp.max_query_len)
        if ev:
            ev[1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    t_start = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t_start) * 1e3 / K
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    for i in range(K):
        step(evs[i])
    torch.cuda.synchronize()
    k_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    k_tflops = flops / (k_ms * 1e-3) / 1e12

    max_err, cpu = None, None
    if not (args.no_parity and args.no_cpu_baseline):
        import oracle

        got = out.double().cpu().numpy()
        H, G = spec.num_heads, spec.num_heads // spec.num_kv_heads
        s0, n0, c0, lo0 = 0, int(pp.query_lens[0]), int(pp.context_lens[0]), int(pp.query_start[0])
        K0 = [gen.sequence_kv(pool, s0, g) for g in range(spec.num_kv_heads)]
        rows = sorted({0, 1, 31, 32, n0 // 2, n0 - 33, n0 - 1} & set(range(n0)))
        heads = (0, G - 1, G, H - 1)
        t_or = time.perf_counter()
        done_flops, worst = 0, 0.0
        first = True
        while first or (not args.no_cpu_baseline and time.perf_counter() - t_or < args.cpu_seconds):
            for t in rows:
                for h in heads:
                    k_rows, v_rows = K0[h // G]
                    ref = oracle.prefill_rows(pp.query[lo0 + t:lo0 + t + 1, h], k_rows, v_rows, c0, t, pp.scale,
                                              "bf16")[0]
                    if first:
                        worst = max(worst, float(np.max(np.abs(got[lo0 + t, h] - ref))))
                    done_flops += 4 * spec.head_size * (c0 + t + 1)
            first = False
        total = time.perf_counter() - t_or
        max_err = worst
        if not args.no_cpu_baseline:
            cpu = {"value": round(done_flops / total / 1e12, 6), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
                   "host_cores": host_cores(), "cpu_model": cpu_model(),
                   "sample": f"{len(rows) * len(heads)} (token, head) output rows of sequence 0 computed one by one "
                             f"by the fp64 oracle, repeated for {total:.1f} s"}
    line = {
        "metric": PREFILL_METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": desc, "num_tokens": pp.num_tokens, "algorithmic_flops_per_step": flops,
                   "accumulate": "fp32", "products": "QK^T bf16 x bf16, P.V fp16 x fp16 (bf16 hi + lo pair where a "
                   "V value exceeds fp16's range)", "seed": spec.seed, "form": form},
        "kernels_ms": {"prefill": round(k_ms, 4)},
        "roofline": {
            "bound": "mfma",
            "achieved": round(k_tflops, 2),
            "peak": BF16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(k_tflops / BF16_MFMA_PEAK_TFLOPS, 4),
            "traffic": None,
            "kernel": "prefill",
            "algorithmic_flops_per_launch": flops,
        },
        "cpu_baseline": cpu,
        "max_abs_err_vs_oracle_sampled_rows": max_err,
    }
    print(json.dumps(line), flush=True)
    return 0


def host_cores() -> int:
    """Cores this process may run on (its CPU affinity set)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def describe(p, layout: str = "") -> str:
    lens = p.seq_lens
    L = f"{int(lens[0])} tokens" if (lens == lens[0]).all() else f"{int(lens.min())}-{int(lens.max())} tokens"
    P = p.partition_size
    return (f"{p.spec.name}: {p.num_seqs} seq x {L}, {p.num_heads} q / {p.num_kv_heads} KV heads, "
            f"head {p.head_size}, {p.dtype} KV, block {p.block_size}, "
            + (f"split P={P}" if P else "one-pass") + (f", {layout} layout" if layout else ""))


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="long",
                    help="decode: tiny | short | long | mixed | stress | batch256; prefill: prefill | prefill_batch")
    ap.add_argument("--partition-size", type=int, default=None, help="override the workload's partition size")
    ap.add_argument("--seq-len", type=int, default=None,
                    help="override every sequence's length (table width and pool follow)")
    ap.add_argument("--copies", type=int, default=0, help="KV pool copies to rotate (0: enough for 1.5 GB)")
    ap.add_argument("--prefill-form", default="auto", choices=["auto", "split", "grid"],
                    help="prefill workloads: the split launch (long walks cut into pieces, served first), one walk "
                         "per workgroup, or the library's choice for the workload's lengths")
    ap.add_argument("--layout", default="tiled", choices=["tiled", "rows"],
                    help="KV cache layout: tiled (K 16-byte chunks x tokens, V dims x tokens) or rows")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU work the oracle baseline repeats the step for (bounded sample)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before the steps, one plain device copy of this many MiB (read + write), "
                         "the reference kernel for calibrating HBM byte counters")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_<config>.json from two rocprofv3 --pmc counter files of this "
                         "script (FETCH_SIZE, WRITE_SIZE; both runs with --copy-probe-mib) and exit")
    args = ap.parse_args()
    if args.record_traffic:
        return record_traffic(args.config, *args.record_traffic, args.copy_probe_mib or 1024)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the decode path is sharded by sequence or KV head with no exchange, so N GPUs run N "
              "independent copies of this step", file=sys.stderr)
        return 2

    if args.config.startswith("prefill"):
        return run_prefill(args)

    import numpy as np
    import torch

    import decode_attention_paged_05_amd as pad
    from decode_attention_paged_05_amd import inputs as gen

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    overrides = {}
    if args.partition_size is not None:
        overrides["partition_size"] = args.partition_size
    if args.seq_len is not None:
        spec = gen.CONFIGS[args.config]
        W = -(-args.seq_len // spec.block_size)
        overrides.update(seq_len=args.seq_len, seq_len_range=None, max_blocks_per_seq=W,
                         num_blocks=max(spec.num_blocks, spec.num_seqs * W))
    p = gen.make_problem(args.config, **overrides)
    P = p.partition_size
    kv_bytes = p.kv_bytes()
    need_host = not (args.no_parity and args.no_cpu_baseline)

    # ---- inputs: generate on the host, upload once --------------------------------
    t0 = time.perf_counter()
    shape = (p.num_blocks, p.num_kv_heads, p.block_size, p.head_size)
    tdt = torch.float32 if p.dtype == "f32" else torch.bfloat16
    if args.layout == "tiled":
        x = 16 // (4 if p.dtype == "f32" else 2)
        k_shape = (p.num_blocks, p.num_kv_heads, p.head_size // x, p.block_size, x)
        v_shape = (p.num_blocks, p.num_kv_heads, p.head_size, p.block_size)
    else:
        k_shape = v_shape = shape
    kc = torch.full(k_shape, float("nan"), dtype=tdt, device=dev)
    vc = torch.full(v_shape, float("nan"), dtype=tdt, device=dev)
    host_k = host_v = None
    if need_host:
        host_k = np.full(shape, gen.poison_value(p.dtype), dtype=gen.storage_dtype(p.dtype))
        host_v = np.full(shape, gen.poison_value(p.dtype), dtype=gen.storage_dtype(p.dtype))

    def up(a):
        a = np.ascontiguousarray(a)
        if p.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    def sink(ids, kb, vb):
        idx = torch.from_numpy(ids.astype(np.int64)).to(dev)
        kd, vd = gen.to_tiled(kb, vb, p.dtype) if args.layout == "tiled" else (kb, vb)
        kc.index_copy_(0, idx, up(kd))
        vc.index_copy_(0, idx, up(vd))
        if need_host:
            host_k[ids] = kb
            host_v[ids] = vb

    gen.fill_pool(p, sink)
    q = up(p.query)
    tables = torch.from_numpy(p.block_tables).to(dev)
    lens = torch.from_numpy(p.seq_lens).to(dev)
    pool_bytes = 2 * kc.numel() * kc.element_size()
    copies = args.copies or max(1, min(8, -(-1536 * 2**20 // pool_bytes)))
    pools = [(kc, vc)] + [(kc.clone(), vc.clone()) for _ in range(copies - 1)]
    torch.cuda.synchronize()
    print(f"[bench] {describe(p, args.layout)}; inputs ready in {time.perf_counter() - t0:.1f}s; "
          f"{copies} pool copies of {pool_bytes / 2**20:.0f} MiB", file=sys.stderr, flush=True)

    out = torch.empty((p.num_seqs, p.num_heads, p.head_size), dtype=torch.float32, device=dev)
    ws = None
    dims = pad.make_dims(q, kc, tables)
    if P:
        ws = pad.alloc_workspace(p.num_seqs, p.num_heads, p.head_size, p.max_blocks_per_seq, p.block_size, P,
                                 device=dev)

    def step(i, ev=None):
        k, v = pools[i % copies]
        if P == 0:
            if ev:
                ev[0].record()
            pad.paged_attention_decode(out, q, k, v, tables, lens, p.scale, p.num_kv_heads, p.block_size, 0)
            if ev:
                ev[1].record()
            return
        if ev:
            ev[0].record()
        pad.paged_attention_decode_phase1(q, k, v, tables, lens, p.scale, p.num_kv_heads, p.block_size, P, ws)
        if ev:
            ev[1].record()
        pad.paged_attention_decode_phase2(out, lens, p.num_kv_heads, p.block_size, P, ws, dims)
        if ev:
            ev[2].record()

    if args.copy_probe_mib:
        n = args.copy_probe_mib * 2**20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copy probe: {n} bytes read, {n} bytes written by one copy kernel", file=sys.stderr,
              flush=True)
        del src, dst

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps, nothing else enqueued between them ----
    K = args.steps
    torch.cuda.synchronize()  # one GPU: the barrier is the synchronisation
    t_start = time.perf_counter()
    for i in range(K):
        step(i)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t_start) * 1e3 / K
    result_gpu = out.detach().cpu().numpy().astype(np.float64)

    # ---- the same K steps again with HIP events around every kernel, recorded on
    # the stream the kernels run on (torch's current stream), for per-kernel
    # durations; the event records themselves stretch this pass a little ----
    n_ev = 2 if P == 0 else 3
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(K)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(K):
        step(i, evs[i])
    torch.cuda.synchronize()
    ms_with_events = (time.perf_counter() - t_start) * 1e3 / K
    k1_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    k2_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs])) if n_ev == 3 else 0.0
    step_us = np.array([e[0].elapsed_time(e[-1]) for e in evs]) * 1e3
    pcts = [round(float(np.percentile(step_us, q)), 2) for q in (10, 50, 90)]

    gbs = kv_bytes / (ms_per_step * 1e-3) / 1e9
    k1_gbs = kv_bytes / (k1_ms * 1e-3) / 1e9
    traffic = load_traffic(args.config)

    # ---- warm figure: the same steps on one pool copy only (labelled warm; the
    # pool still exceeds the 256 MB memory-side cache when it is larger) ----
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(K):
        step(0)
    torch.cuda.synchronize()
    ms_warm = (time.perf_counter() - t_start) * 1e3 / K

    # ---- a measured HBM reference: one 1 GiB device-to-device copy (read plus
    # write bytes over its time), next to the published 8 TB/s ----
    n_copy = 1 << 30
    src = torch.empty(n_copy, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(3):
        dst.copy_(src)
    c1.record()
    c1.synchronize()
    copy_gbs = 3 * 2 * n_copy / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst

    # ---- oracle: parity of the timed output and the CPU baseline ---------------
    max_err = None
    cpu = None
    if need_host:
        import oracle

        try:
            from threadpoolctl import threadpool_info
            blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:  # noqa: BLE001 - reporting only
            blas_threads = 1
        def oracle_step():
            return oracle.decode_attention(p.query, host_k, host_v, p.block_tables, p.seq_lens, p.scale,
                                           p.num_kv_heads, p.block_size, p.dtype)

        t_or = time.perf_counter()
        ref = oracle_step()
        or_s = time.perf_counter() - t_or
        max_err = float(np.max(np.abs(result_gpu - ref)))
        print(f"[bench] oracle {or_s:.2f}s per step, max |gpu - oracle| = {max_err:.3e}", file=sys.stderr,
              flush=True)
        if not args.no_cpu_baseline:
            # a bounded sample: whole steps repeated until about --cpu-seconds of CPU work
            reps, total = 1, or_s
            while total < args.cpu_seconds and reps < 200:
                t_or = time.perf_counter()
                oracle_step()
                total += time.perf_counter() - t_or
                reps += 1
            cpu = {"value": round(reps * kv_bytes / total / 1e9, 4), "unit": "GB/s", "cores": int(blas_threads),
                   "kind": "oracle", "host_cores": host_cores(), "cpu_model": cpu_model(),
                   "sample": f"{reps} full steps of the same workload ({describe(p, args.layout)}) in {total:.1f} s, "
                             f"fp64 NumPy on a host with {host_cores()} usable cores: matrix products on "
                             f"{int(blas_threads)} BLAS threads, the rest on one thread; "
                             f"{total / reps * 1e6:.0f} us per step"}

    line = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "pct_hbm_roofline": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.dtype,
        "data": "synthetic",
        "config": {
            "workload": describe(p, args.layout),
            "num_seqs": p.num_seqs,
            "seq_len": int(p.seq_lens.max()),
            "num_heads": p.num_heads,
            "num_kv_heads": p.num_kv_heads,
            "head_size": p.head_size,
            "partition_size": P,
            "kv_bytes_per_step": kv_bytes,
            "seed": p.spec.seed,
            "pool_copies": copies,
            "accumulate": "fp32",
            "kv_layout": args.layout,
        },
        "kernels_ms": {"phase1" if P else "one_pass": round(k1_ms, 5), **({"phase2": round(k2_ms, 5)} if P else {})},
        "ms_per_step_with_kernel_events": round(ms_with_events, 5),
        "event_step_us_p10_p50_p90": pcts,
        "us_per_step_warm_one_pool_copy": round(ms_warm * 1e3, 2),
        "measured_copy_gbs_read_plus_write": round(copy_gbs, 1),
        "roofline": {
            "bound": "hbm",
            "achieved": round(k1_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(k1_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "phase1" if P else "one_pass",
            "step_frac": round(gbs / HBM_PEAK_GBS, 4),
            "algorithmic_bytes_per_launch": kv_bytes,
        },
        "cpu_baseline": cpu,
        "max_abs_err_vs_oracle": max_err,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
