#!/usr/bin/env python3
"""Decode-attention benchmark: paged GQA decode on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--kernel auto|dot|mfma]

One step = the whole path on device-resident inputs: partition plan (host),
decode kernel, partition reduce kernel (or, with --fused, the single launch
that merges the partials in place).  W untimed steps, then K steps timed
between two device synchronisations, first as eager launches with HIP events
around each kernel, then (the headline) with each step's launches replayed
from a captured HIP graph, as a serving loop runs its decode steps; the plan
still runs on the host every step.  Prints ONE JSON line:

  value            KV-read throughput, GB/s: algorithmic K+V bytes of one step
                   (4 * Hkv * D * sum L) / (timed wall time / K)
  ms_per_step      timed wall time / K (us_per_step_eager: the eager loop's)
  roofline         the decode kernel against HBM peak (8 TB/s): algorithmic
                   bytes per launch / mean launch duration (HIP events on the
                   launch stream, in the eager timed loop); `traffic` is the
                   HBM bytes per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE
                   (profiles/), null if the kernel sources changed since
  cpu_baseline     the float64 oracle on a bounded sample of the same workload,
                   on this host's cores
  ceiling          this box's read ceilings on the workload's KV pools
  configs          (default run) the other long-context decode workloads, each
                   with its own read ceiling and the fraction of it reached,
                   and the multi-token workloads, timed the same way

Default workload: 4 sequences x 131072 tokens, (16 q, 2 kv, 256) heads,
block 32, the planner choosing the partition size.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20          # MI355X Infinity Cache
DESCRIPTIONS = {
    "tiny_1x64": "1 seq x 64 tokens, (32q, 8kv, 128), block 16, unsplit",
    "batch8_2k": "8 seqs, L uniform in [1, 2048], (32q, 8kv, 128), block 16, P=512",
    "long32_16k": "32 seqs, L uniform in [4096, 16384], (24q, 4kv, 256), block 32, K x3",
    "mixed64_32k": "64 seqs, mixed L (25% L=1, 25% 1-3 token tails, rest up to 32768), "
                   "(16q, 2kv, 128), block 8, P=512",
    "long4_128k": "4 seqs x 131072 tokens, (16q, 2kv, 256), block 32, pool 2x, planner",
    "verify32_q4": "speculative-decode verification: 32 seqs, L uniform in [4096, 16384], "
                   "4 query tokens each, (32q, 8kv, 128), block 16, planner",
    "prefill4_chunk1k": "chunked prefill: 4 seqs, a 1024-token chunk on a context uniform in "
                        "[1024, 8192], (24q, 4kv, 256), block 32, planner",
}
VARLEN = ("verify32_q4", "prefill4_chunk1k")
_MFMA_SOURCES = ["paged_gqa_kv_decode_amd/csrc/decode_mfma.hip",
                 "paged_gqa_kv_decode_amd/csrc/decode_mfma_impl.h"]
KERNEL_SOURCES = {
    1: ["paged_gqa_kv_decode_amd/csrc/decode_dot.hip"],
    3: _MFMA_SOURCES, 4: _MFMA_SOURCES, 5: _MFMA_SOURCES, 6: _MFMA_SOURCES,
}
KERNEL_NAMES = {1: "dot", 3: "mfma_w1", 4: "mfma_w2", 5: "mfma_w4", 6: "mfma_w4p2"}


def sources_sha(kernel: int) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES.get(kernel, []) + ["paged_gqa_kv_decode_amd/csrc/vk_kernels.h",
                                                 "paged_gqa_kv_decode_amd/csrc/mfma_ops.h",
                                                 "paged_gqa_kv_decode_amd/csrc/merge_ops.h"]:
        p = os.path.join(ROOT, rel)
        if os.path.exists(p):
            h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, partition: int, kernel: int, fused: bool = False):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary,
    or None if absent or stale."""
    tag = "_fused" if fused else ""
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_P{partition}{tag}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_sources_sha256_16") != sources_sha(kernel):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _bench_lib():
    import ctypes
    path = os.path.join(ROOT, "paged_gqa_kv_decode_amd", "libvkbench.so")
    L = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.vkb_stream_read.argtypes = [vp, i64, vp, i32, vp]
    L.vkb_stream_read_nt.argtypes = [vp, i64, vp, i32, vp]
    L.vkb_page_read.argtypes = [vp, i64, vp, i64, i32, i64, vp, vp]
    L.vkb_page_read_nt.argtypes = [vp, i64, vp, i64, i32, i64, vp, vp]
    L.vkb_fill.argtypes = [vp, i64, ctypes.c_uint32, vp]
    return L


def ceilings(wl, dev, P, reps=10):
    """Read-bandwidth ceilings of this machine for the workload's KV pools: a
    streaming read of both pools (16-byte loads, 8192 workgroups of 256
    threads, 8 loads in flight per thread), with plain and with nontemporal
    loads; the exact page list of the decode (partition-major, P/bs pages per
    workgroup), in order and sorted, plain and nontemporal.  Each timed run
    follows a 512 MiB read, so nothing is served from the caches."""
    import numpy as np
    import torch
    L = _bench_lib()
    q, k, v, bt, sl = dev
    st = torch.cuda.current_stream()
    h = st.cuda_stream
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    blocks = 8192
    sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    bs, D, Hkv = wl.block_size, wl.head_dim, wl.num_kv_heads
    page_bytes = bs * D * 2
    pool_pages = wl.num_blocks * Hkv
    ppg = max(1, (P if P > 0 else 512) // bs)
    ids = []
    for s_ in range(wl.num_seqs):
        n = -(-int(wl.seq_lens[s_]) // bs)
        for g in range(Hkv):
            ids.append(wl.block_tables[s_, :n].astype(np.int64) * Hkv + g)
    ids = np.concatenate(ids).astype(np.int32)
    ids_dev = torch.from_numpy(ids).cuda()
    ids_sorted = torch.from_numpy(np.sort(ids)).cuda()
    groups = -(-len(ids) // ppg)
    psink = torch.empty(groups * 256, dtype=torch.int32, device="cuda")

    L.vkb_fill(flush.data_ptr(), flush.numel(), 0, h)
    fsink = torch.empty(4096 * 256, dtype=torch.int32, device="cuda")

    def timed(fn):
        ts = []
        for _ in range(reps):
            L.vkb_stream_read(flush.data_ptr(), flush.numel(), fsink.data_ptr(), 4096, h)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            fn()
            e1.record(st)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts))

    pool_bytes = k.numel() * k.element_size()

    def stream(fn):
        return timed(lambda: (fn(k.data_ptr(), pool_bytes, sink.data_ptr(), blocks, h),
                              fn(v.data_ptr(), pool_bytes, sink.data_ptr(), blocks, h)))

    t_plain, t_nt = stream(L.vkb_stream_read), stream(L.vkb_stream_read_nt)
    page_total = 2 * len(ids) * page_bytes

    def pages(fn, idt):
        return timed(lambda: (fn(k.data_ptr(), pool_pages, idt.data_ptr(), len(ids), ppg,
                                 page_bytes, psink.data_ptr(), h),
                              fn(v.data_ptr(), pool_pages, idt.data_ptr(), len(ids), ppg,
                                 page_bytes, psink.data_ptr(), h)))

    gbs = {"stream_read_plain_GBps": 2 * pool_bytes / t_plain / 1e9,
           "stream_read_nt_GBps": 2 * pool_bytes / t_nt / 1e9,
           "page_read_GBps": page_total / pages(L.vkb_page_read, ids_dev) / 1e9,
           "page_read_nt_GBps": page_total / pages(L.vkb_page_read_nt, ids_dev) / 1e9,
           "page_read_sorted_GBps": page_total / pages(L.vkb_page_read, ids_sorted) / 1e9}
    out = {k_: round(v_, 1) for k_, v_ in gbs.items()}
    out["stream_read_GBps"] = max(out["stream_read_plain_GBps"], out["stream_read_nt_GBps"])
    best = max(gbs, key=gbs.get)
    out["read_ceiling_GBps"], out["read_ceiling_kernel"] = out[best], best.replace("_GBps", "")
    out.update({"page_bytes": page_bytes, "pages_per_group": ppg, "stream_blocks": blocks,
                "flushed": "512 MiB read before each timed run"})
    return out


def cpu_model() -> str:
    """The host CPU's model name (first entry of /proc/cpuinfo), or ""."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def cpu_baseline(wl, min_seconds: float = 10.0, max_seconds: float = 30.0):
    """Time the float64 oracle, as it stands, on whole steps of the workload
    (every sequence and query head in one call, threaded over the (sequence,
    head) rows): one warm-up step, then at least 3 timed steps, more while
    the timed total stays under `min_seconds`; a step that alone takes longer
    than `max_seconds` is timed once.  Reported: the median step."""
    import numpy as np
    import oracle
    from paged_gqa_kv_decode_amd.workloads import kv_read_bytes
    nthreads = oracle.default_threads()
    dtype = wl.meta.get("dtype", "f16")

    def step():
        t = time.perf_counter()
        oracle.paged_attention_arrays(wl.q, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens,
                                      wl.scale, nthreads=nthreads, dtype=dtype)
        return time.perf_counter() - t

    first = step()
    ts = [first] if first > max_seconds else []
    while not ts or (len(ts) < 3 or sum(ts) < min_seconds) and sum(ts) + first <= max_seconds:
        ts.append(step())
    med = float(np.median(ts))
    kv = kv_read_bytes(wl.seq_lens, wl.num_kv_heads, wl.head_dim, 4 if dtype == "f32" else 2)
    return {"value": round(kv / med / 1e9, 4), "unit": "GB/s (KV-read)",
            "cores": nthreads, "kind": "oracle", "cpu_model": cpu_model(),
            "ms_per_step": round(med * 1e3, 1),
            "sample": f"whole steps ({wl.num_seqs} sequences, {int(wl.seq_lens.sum())} tokens, "
                      f"all {wl.num_q_heads} q heads): median of {len(ts)} after "
                      f"{'none' if first > max_seconds else 'one'} warm-up, "
                      f"{sum(ts) + (0 if first > max_seconds else first):.2f} s wall in all",
            "seconds": round(sum(ts), 3)}


MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 matrix peak


def cpu_baseline_varlen(wl, min_seconds: float, max_seconds: float, flops_unit: bool):
    """The float64 oracle on whole sequences of a multi-token workload, in
    order and cycling, until at least `min_seconds` (bounded by `max_seconds`)."""
    import numpy as np
    import oracle
    from paged_gqa_kv_decode_amd.workloads import kv_read_bytes, varlen_pairs
    nthreads = oracle.default_threads()
    cu, ql = wl.meta["cu_q"], wl.meta["q_lens"]
    done, total, runs, work = 0, 0.0, 0, 0.0
    per = None
    while total < min_seconds:
        s = runs % wl.num_seqs
        w = (4.0 * wl.head_dim * wl.num_q_heads * varlen_pairs(wl.seq_lens[s:s + 1], ql[s:s + 1])
             if flops_unit else kv_read_bytes(wl.seq_lens[s:s + 1], wl.num_kv_heads, wl.head_dim))
        if per is not None and total + per * w > max_seconds:
            break
        t = time.perf_counter()
        oracle.paged_varlen_arrays(wl.q[cu[s]:cu[s + 1]], wl.k_cache, wl.v_cache,
                                   wl.block_tables[s:s + 1], wl.seq_lens[s:s + 1],
                                   np.array([0, ql[s]], dtype=np.int32), wl.scale,
                                   nthreads=nthreads,
                                   dtype="bf16" if wl.q.dtype == np.uint16 else "f16")
        total += time.perf_counter() - t
        runs += 1
        done += int(ql[s])
        work += w
        per = total / work
    value = work / total / (1e12 if flops_unit else 1e9)
    return {"value": round(value, 6), "unit": "TFLOP/s" if flops_unit else "GB/s (KV-read)",
            "cores": nthreads, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{runs} single-sequence oracle calls cycling over the {wl.num_seqs} "
                      f"sequences ({done} query rows, all {wl.num_q_heads} q heads), "
                      f"{total:.2f} s wall",
            "seconds": round(total, 3)}


def bench_varlen(args, wl, gen_s, emit=True):
    """Several query tokens per sequence: plan (host) + the multi-token kernel
    (+ its reduce when split) per step, pools rotated as for the decode.
    Prints the JSON line (with the CPU baseline) when `emit`, and returns it."""
    import numpy as np
    import torch
    from paged_gqa_kv_decode_amd import binding as vb
    from paged_gqa_kv_decode_amd.workloads import kv_read_bytes, varlen_pairs
    P_req = args.partition if args.partition is not None else wl.partition_sizes[0]
    ql = wl.meta["q_lens"]

    def dev(x):       # bf16 workloads hold bit patterns as uint16
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()
    q, k, v = dev(wl.q), dev(wl.k_cache), dev(wl.v_cache)
    bt = torch.from_numpy(wl.block_tables).cuda()
    sl = torch.from_numpy(wl.seq_lens).cuda()
    cu = torch.from_numpy(wl.meta["cu_q"]).cuda()
    kv_bytes = kv_read_bytes(wl.seq_lens, wl.num_kv_heads, wl.head_dim)
    flops = 4.0 * wl.head_dim * wl.num_q_heads * varlen_pairs(wl.seq_lens, ql)
    ncopies = max(2, min(args.max_copies, -(-(4 * MALL_BYTES) // kv_bytes)))
    pools = [(k, v)] + [(k.clone(), v.clone()) for _ in range(ncopies - 1)]
    stream = torch.cuda.current_stream()
    vb.select_varlen_kernel({"auto": vb.KERNEL_AUTO, "columns": vb.KERNEL_VARLEN_COLUMNS,
                             "tiles": vb.KERNEL_VARLEN_TILES}[args.varlen_kernel])
    vb.select_work_order({"auto": vb.ORDER_AUTO, "grid": vb.ORDER_GRID,
                          "longest": vb.ORDER_LONGEST_FIRST}[args.order])
    step0 = vb.VarlenStep(q, k, v, bt, sl, cu, wl.seq_lens, ql, wl.scale, P_req)
    kname = {vb.KERNEL_VARLEN_COLUMNS: "varlen_columns",
             vb.KERNEL_VARLEN_TILES: "varlen_tiles"}[step0.plan.kernel]
    P, NP, mq = step0.plan.partition_size, step0.plan.max_num_partitions, step0.max_q_len
    counter = [0]

    def one_step(ev=None):
        kk, vv = pools[counter[0] % ncopies]
        counter[0] += 1
        plan = vb.plan_varlen(wl.seq_lens, ql, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                              wl.block_size, wl.max_blocks_per_seq, P_req)
        assert plan.partition_size == P and plan.max_num_partitions == NP
        if ev is not None:
            ev[0].record(stream)
        if P:
            vb.paged_gqa_varlen(q, kk, vv, bt, sl, cu, mq, wl.scale, P, NP, None,
                                step0.max_logits, step0.exp_sums, step0.tmp_out, stream)
            if ev is not None:
                ev[1].record(stream)
            vb.paged_gqa_varlen_reduce(step0.max_logits, step0.exp_sums, step0.tmp_out, sl, cu,
                                       mq, P, step0.out, stream)
        else:
            vb.paged_gqa_varlen(q, kk, vv, bt, sl, cu, mq, wl.scale, 0, 1, step0.out,
                                stream=stream)
            if ev is not None:
                ev[1].record(stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t = time.perf_counter()
    for i in range(args.steps):
        one_step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t
    order_ran = vb.last_plan().work_order   # of the last launch
    dec_ms = np.array([e[0].elapsed_time(e[1]) for e in events])
    red_ms = np.array([e[1].elapsed_time(e[2]) for e in events])
    ms = wall * 1e3 / args.steps
    dec_s = float(dec_ms.mean()) * 1e-3
    ridge = MFMA_F16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    compute_bound = flops / kv_bytes > ridge
    if compute_bound:
        value, unit = flops / (ms * 1e-3) / 1e12, "TFLOP/s"
        roof = {"bound": "mfma", "achieved": round(flops / dec_s / 1e12, 2),
                "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(flops / dec_s / 1e12 / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None}
    else:
        value, unit = kv_bytes / (ms * 1e-3) / 1e9, "GB/s"
        roof = {"bound": "hbm", "achieved": round(kv_bytes / dec_s / 1e9, 2),
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(kv_bytes / dec_s / 1e9 / HBM_PEAK_GBS, 4), "traffic": None}
    result = {
        "metric": "multi-token paged attention µs/step (" +
                  ("causal attention TFLOP/s" if compute_bound else "KV-read HBM GB/s") + ")",
        "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "us_per_step": round(ms * 1e3, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": args.dtype,
        "data": f"synthetic (seeded N(0, 1) {args.dtype} K/V/q, shuffled pages)",
        "config": {"workload": wl.name, "description": DESCRIPTIONS[wl.name],
                   "num_seqs": wl.num_seqs, "num_q_heads": wl.num_q_heads,
                   "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
                   "block_size": wl.block_size, "sum_seq_len": int(wl.seq_lens.sum()),
                   "total_q": int(ql.sum()), "max_q_len": mq, "partition_size": P,
                   "max_num_partitions": NP, "decode_kernel": kname,
                   "work_order": {1: "grid", 2: "longest_first"}.get(order_ran, str(order_ran))},
        "roofline": roof,
        "kernel_us": {"varlen_mean": round(float(dec_ms.mean()) * 1e3, 2),
                      "varlen_median": round(float(np.median(dec_ms)) * 1e3, 2),
                      "reduce_median": round(float(np.median(red_ms)) * 1e3, 2)},
        "kv_read_bytes": kv_bytes, "causal_flops": flops, "kv_pool_copies": ncopies,
        "input_gen_s": round(gen_s, 1),
    }
    if not compute_bound and not args.no_ceiling:
        # an HBM-bound launch: this box's read ceilings on the workload's pools
        result["ceiling"] = ceilings(wl, (q, k, v, bt, sl), P)
        result["roofline"]["of_ceiling"] = round(roof["achieved"] /
                                                 result["ceiling"]["read_ceiling_GBps"], 4)
    if emit:
        result["cpu_baseline"] = (None if args.no_cpu_baseline else
                                  cpu_baseline_varlen(wl, args.cpu_seconds, 3 * args.cpu_seconds,
                                                      compute_bound))
        print(json.dumps(result), flush=True)
    return result


ORDER_NAMES = {1: "grid", 2: "longest_first"}


class DecodeBench:
    """One decode workload on the device: inputs, rotated K/V pool copies,
    scratch, and the step (host plan + decode + reduce, or the single launch)
    timed with HIP events on the launch stream."""

    def __init__(self, wl, P_req, max_copies, fused=False, append=False):
        import numpy as np
        import torch
        from paged_gqa_kv_decode_amd import binding as vb
        from paged_gqa_kv_decode_amd.workloads import kv_read_bytes
        self.wl, self.P_req, self.fused, self.append = wl, P_req, fused, append
        self.dev = vb.device_inputs(wl)
        q, k, v, bt, sl = self.dev
        self.dtype_code = {"f16": vb.DTYPE_F16, "bf16": vb.DTYPE_BF16,
                           "f32": vb.DTYPE_F32}[wl.meta.get("dtype", "f16")]
        self.kv_bytes = kv_read_bytes(wl.seq_lens, wl.num_kv_heads, wl.head_dim,
                                      4 if self.dtype_code == vb.DTYPE_F32 else 2)
        # Successive steps rotate over identical copies of the K/V pools so
        # that at least 4x the 256 MB Infinity Cache is read between two reads
        # of the same page: every step streams its KV from HBM, as a layer's
        # decode does when the other layers' caches are read in between.
        self.ncopies = max(2, min(max_copies, -(-(4 * MALL_BYTES) // self.kv_bytes)))
        self.pools = [(k, v)] + [(k.clone(), v.clone()) for _ in range(self.ncopies - 1)]
        torch.cuda.synchronize()
        self.stream = torch.cuda.current_stream()
        self.out = torch.empty((wl.num_seqs, wl.num_q_heads, wl.head_dim), dtype=torch.float32,
                               device="cuda")
        # Scratch sized once from a first plan; every step plans again (host)
        # and reuses it (the plan depends only on the host seq_lens).
        self.step0 = vb.DecodeStep(q, k, v, bt, sl, wl.seq_lens, wl.scale, P_req, out=self.out,
                                   fused=fused, dtype=self.dtype_code)
        self.P, self.NP = self.step0.plan.partition_size, self.step0.plan.max_num_partitions
        self.counter = 0
        if append:
            # the K/V rows at slot L-1 of the workload and their positions
            self.last = torch.from_numpy((wl.seq_lens - 1).astype(np.int32)).cuda()
            blk = wl.block_tables[np.arange(wl.num_seqs), (wl.seq_lens - 1) // wl.block_size]
            slot = (wl.seq_lens - 1) % wl.block_size
            self.k_new = torch.from_numpy(np.ascontiguousarray(wl.k_cache[blk, :, slot, :])).cuda()
            self.v_new = torch.from_numpy(np.ascontiguousarray(wl.v_cache[blk, :, slot, :])).cuda()

    def one_step(self, ev=None, stream=None):
        from paged_gqa_kv_decode_amd import binding as vb
        wl, P, NP, st0, out = self.wl, self.P, self.NP, self.step0, self.out
        stream = stream if stream is not None else self.stream
        q, _, _, bt, sl = self.dev
        k, v = self.pools[self.counter % self.ncopies]
        self.counter += 1
        if self.append:
            if ev is not None:
                ev[3].record(stream)
            vb.paged_kv_append(self.k_new, self.v_new, bt, self.last, k, v, 10000.0, stream)
        plan = vb.plan_partitions(wl.seq_lens, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                  wl.block_size, wl.max_blocks_per_seq, self.P_req, 0)
        assert plan.partition_size == P and plan.max_num_partitions == NP
        if ev is not None:
            ev[0].record(stream)
        if self.fused:
            vb.paged_gqa_decode_fused(q, k, v, bt, sl, wl.scale, P, NP, out, st0.max_logits,
                                      st0.exp_sums, st0.tmp_out, st0.counters, stream)
            if ev is not None:
                ev[1].record(stream)
        elif self.dtype_code != vb.DTYPE_F16:
            vb.paged_gqa_decode_dt(self.dtype_code, q, k, v, bt, sl, wl.scale, P, NP,
                                   None if P else out, st0.max_logits, st0.exp_sums,
                                   st0.tmp_out, stream)
            if ev is not None:
                ev[1].record(stream)
            if P:
                vb.paged_gqa_reduce(st0.max_logits, st0.exp_sums, st0.tmp_out, sl, P, out, stream)
        elif P:
            vb.paged_gqa_decode(q, k, v, bt, sl, wl.scale, P, NP, None, st0.max_logits,
                                st0.exp_sums, st0.tmp_out, stream)
            if ev is not None:
                ev[1].record(stream)
            vb.paged_gqa_reduce(st0.max_logits, st0.exp_sums, st0.tmp_out, sl, P, out, stream)
        else:
            vb.paged_gqa_decode(q, k, v, bt, sl, wl.scale, 0, 1, out, stream=stream)
            if ev is not None:
                ev[1].record(stream)
        if ev is not None:
            ev[2].record(stream)

    def time(self, steps, warmup):
        """W untimed steps, then K steps between two device synchronisations;
        per-launch durations from HIP events recorded on the launch stream."""
        import numpy as np
        import torch
        from paged_gqa_kv_decode_amd import binding as vb
        for _ in range(warmup):
            self.one_step()
        torch.cuda.synchronize()
        kernel_ran, order_ran = vb.last_plan().kernel, vb.last_plan().work_order
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        torch.cuda.synchronize()
        t = time.perf_counter()
        for i in range(steps):
            self.one_step(events[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t
        dec_ms = np.array([e[0].elapsed_time(e[1]) for e in events])
        red_ms = np.array([e[1].elapsed_time(e[2]) for e in events])
        r = {"ms_per_step": wall * 1e3 / steps, "kernel": kernel_ran, "order": order_ran,
             "achieved_GBps": self.kv_bytes / (float(dec_ms.mean()) * 1e-3) / 1e9,
             "kernel_us": {"decode_mean": round(float(dec_ms.mean()) * 1e3, 2),
                           "decode_median": round(float(np.median(dec_ms)) * 1e3, 2),
                           "decode_p5": round(float(np.percentile(dec_ms, 5)) * 1e3, 2),
                           "decode_p95": round(float(np.percentile(dec_ms, 95)) * 1e3, 2),
                           "reduce_median": round(float(np.median(red_ms)) * 1e3, 2)}}
        if self.append:
            app_ms = np.array([e[3].elapsed_time(e[0]) for e in events])
            r["append_us_median"] = round(float(np.median(app_ms)) * 1e3, 2)
        return r

    def graphs(self):
        """One captured HIP graph per K/V pool copy, each holding one step's
        launches (decode + reduce, or the single launch; the append first when
        asked).  The kernels take no scratch that needs clearing, so nothing
        but the launches is recorded."""
        import torch
        if getattr(self, "_graphs", None) is None:
            cap = torch.cuda.Stream()
            torch.cuda.synchronize()
            gs = []
            for i in range(self.ncopies):
                g = torch.cuda.CUDAGraph()
                self.counter = i
                with torch.cuda.graph(g, stream=cap):
                    self.one_step(stream=cap)
                gs.append(g)
            torch.cuda.synchronize()
            self._graphs = gs
        return self._graphs

    def time_graph(self, steps, warmup):
        """W untimed steps, then exactly K steps between two device
        synchronisations, each the host plan and one graph replay (the pool
        copies in turn): ms per step."""
        import torch
        from paged_gqa_kv_decode_amd import binding as vb
        wl, gs = self.wl, self.graphs()
        for k in range(warmup):
            gs[k % len(gs)].replay()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for k in range(steps):
            plan = vb.plan_partitions(wl.seq_lens, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                      wl.block_size, wl.max_blocks_per_seq, self.P_req, 0)
            assert plan.partition_size == self.P
            gs[k % len(gs)].replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) * 1e3 / steps

    def time_flushed(self):
        """Median decode duration with a 512 MiB read before each step."""
        import numpy as np
        import torch
        L = _bench_lib()
        flush = torch.zeros(512 << 20, dtype=torch.uint8, device="cuda")
        fsink = torch.empty(4096 * 256, dtype=torch.int32, device="cuda")
        fl = []
        for _ in range(20):
            L.vkb_stream_read(flush.data_ptr(), flush.numel(), fsink.data_ptr(), 4096,
                              self.stream.cuda_stream)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            self.one_step(ev)
            torch.cuda.synchronize()
            fl.append(ev[0].elapsed_time(ev[1]))
        return round(float(np.median(fl)) * 1e3, 2)

    def release(self):
        import torch
        torch.cuda.synchronize()
        self.pools = None
        self.step0 = None
        self.out = None
        torch.cuda.empty_cache()


def cpu_single_thread():
    """The float64 oracle on one thread for the two small decode workloads
    (one sequence of 64 tokens; 8 sequences of up to 2048): median of 3 whole
    steps after one warm-up, ms."""
    import numpy as np
    import oracle
    from paged_gqa_kv_decode_amd.workloads import make_workload
    res = {}
    for name in ("tiny_1x64", "batch8_2k"):
        wl = make_workload(name)
        ts = []
        for _ in range(4):
            t = time.perf_counter()
            oracle.paged_attention_arrays(wl.q, wl.k_cache, wl.v_cache, wl.block_tables,
                                          wl.seq_lens, wl.scale, nthreads=1)
            ts.append(time.perf_counter() - t)
        res[name] = round(float(np.median(ts[1:])) * 1e3, 3)
    return res


def partition_sweep(args):
    """Multi-head and multi-query geometries, which the planner's budget was
    not calibrated on: decode + reduce at P = 256, 512 and 1024 (waves and
    order on auto; HIP events on the launch stream, 10 steps per segment in
    the order 256, 512, 1024, 1024, 512, 256, K/V pools rotated as in the
    timed step), beside the planner's own choice.  Inputs are random fp16
    drawn on the device (timing only).  One JSON line per batch."""
    import numpy as np
    import torch
    from paged_gqa_kv_decode_amd import binding as vb
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    geoms = [((16, 16, 128), 16), ((8, 8, 256), 16), ((16, 1, 128), 16), ((16, 1, 256), 32)]
    rng = np.random.default_rng(5)
    batches = [(f"{S}x32768", [32768] * S) for S in (1, 2, 4, 8, 16, 32)]
    batches += [(f"{S}xU[1,32768]", list(rng.integers(1, 32769, S))) for S in (8, 32, 64)]
    stream = torch.cuda.current_stream()
    sizes = (256, 512, 1024)
    for (Hq, Hkv, D), bs in geoms:
        for name, lens in batches:
            lens = np.asarray(lens, dtype=np.int32)
            S = len(lens)
            pages = [-(-int(L) // bs) for L in lens]
            pool = int(sum(pages))
            perm = rng.permutation(pool).astype(np.int32)
            bt = np.zeros((S, max(pages)), dtype=np.int32)
            o = 0
            for i, n in enumerate(pages):
                bt[i, :n] = perm[o:o + n]
                o += n
            kv_bytes = 4 * Hkv * D * int(lens.sum())
            ncopies = max(2, min(16, -(-(4 * MALL_BYTES) // kv_bytes)))
            q = torch.randn((S, Hq, D), device="cuda").half()
            pools = [(torch.randn((pool, Hkv, bs, D), device="cuda").half(),
                      torch.randn((pool, Hkv, bs, D), device="cuda").half()) for _ in range(ncopies)]
            btd, sld = torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda()
            steps = {P: vb.DecodeStep(q, pools[0][0], pools[0][1], btd, sld, lens, D ** -0.5, P)
                     for P in sizes}
            times = {P: [] for P in sizes}
            ctr = [0]

            def seg(P, n, record):
                st = steps[P]
                for _ in range(n):
                    k, v = pools[ctr[0] % ncopies]
                    ctr[0] += 1
                    st.args = (q, k, v, btd, sld)
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    st.run()
                    e1.record(stream)
                    if record:
                        times[P].append((e0, e1))
            for P in sizes:
                seg(P, 3, False)
            for P in sizes + sizes[::-1]:
                seg(P, 10, True)
            torch.cuda.synchronize()
            us = {P: round(float(np.mean([a.elapsed_time(b) for a, b in times[P]])) * 1e3, 2)
                  for P in sizes}
            plan = vb.plan_partitions(lens, Hq, Hkv, D, bs, bt.shape[1], -1, cu)
            best = min(us, key=us.get)
            print(json.dumps({"partition_sweep": f"{Hq}q{Hkv}kv{D}", "block_size": bs, "batch": name,
                              "us_per_step": {str(P): us[P] for P in sizes},
                              "planner": plan.partition_size, "best": best,
                              "planner_loss_pct": round(100 * (us[plan.partition_size] / us[best] - 1), 1),
                              "w512_per_cu": round(Hq * int((lens // 512).sum()) / cu, 1),
                              "kv_GB": round(kv_bytes / 1e9, 3)}), flush=True)
            del pools, steps
            torch.cuda.empty_cache()


def wave_sweep(args):
    """The data behind the 1024-first planner step and the four-wave launch
    of 1024-token partitions: decode + reduce at P = 512 (waves on auto) and
    at P = 1024 with auto, one, two and four waves per partition, over the
    eight geometries and 15 batches (HIP events, 8 steps per segment in the
    order of the variants and back, K/V pools rotated).  Random fp16 inputs
    drawn on the device (timing only).  One JSON line per batch."""
    import numpy as np
    import torch
    from paged_gqa_kv_decode_amd import binding as vb
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    geoms = [((32, 8, 128), 16), ((24, 4, 256), 32), ((16, 2, 128), 8), ((16, 2, 256), 32),
             ((16, 16, 128), 16), ((8, 8, 256), 16), ((16, 1, 128), 16), ((16, 1, 256), 32)]
    rng = np.random.default_rng(5)
    batches = [(f"{S}x32768", [32768] * S) for S in (1, 2, 3, 4, 6, 8, 10, 12, 16, 24)]
    batches += [(f"{S}xU[1,32768]", list(rng.integers(1, 32769, S))) for S in (8, 16, 32, 64)]
    batches += [("32xU[4k,16k]", list(rng.integers(4096, 16385, 32)))]
    stream = torch.cuda.current_stream()
    variants = [("512", 512, vb.KERNEL_AUTO), ("1024", 1024, vb.KERNEL_AUTO),
                ("1024_w1", 1024, vb.KERNEL_MFMA_W1), ("1024_w2", 1024, vb.KERNEL_MFMA_W2),
                ("1024_w4", 1024, vb.KERNEL_MFMA_W4)]
    for (Hq, Hkv, D), bs in geoms:
        for name, lens in batches:
            lens = np.asarray(lens, dtype=np.int32)
            S = len(lens)
            pages = [-(-int(L) // bs) for L in lens]
            pool = int(sum(pages))
            perm = rng.permutation(pool).astype(np.int32)
            bt = np.zeros((S, max(pages)), dtype=np.int32)
            o = 0
            for i, n in enumerate(pages):
                bt[i, :n] = perm[o:o + n]
                o += n
            kv_bytes = 4 * Hkv * D * int(lens.sum())
            ncopies = max(2, min(16, -(-(4 * MALL_BYTES) // kv_bytes)))
            q = torch.randn((S, Hq, D), device="cuda").half()
            pools = [(torch.randn((pool, Hkv, bs, D), device="cuda").half(),
                      torch.randn((pool, Hkv, bs, D), device="cuda").half()) for _ in range(ncopies)]
            btd, sld = torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda()
            steps = {t: vb.DecodeStep(q, pools[0][0], pools[0][1], btd, sld, lens, D ** -0.5, P)
                     for t, P, _ in variants}
            kern = {t: k for t, _, k in variants}
            times = {t: [] for t, _, _ in variants}
            ctr = [0]

            def seg(t, n, record):
                prev = vb.select_decode_kernel(kern[t])
                try:
                    st = steps[t]
                    for _ in range(n):
                        k, v = pools[ctr[0] % ncopies]
                        ctr[0] += 1
                        st.args = (q, k, v, btd, sld)
                        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                        e0.record(stream)
                        st.run()
                        e1.record(stream)
                        if record:
                            times[t].append((e0, e1))
                finally:
                    vb.select_decode_kernel(prev)
            tags = [t for t, _, _ in variants]
            for t in tags:
                seg(t, 3, False)
            for t in tags + tags[::-1]:
                seg(t, 8, True)
            torch.cuda.synchronize()
            us = {t: round(float(np.mean([a.elapsed_time(b) for a, b in times[t]])) * 1e3, 2) for t in tags}
            plan = vb.plan_partitions(lens, Hq, Hkv, D, bs, bt.shape[1], -1, cu)
            print(json.dumps({"wave_sweep": f"{Hq}q{Hkv}kv{D}", "block_size": bs, "batch": name,
                              "us_per_step": us, "planner": plan.partition_size,
                              "full1024_workgroups_per_cu": round(Hkv * int((lens // 1024).sum()) / cu, 2),
                              "kv_GB": round(kv_bytes / 1e9, 3)}), flush=True)
            del pools, steps
            torch.cuda.empty_cache()


def planner_sweep(args):
    """The data behind the partition planner's budget: for the four
    grouped-query geometries and a range of batches, decode + reduce at P =
    256 against P = 512 (HIP events on the launch stream, 10 steps per
    segment in ABBA order, K/V pools rotated as in the timed step), beside
    the full-partition work W(512) = Hq * sum_s floor(L_s / 512) per CU in
    the pages' query-head units (their budget: 33 per CU) and in workgroups,
    Hkv * sum_s floor(L_s / 512) per CU (the library's default budget: 4 per
    CU, i.e. 4 * G query-head units).  The summary scores both rules and the
    best threshold in each unit by the time lost against the faster size.
    Inputs are random fp16 drawn on the device (timing only)."""
    import numpy as np
    import torch
    from paged_gqa_kv_decode_amd import binding as vb
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    geoms = [((32, 8, 128), 16), ((24, 4, 256), 32), ((16, 2, 128), 8), ((16, 2, 256), 32)]
    rng = np.random.default_rng(5)
    batches = [(f"{S}x32768", [32768] * S) for S in (1, 2, 3, 4, 6, 8, 10, 12, 16, 24)]
    batches += [(f"{S}xU[1,32768]", list(rng.integers(1, 32769, S))) for S in (8, 16, 32, 64)]
    stream = torch.cuda.current_stream()
    rows = []
    for (Hq, Hkv, D), bs in geoms:
        for name, lens in batches:
            lens = np.asarray(lens, dtype=np.int32)
            S = len(lens)
            pages = [-(-int(L) // bs) for L in lens]
            pool = int(sum(pages))
            perm = rng.permutation(pool).astype(np.int32)
            bt = np.zeros((S, max(pages)), dtype=np.int32)
            o = 0
            for i, n in enumerate(pages):
                bt[i, :n] = perm[o:o + n]
                o += n
            kv_bytes = 4 * Hkv * D * int(lens.sum())
            ncopies = max(2, min(16, -(-(4 * MALL_BYTES) // kv_bytes)))
            q = torch.randn((S, Hq, D), device="cuda").half()
            pools = [(torch.randn((pool, Hkv, bs, D), device="cuda").half(),
                      torch.randn((pool, Hkv, bs, D), device="cuda").half()) for _ in range(ncopies)]
            btd, sld = torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda()
            steps = {P: vb.DecodeStep(q, pools[0][0], pools[0][1], btd, sld, lens, D ** -0.5, P)
                     for P in (256, 512)}
            times = {256: [], 512: []}
            ctr = [0]

            def seg(P, n, record):
                st = steps[P]
                for _ in range(n):
                    k, v = pools[ctr[0] % ncopies]
                    ctr[0] += 1
                    st.args = (q, k, v, btd, sld)
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    st.run()
                    e1.record(stream)
                    if record:
                        times[P].append((e0, e1))
            for P in (256, 512):
                seg(P, 3, False)
            for P in (256, 512, 512, 256):
                seg(P, 10, True)
            torch.cuda.synchronize()
            us = {P: float(np.mean([a.elapsed_time(b) for a, b in times[P]])) * 1e3 for P in times}
            w512 = Hq * int((lens // 512).sum())
            plan = vb.plan_partitions(lens, Hq, Hkv, D, bs, bt.shape[1], -1, cu)
            r = {"geometry": [Hq, Hkv, D], "block_size": bs, "batch": name,
                 "w512_per_cu": round(w512 / cu, 2),
                 "wg512_per_cu": round(Hkv * int((lens // 512).sum()) / cu, 3),
                 "us_P256": round(us[256], 2),
                 "us_P512": round(us[512], 2), "faster": 256 if us[256] < us[512] else 512,
                 "planner": plan.partition_size}
            rows.append(r)
            print(json.dumps(r), flush=True)
            del pools, steps, q
            torch.cuda.empty_cache()
    # each rule's misses against the faster size and the time they lose; the
    # best threshold per unit is the one losing the least time (ties: fewer
    # misses)
    def score(key, b):
        wrong = [r for r in rows if (512 if r[key] >= b else 256) != r["faster"]]
        loss = sum(abs(r["us_P256"] - r["us_P512"]) for r in wrong)
        return (round(loss, 2), len(wrong))
    best_q = min(sorted({r["w512_per_cu"] for r in rows} | {33.0}), key=lambda b: score("w512_per_cu", b))
    best_w = min(sorted({r["wg512_per_cu"] for r in rows} | {4.0}), key=lambda b: score("wg512_per_cu", b))
    print(json.dumps({"planner_sweep": "summary", "cu_count": cu, "configs": len(rows),
                      "pages_budget_33": dict(zip(("loss_us", "wrong"), score("w512_per_cu", 33.0))),
                      "default_4_workgroups": dict(zip(("loss_us", "wrong"), score("wg512_per_cu", 4.0))),
                      "best_query_head_threshold": best_q,
                      "best_query_head": dict(zip(("loss_us", "wrong"), score("w512_per_cu", best_q))),
                      "best_workgroup_threshold": best_w,
                      "best_workgroup": dict(zip(("loss_us", "wrong"), score("wg512_per_cu", best_w)))}),
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="long4_128k", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--dtype", default="f16", choices=["f16", "bf16", "f32"],
                    help="element type of q / K / V (with --shape)")
    ap.add_argument("--shape", default=None,
                    help="time a custom shape instead: S,Hq,Hkv,D,bs,Lmin,Lmax (lengths uniform "
                         "in [Lmin, Lmax], seeded; pages shuffled in an exact-fit pool)")
    ap.add_argument("--partition", type=int, default=None,
                    help="-1 planner, 0 unsplit, 256/512 forced (default: the workload's own)")
    ap.add_argument("--kernel", default="auto", choices=["auto", "dot", "mfma", "mfma1", "mfma2", "mfma4", "mfma4p2"])
    ap.add_argument("--varlen-kernel", default="auto", choices=["auto", "columns", "tiles"],
                    help="multi-token workloads: kernel (auto: tiles from 4 query tokens)")
    ap.add_argument("--order", default="auto", choices=["auto", "grid", "longest"],
                    help="work order of the matrix-core decode (A/B switch)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum wall time of the oracle sample (cpu_baseline)")
    ap.add_argument("--append", action="store_true",
                    help="each step first appends one token per sequence to the paged cache "
                         "(vk_paged_kv_append with rotary K, theta 10000): it rewrites slot L-1 "
                         "with that token's K rotated for position L-1 and its V, the same "
                         "values every step; reported as append_us_median")
    ap.add_argument("--eager", action="store_true",
                    help="time the headline steps as eager launches (default: each step's "
                         "launches replayed from a captured HIP graph, the host plan still run "
                         "every step; the eager time is reported beside it either way)")
    ap.add_argument("--fused", action="store_true",
                    help="single launch: decode with the partials merged in place "
                         "(vk_paged_gqa_decode_fused) instead of decode + reduce")
    ap.add_argument("--max-copies", type=int, default=256,
                    help="cap on the rotated K/V pool copies")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the box's read-bandwidth ceilings on the KV pools")
    ap.add_argument("--no-configs", action="store_true",
                    help="default workload: skip timing the other long-context workloads "
                         "(long32_16k at P=256, 512 and the planner's choice, mixed64_32k at 512 and the planner's choice)")
    ap.add_argument("--flush", action="store_true",
                    help="also time the decode with a 512 MiB cache flush before each run")
    ap.add_argument("--planner-sweep", action="store_true",
                    help="time P=256 against P=512 over geometries and batches (the data "
                         "behind the planner's budget); prints one JSON line per batch")
    ap.add_argument("--partition-sweep", action="store_true",
                    help="time P=256, 512 and 1024 on multi-head and multi-query geometries "
                         "beside the planner's choice; prints one JSON line per batch")
    ap.add_argument("--wave-sweep", action="store_true",
                    help="time P=512 against P=1024 with 1, 2 and 4 waves per partition over "
                         "eight geometries and 15 batches; prints one JSON line per batch")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy, --steps times (the "
                         "known-size reference for the HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(f"bench.py: this path runs on one GPU only (asked for {max(args.gpus, world)}); "
              "the library has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from paged_gqa_kv_decode_amd import binding as vb

    if args.planner_sweep:
        return planner_sweep(args)
    if args.partition_sweep:
        return partition_sweep(args)
    if args.wave_sweep:
        return wave_sweep(args)
    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t) / args.steps
        print(json.dumps({"copy_bytes": n, "steps": args.steps, "ms": round(dt * 1e3, 4),
                          "read_GBps": round(n / dt / 1e9, 1)}), flush=True)
        return
    from paged_gqa_kv_decode_amd.workloads import kv_read_bytes, make_workload

    t0 = time.time()
    if args.shape:
        from paged_gqa_kv_decode_amd.workloads import make_custom
        S_, Hq_, Hkv_, D_, bs_, lo_, hi_ = (int(x) for x in args.shape.split(","))
        lens_ = np.random.default_rng(7).integers(lo_, hi_ + 1, S_)
        wl = make_custom(seq_lens=lens_, num_q_heads=Hq_, num_kv_heads=Hkv_, head_dim=D_,
                         block_size=bs_, seed=7, dtype=args.dtype)
        wl.partition_sizes = (-1,)
        args.workload = f"custom_{args.shape}"
        DESCRIPTIONS[args.workload] = (f"{S_} seqs, L uniform in [{lo_}, {hi_}], "
                                       f"({Hq_}q, {Hkv_}kv, {D_}), block {bs_}, {args.dtype}")
    elif args.workload in VARLEN:
        from paged_gqa_kv_decode_amd.workloads import make_varlen
        if args.dtype not in ("f16", "bf16"):
            raise SystemExit("bench.py: multi-token workloads run in f16 or bf16")
        wl = make_varlen(args.workload, dtype=args.dtype)
        return bench_varlen(args, wl, time.time() - t0)
    else:
        if args.dtype != "f16":
            raise SystemExit("bench.py: the named decode workloads are fp16; "
                             "use --shape S,Hq,Hkv,D,bs,lo,hi with --dtype bf16 or f32")
        wl = make_workload(args.workload)
    gen_s = time.time() - t0
    P_req = args.partition if args.partition is not None else wl.partition_sizes[0]
    kernel = {"auto": vb.KERNEL_AUTO, "dot": vb.KERNEL_DOT, "mfma": vb.KERNEL_MFMA,
              "mfma1": vb.KERNEL_MFMA_W1, "mfma2": vb.KERNEL_MFMA_W2,
              "mfma4": vb.KERNEL_MFMA_W4, "mfma4p2": vb.KERNEL_MFMA_W4P2}[args.kernel]
    vb.select_decode_kernel(kernel)
    vb.select_work_order({"auto": vb.ORDER_AUTO, "grid": vb.ORDER_GRID,
                          "longest": vb.ORDER_LONGEST_FIRST}[args.order])

    db = DecodeBench(wl, P_req, args.max_copies, fused=args.fused, append=args.append)
    tm = db.time(args.steps, args.warmup)          # eager launches, per-kernel HIP events
    P, NP, kv_bytes, ncopies = db.P, db.NP, db.kv_bytes, db.ncopies
    ms_eager = tm["ms_per_step"]
    ms_step = ms_eager if args.eager else db.time_graph(args.steps, args.warmup)
    traffic = load_traffic(args.workload, P, tm["kernel"], args.fused)

    result = {
        "metric": "decode-attention µs/step and KV-read HBM GB/s (% of MI355X peak)",
        "value": round(kv_bytes / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "us_per_step": round(ms_step * 1e3, 2),
        "step_launch": "eager" if args.eager else "graph",
        "us_per_step_eager": round(ms_eager * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.meta.get("dtype", "f16"),
        "data": f"synthetic (seeded N(0, sigma) {wl.meta.get('dtype', 'f16')} K/V/q, shuffled pages)",
        "config": {"workload": args.workload, "description": DESCRIPTIONS[args.workload],
                   "num_seqs": wl.num_seqs, "num_q_heads": wl.num_q_heads,
                   "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
                   "block_size": wl.block_size, "sum_seq_len": int(wl.seq_lens.sum()),
                   "partition_size": P, "max_num_partitions": NP,
                   "decode_kernel": KERNEL_NAMES.get(tm["kernel"], str(tm["kernel"])),
                   "work_order": ORDER_NAMES.get(tm["order"], str(tm["order"])),
                   "single_launch": bool(args.fused), "with_append": bool(args.append)},
        "roofline": {"bound": "hbm", "achieved": round(tm["achieved_GBps"], 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(tm["achieved_GBps"] / HBM_PEAK_GBS, 4), "traffic": traffic},
        "traffic_source": (None if traffic is None else
                           f"stored: profiles/decode_{args.workload}_P{P}"
                           f"{'_fused' if args.fused else ''}_traffic.txt (rocprofv3 FETCH_SIZE + "
                           "WRITE_SIZE per launch, calibrated; used only while the kernel "
                           "sources hash to the value recorded there)"),
        "kernel_us": tm["kernel_us"],
        **({"append_us_median": tm["append_us_median"]} if args.append else {}),
        "kv_read_bytes": kv_bytes,
        "kv_pool_copies": ncopies,
        "bytes_read_between_reuse": (ncopies - 1) * kv_bytes,
        "input_gen_s": round(gen_s, 1),
    }
    if args.flush:
        result["kernel_us"]["decode_median_flushed"] = db.time_flushed()
    if not args.no_ceiling:
        result["ceiling"] = ceilings(wl, db.dev, P)
    db.release()
    if (not args.no_configs and not args.shape and not args.fused and not args.append
            and args.workload == "long4_128k" and args.partition is None):
        # The other long-context workloads, timed the same way in this run.
        configs = {}
        for name, p_req in (("long32_16k", 256), ("long32_16k", 512), ("long32_16k", -1),
                            ("mixed64_32k", 512), ("mixed64_32k", -1)):
            key = f"{name}_P{p_req}" if p_req > 0 else f"{name}_planner"
            wl2 = make_workload(name)
            db2 = DecodeBench(wl2, p_req, args.max_copies)
            t2 = db2.time(args.steps, args.warmup)
            configs[key] = {
                "partition_size": db2.P, "kv_read_bytes": db2.kv_bytes,
                "decode_us_mean": t2["kernel_us"]["decode_mean"],
                "decode_us_median": t2["kernel_us"]["decode_median"],
                "reduce_us_median": t2["kernel_us"]["reduce_median"],
                "us_per_step": round(t2["ms_per_step"] * 1e3, 2),
                "kv_TBps": round(t2["achieved_GBps"] / 1e3, 3),
                "frac": round(t2["achieved_GBps"] / HBM_PEAK_GBS, 4),
                "decode_kernel": KERNEL_NAMES.get(t2["kernel"], str(t2["kernel"])),
                "work_order": ORDER_NAMES.get(t2["order"], str(t2["order"]))}
            if not args.no_ceiling:
                # this workload's own read ceiling (its page size and page list)
                c2 = ceilings(wl2, db2.dev, db2.P)
                configs[key].update({
                    "read_ceiling_GBps": c2["read_ceiling_GBps"],
                    "read_ceiling_kernel": c2["read_ceiling_kernel"],
                    "page_bytes": c2["page_bytes"],
                    "of_ceiling": round(t2["achieved_GBps"] / c2["read_ceiling_GBps"], 4)})
            db2.release()
            del wl2
            print(f"bench: {key}: decode {t2['kernel_us']['decode_mean']} us "
                  f"({configs[key]['frac']:.3f} of peak)", file=sys.stderr,
                  flush=True)
        # The multi-token workloads (verification rows, a chunked prefill),
        # timed as `--workload <name>` would, planner and kernel choice auto.
        import copy
        import torch
        from paged_gqa_kv_decode_amd.workloads import make_varlen
        for name in VARLEN:
            a3 = copy.copy(args)
            a3.partition, a3.varlen_kernel, a3.order, a3.dtype = None, "auto", "auto", "f16"
            r3 = bench_varlen(a3, make_varlen(name), 0.0, emit=False)
            torch.cuda.empty_cache()
            roof = r3["roofline"]
            configs[name] = {
                "partition_size": r3["config"]["partition_size"],
                "kernel": r3["config"]["decode_kernel"],
                "kernel_us_mean": r3["kernel_us"]["varlen_mean"],
                "reduce_us_median": r3["kernel_us"]["reduce_median"],
                "us_per_step": r3["us_per_step"],
                "bound": roof["bound"], "rate": roof["achieved"], "rate_unit": roof["unit"],
                "frac": roof["frac"]}
            if "ceiling" in r3:
                configs[name].update({"read_ceiling_GBps": r3["ceiling"]["read_ceiling_GBps"],
                                      "read_ceiling_kernel": r3["ceiling"]["read_ceiling_kernel"],
                                      "page_bytes": r3["ceiling"]["page_bytes"],
                                      "of_ceiling": roof["of_ceiling"]})
            print(f"bench: {name}: kernel {r3['kernel_us']['varlen_mean']} us "
                  f"({roof['frac']:.3f} of the {roof['bound']} peak)", file=sys.stderr, flush=True)
        result["configs"] = configs
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, 3 * args.cpu_seconds)
        if args.workload == "long4_128k" and not args.shape:
            result["cpu_baseline"]["single_thread_ms"] = cpu_single_thread()
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
