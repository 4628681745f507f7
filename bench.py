"""Benchmark: one decode step of PagedAttention on MI355X.

A step is the whole hot path for one batch: the slot write of the step's new
tokens (pa_reshape_and_cache) followed by PagedAttention decode (pa_decode:
the per-partition kernel, plus the log-sum-exp reduce in split mode), all on
one HIP stream, with every input already resident in HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

NAME is one of the decode workloads (default gqa_bf16), a beam-search
workload (beam_bf16, beam_tiny_bf16), whose measured step is its last one:
that step's copy-on-write block copies (pa_copy_blocks), its slot write and
the decode of every beam, or the chunked-prefill workload (prefill_bf16):
the chunk's slot write plus pa_prefill, priced against the matrix-core peak.

Prints ONE JSON line.  `value` is the achieved KV-read bandwidth of the whole
step (logical KV bytes the step's queries read / step time, in GB/s);
`tokens_per_s` is the decode throughput (sequences advanced per second, one
layer).  `roofline` prices the dominant kernel (the decode kernel) against
MI355X's 8 TB/s HBM peak with its algorithmic bytes (unique KV blocks + q +
out + block tables + context lengths) over its average duration, measured
with HIP events on the launch stream.  With the default workload the same
line also carries, under `workloads`, the two other bf16 GQA decode
workloads (shared-prefix sampling and long-context split decode), each timed
the same way with its own roofline, and `stream_read`, the rate of a plain
streaming read of a 2 GiB buffer on the same GPU (context for the roofline).
`cpu_baseline` times the CPU oracle (float64 concatenate-then-attend plus
the slot write) on a bounded sample of the headline workload on this host's
cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import types
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention: achieved KV-read GB/s (% HBM peak) and tokens/s"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix-core peak
DEFAULT_CONFIG = "gqa_bf16"
# Sources of the decode launch (slot write, decode kernels, merges and the
# host code that plans them): HBM byte counters stored for a decode workload
# stay valid while these hash the same.  The copy-on-write and prefill kernels
# are separate launches and do not take part.
KERNEL_SOURCES = ["pa_decode_mfma.hip", "pa_decode_shared.hip", "pa_decode_vector.hip",
                  "pa_reduce.hip", "pa_cache_write.hip", "pa_api.cpp", "pa_internal.h",
                  "pa_mfma_tile.h"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default=DEFAULT_CONFIG)
    ap.add_argument("--algo", default="auto", choices=["auto", "vector", "mfma"])
    ap.add_argument("--partition", type=int, default=None,
                    help="partition size (0 single pass, -1 library choice); default: workload's")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU work for the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra-workloads", action="store_true",
                    help="time only --config (no shared-prefix / long-context records, no "
                         "streaming-read ceiling): for per-workload profiler runs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="instead of the benchmark, copy a 1 GiB buffer with torch 5 times "
                         "(reference for scaling HBM byte counters)")
    return ap.parse_args()


def copy_calibration():
    """A plain device copy of known size, to calibrate FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}), flush=True)


def decode_kernel_name(c, part, algo):
    """The kernel the decode phase runs (the roofline's dominant kernel)."""
    mfma = (c.dtype == "bf16" and c.head_dim == 128 and c.block_size >= 16
            and c.num_q_heads // c.num_kv_heads <= 16 and algo != "vector")
    if part == -3:
        return "decode_shared_kernel (after plan_shared_kernel)"
    if not mfma:
        return "decode_vector_balanced_kernel" if part == -2 else "decode_vector_kernel"
    return "decode_mfma_kernel" if part == 0 else "decode_mfma_balanced_kernel"


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_261_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(config, algo_name, partition):
    """HBM traffic per decode launch from committed rocprofv3 counter runs,
    if they were taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(f"{config}/{algo_name}/{partition}")
    if not rec or rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


class BeamLastStep:
    """The last step of a beam-search workload, seen as a one-step decode
    workload: the steps before it are replayed (copies and writes) before
    timing; the timed step is its copy-on-write copies, its slot write and
    the decode of every beam."""

    def __init__(self, bw):
        self.bw = bw
        c = bw.cfg
        last = bw.steps[-1]
        self.cfg = types.SimpleNamespace(
            name=c.name, description=c.description, num_seqs=c.num_seqs,
            num_q_heads=c.num_q_heads, num_kv_heads=c.num_kv_heads, head_dim=c.head_dim,
            block_size=c.block_size, num_blocks=c.num_blocks, dtype=c.dtype, scale=c.scale,
            partition_size=c.partition_size)
        self.prefill_k, self.prefill_v, self.prefill_slots = bw.prefill_k, bw.prefill_v, \
            bw.prefill_slots
        self.earlier_steps = bw.steps[:-1]
        self.cow = last.cow
        self.step_k, self.step_v, self.step_slots, self.q = [last.k], [last.v], [last.slots], \
            [last.q]
        self._last = last

    def ctx_at(self, s):
        return self._last.ctx

    def tables_at(self, s):
        return self._last.tables

    def kv_logical_bytes(self, s):
        return self.bw.kv_logical_bytes(len(self.bw.steps) - 1)

    def kv_unique_bytes(self, s):
        return self.bw.kv_unique_bytes(len(self.bw.steps) - 1)


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_threads():
    """Threads for the oracle baseline: every core this process may run on,
    but no more than the host's CPU share for one GPU where the environment
    states it (OMP_NUM_THREADS)."""
    n = len(os.sched_getaffinity(0))
    share = os.environ.get("OMP_NUM_THREADS", "")
    if share.isdigit() and int(share) > 0:
        n = min(n, int(share))
    return max(1, n)


def cpu_baseline(w, target_seconds):
    """Time the oracle (slot write of the step's tokens + float64
    concatenate-then-attend) on a bounded prefix of the batch, on every
    thread cpu_threads() allows and on one thread."""
    from oracle import pao
    c = w.cfg
    cores = cpu_threads()
    kh = np.zeros((c.num_blocks, c.num_kv_heads, c.block_size, c.head_dim),
                  dtype=w.prefill_k.dtype)
    vh = np.zeros_like(kh)
    pao.slot_write(kh, vh, w.prefill_k, w.prefill_v, w.prefill_slots, c.block_size)
    for st in getattr(w, "earlier_steps", []):
        for src, dst in st.cow:
            pao.copy_block(kh, vh, int(src), int(dst))
        pao.slot_write(kh, vh, st.k, st.v, st.slots, c.block_size)
    cow = getattr(w, "cow", [])
    ctx, tab, q = w.ctx_at(0), w.tables_at(0), w.q[0]
    es = 2 if c.dtype == "bf16" else 4

    def run(n, threads):
        t = time.perf_counter()
        for src, dst in cow:
            pao.copy_block(kh, vh, int(src), int(dst))
        pao.slot_write(kh, vh, w.step_k[0][:n], w.step_v[0][:n], w.step_slots[0][:n],
                       c.block_size)
        pao.decode_concat(q[:n], kh, vh, tab[:n], ctx[:n], c.scale, nthreads=threads)
        return time.perf_counter() - t

    def kv_bytes(n):
        return int(ctx[:n].astype(np.int64).sum()) * c.num_kv_heads * c.head_dim * 2 * es

    # all threads: grow the prefix until one run takes a quarter of the
    # budget (or the batch is whole), then repeat it within the budget; median
    n = min(c.num_seqs, max(1, cores))
    dt = run(n, cores)
    while n < c.num_seqs and dt < target_seconds / 4:
        n = min(c.num_seqs, n * 2)
        dt = run(n, cores)
    times = [dt]
    while sum(times) < target_seconds and len(times) < 40:
        times.append(run(n, cores))
    dt = statistics.median(times)
    # one thread, on a prefix about 1/cores as long
    n1 = max(1, n // cores)
    t1 = run(n1, 1)
    return {"value": round(kv_bytes(n) / dt / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"first {n} of {c.num_seqs} sequences of {c.name} "
                      f"(sum ctx {int(ctx[:n].sum())}), one step, median of {len(times)} "
                      f"runs, {dt:.3f} s each",
            "cpu_model": cpu_model(),
            "cores_available": len(os.sched_getaffinity(0)),
            "threads_rule": "every core in the process's affinity mask, capped by "
                            "OMP_NUM_THREADS (the host's CPU share per GPU) where set",
            "tokens_per_s": round(n / dt, 3),
            "single_thread": {"value": round(kv_bytes(n1) / t1 / 1e9, 4), "unit": "GB/s",
                              "sample": f"first {n1} sequences, {t1:.3f} s"}}


def bench_prefill(args, torch, pa, S, dev):
    """A prefill step: the chunk's slot write plus causal prefill of every
    chunk row.  The prefill kernel is priced against the bf16 matrix-core
    peak (its flops: 4 d Hq per (query row, visible key))."""
    w = S.make_prefill_workload(args.config)
    c = w.cfg

    def dev_t(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    shape = (c.num_blocks, c.num_kv_heads, c.block_size, c.head_dim)
    k_cache = torch.zeros(shape, dtype=torch.bfloat16, device=dev)
    v_cache = torch.zeros(shape, dtype=torch.bfloat16, device=dev)
    pa.pa_reshape_and_cache(dev_t(w.prefix_k), dev_t(w.prefix_v), k_cache, v_cache,
                            dev_t(w.prefix_slots))
    ck, cv, cs = dev_t(w.chunk_k), dev_t(w.chunk_v), dev_t(w.chunk_slots)
    q, tables, cu, ctx = dev_t(w.q), dev_t(w.tables), dev_t(w.cu_seqlens_q), dev_t(w.ctx)
    out = torch.empty_like(q)
    max_ctx, max_q = int(w.ctx.max()), int(w.chunk_lens.max())
    stream = torch.cuda.current_stream()

    def step(evs=None):
        if evs is not None:
            evs[0].record(stream)
        pa.pa_reshape_and_cache(ck, cv, k_cache, v_cache, cs, stream=stream)
        if evs is not None:
            evs[1].record(stream)
        pa.pa_prefill(out, q, k_cache, v_cache, tables, cu, ctx, max_ctx, max_q, c.scale,
                      stream=stream)
        if evs is not None:
            evs[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    t_write = statistics.mean(e[0].elapsed_time(e[1]) for e in evs)
    t_pf = statistics.mean(e[1].elapsed_time(e[2]) for e in evs)
    ms_step = wall / args.steps * 1e3
    flops = w.flops()
    kv = w.kv_bytes()
    tflops = flops / (t_pf * 1e-3) / 1e12
    result = {
        "metric": METRIC, "value": round(kv / (ms_step * 1e-3) / 1e9, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": c.dtype, "data": "synthetic",
        "config": {"workload": c.name, "description": c.description, "batch": c.num_seqs,
                   "total_q": int(w.cu_seqlens_q[-1]), "sum_context": int(w.ctx.sum()),
                   "num_q_heads": c.num_q_heads, "num_kv_heads": c.num_kv_heads,
                   "head_dim": c.head_dim, "block_size": c.block_size,
                   "parallelism": "none (1 GPU)"},
        "tokens_per_s": round(int(w.cu_seqlens_q[-1]) / (ms_step * 1e-3), 1),
        "kernels_ms": {"reshape_and_cache": round(t_write, 5), "prefill": round(t_pf, 5)},
        "flops": flops,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "prefill_mfma_kernel"},
    }
    print(json.dumps(result), flush=True)


class DecodeRun:
    """One decode workload resident on the GPU: pools built through the slot
    write, the step's inputs, the workspace of its split mode, and the step
    itself (copy-on-write copies where the workload has them, the slot
    write, decode phase 1 and the merge)."""

    def __init__(self, w, torch, pa, dev, algo, algo_name, part_req):
        self.w, self.torch, self.pa, self.algo, self.algo_name = w, torch, pa, algo, algo_name
        c = self.c = w.cfg
        tdt = torch.bfloat16 if c.dtype == "bf16" else torch.float32

        def dev_t(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
            return torch.from_numpy(a).to(dev)

        self.dev_t = dev_t
        shape = (c.num_blocks, c.num_kv_heads, c.block_size, c.head_dim)
        self.k_cache = torch.zeros(shape, dtype=tdt, device=dev)
        self.v_cache = torch.zeros(shape, dtype=tdt, device=dev)
        pa.pa_reshape_and_cache(dev_t(w.prefill_k), dev_t(w.prefill_v), self.k_cache,
                                self.v_cache, dev_t(w.prefill_slots))
        for st in getattr(w, "earlier_steps", []):   # beam workloads: steps before the last
            if len(st.cow):
                pa.pa_copy_blocks(self.k_cache, self.v_cache, dev_t(st.cow))
            pa.pa_reshape_and_cache(dev_t(st.k), dev_t(st.v), self.k_cache, self.v_cache,
                                    dev_t(st.slots))
        cow_h = getattr(w, "cow", np.zeros((0, 2), dtype=np.int32))
        self.cow = dev_t(cow_h) if len(cow_h) else None
        self.q = dev_t(w.q[0])
        self.new_k, self.new_v = dev_t(w.step_k[0]), dev_t(w.step_v[0])
        self.slots = dev_t(w.step_slots[0])
        self.ctx_h = w.ctx_at(0)
        self.tables = dev_t(w.tables_at(0))
        self.ctx = dev_t(self.ctx_h)
        self.max_ctx = int(self.ctx_h.max())
        self.out = torch.empty_like(self.q)
        part = (pa.pa_decode_auto_partition(c.num_seqs, c.num_q_heads, c.num_kv_heads,
                                            c.head_dim, c.block_size, self.max_ctx,
                                            pa.dtype_code(self.q))
                if part_req == -1 else part_req)
        if part == pa.PA_PARTITION_BALANCED and algo_name == "vector" and c.dtype == "bf16" \
                and c.head_dim < 32:
            part = 512
        self.part = part
        self.ws = pa.workspace_for(self.q, self.k_cache, self.max_ctx, part)
        torch.cuda.synchronize()

    def decode(self, stream, evs=None):
        """The decode phase: phase 1 (evs[0] after it) and the merge."""
        pa, c = self.pa, self.c
        if self.part == 0:
            pa.pa_decode(self.out, self.q, self.k_cache, self.v_cache, self.tables, self.ctx,
                         c.scale, self.max_ctx, 0, None, self.algo, stream=stream)
            if evs is not None:
                evs[0].record(stream)
            return
        pa.pa_decode_partitions(self.out, self.q, self.k_cache, self.v_cache, self.tables,
                                self.ctx, c.scale, self.max_ctx, self.part, self.ws, self.algo,
                                stream=stream)
        if evs is not None:
            evs[0].record(stream)
        pa.pa_decode_reduce(self.out, self.ctx, c.num_kv_heads, self.max_ctx, self.part,
                            self.ws, stream=stream)

    def step(self, stream, evs=None):
        if evs is not None:
            evs[0].record(stream)
        if self.cow is not None:    # the step's copy-on-write copies, then its writes
            self.pa.pa_copy_blocks(self.k_cache, self.v_cache, self.cow, stream=stream)
        self.pa.pa_reshape_and_cache(self.new_k, self.new_v, self.k_cache, self.v_cache,
                                     self.slots, stream=stream)
        if evs is not None:
            evs[1].record(stream)
        self.decode(stream, None if evs is None else evs[2:3])
        if evs is not None:
            evs[3].record(stream)

    def time(self, steps, warmup):
        """Wall clock over exactly `steps` steps after `warmup`, then per-phase
        HIP-event durations on the launch stream and the decode phase with
        cold caches."""
        torch = self.torch
        stream = torch.cuda.current_stream()
        for _ in range(warmup):
            self.step(stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        for e in evs:
            self.step(stream, e)
        torch.cuda.synchronize()
        t_write = [e[0].elapsed_time(e[1]) for e in evs]
        t_main = [e[1].elapsed_time(e[2]) for e in evs]
        t_reduce = [e[2].elapsed_time(e[3]) for e in evs]
        t_step = [e[0].elapsed_time(e[3]) for e in evs]
        # cold caches: reading a 1 GiB buffer between launches evicts L2 and
        # the MALL (not timed; a read leaves no dirty lines to write back)
        flush = torch.ones(1 << 27, dtype=torch.int64, device=self.q.device)
        cold = []
        for _ in range(min(steps, 20)):
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            self.decode(stream, [e1])
            torch.cuda.synchronize()
            cold.append(e0.elapsed_time(e1))
        del flush
        return {"wall_ms": wall * 1e3, "write": t_write, "main": t_main, "reduce": t_reduce,
                "step": t_step, "cold": cold}

    def tile_list(self):
        """The 16-token (block, KV head) tiles the decode reads, in the order
        of its tile stream (KV head slowest, then sequence or pack, then
        tile); in shared-prefix mode a tile several members of a pack
        reference is listed once.  Index = the tile's position in the pool
        counted in 16-row tiles.  None where the block size is below 16."""
        c, w = self.c, self.w
        if c.block_size < 16:
            return None
        ctx, tab = w.ctx_at(0), w.tables_at(0)
        per_block = c.block_size // 16
        ids = []
        if self.part == -3:
            pack = 8
            while pack > 1 and pack * (c.num_q_heads // c.num_kv_heads) > 32:
                pack //= 2
            for g in range(c.num_kv_heads):
                for k0 in range(0, c.num_seqs, pack):
                    mem = range(k0, min(c.num_seqs, k0 + pack))
                    nt = max((int(ctx[b]) + 15) // 16 for b in mem)
                    for t in range(nt):
                        seen = []
                        for b in mem:
                            if t * 16 < int(ctx[b]):
                                blk = int(tab[b, t * 16 // c.block_size])
                                if blk not in seen:
                                    seen.append(blk)
                        ids += [(blk * c.num_kv_heads + g) * per_block + t % per_block
                                for blk in seen]
        else:
            for g in range(c.num_kv_heads):
                for b in range(c.num_seqs):
                    t = np.arange((int(ctx[b]) + 15) // 16)
                    blk = tab[b, t * 16 // c.block_size].astype(np.int64)
                    ids.append((blk * c.num_kv_heads + g) * per_block + t % per_block)
            ids = np.concatenate(ids) if ids else np.zeros(0, dtype=np.int64)
        return np.asarray(ids, dtype=np.int32)

    def paged_read(self, reps=20):
        """The decode's own tiles read with no arithmetic (calibration kernel
        pa_measure_tile_read): the paged-read ceiling of this workload."""
        torch, pa = self.torch, self.pa
        ids = self.tile_list()
        if ids is None or len(ids) == 0:
            return None
        tiles = self.dev_t(ids)
        sink = torch.empty(pa.MEASURE_SINK_WORDS, dtype=torch.int32, device=self.q.device)
        stream = torch.cuda.current_stream()
        for _ in range(3):
            pa.pa_measure_tile_read(self.k_cache, self.v_cache, tiles, sink, stream=stream)
        ms = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            pa.pa_measure_tile_read(self.k_cache, self.v_cache, tiles, sink, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        t = statistics.median(ms)
        nbytes = int(len(ids)) * 2 * 16 * self.c.head_dim * (2 if self.c.dtype == "bf16" else 4)
        return {"tiles": int(len(ids)), "bytes": nbytes, "ms": round(t, 5),
                "GBs": round(nbytes / (t * 1e-3) / 1e9, 1), "kernel": "tile_read_kernel"}

    def bytes(self):
        c, w, ctx_h = self.c, self.w, self.ctx_h
        es = 2 if c.dtype == "bf16" else 4
        kv_logical = w.kv_logical_bytes(0)
        kv_unique = w.kv_unique_bytes(0)
        qo = 2 * c.num_seqs * c.num_q_heads * c.head_dim * es
        tables = int(((ctx_h + c.block_size - 1) // c.block_size).sum()) * 4 + 4 * c.num_seqs
        return {"kv_logical": kv_logical, "kv_unique": kv_unique,
                "decode_algorithmic": kv_unique + qo + tables}

    def free(self):
        for name in ("k_cache", "v_cache", "q", "out", "ws", "tables", "ctx", "new_k", "new_v",
                     "slots", "cow"):
            setattr(self, name, None)
        self.torch.cuda.empty_cache()


def decode_record(run, t, steps, args):
    """The numbers of one timed decode workload (shared by the headline and
    the extra workloads), with the paged-read ceiling of its own tiles."""
    c = run.c
    by = run.bytes()
    ms_step = t["wall_ms"] / steps
    main_ms = statistics.mean(t["main"])
    red_ms = statistics.mean(t["reduce"])
    alg = by["decode_algorithmic"]
    achieved = alg / (main_ms * 1e-3) / 1e9
    with_merge = alg / ((main_ms + red_ms) * 1e-3) / 1e9
    shared = run.part == -3
    roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "frac_with_merge": round(with_merge / HBM_PEAK_GBS, 4),
            "kernel": decode_kernel_name(c, run.part, run.algo_name),
            "bytes_per_launch": alg,
            "time": "plan + decode kernels (merge in frac_with_merge)" if shared
                    else "decode kernel (merge in frac_with_merge)"}
    traffic = load_traffic(c.name, run.algo_name, run.part)
    pr = run.paged_read()
    if pr is not None:
        # the same tiles read with no arithmetic: how close the decode phase
        # comes to a pure paged read of what it reads
        pr["read_over_decode_kernel"] = round(pr["ms"] / main_ms, 4)
        pr["read_over_decode_phase"] = round(pr["ms"] / (main_ms + red_ms), 4)
        roof["paged_read"] = pr
    roof["traffic"] = traffic
    roof["traffic_source"] = ("rocprofv3 FETCH_SIZE/WRITE_SIZE per launch, committed in "
                              "profiles/traffic.json and taken on kernel sources that hash the "
                              "same as these" if traffic is not None else
                              "none: no counter run on the current kernel sources")
    return {
        "value": round(by["kv_logical"] / (ms_step * 1e-3) / 1e9, 2), "unit": "GB/s",
        "ms_per_step": round(ms_step, 5),
        "config": {"workload": c.name, "description": c.description, "batch": c.num_seqs,
                   "num_q_heads": c.num_q_heads, "num_kv_heads": c.num_kv_heads,
                   "head_dim": c.head_dim, "block_size": c.block_size,
                   "sum_context": int(run.ctx_h.sum()), "max_context": run.max_ctx,
                   "partition_size": run.part, "algo": run.algo_name,
                   "parallelism": "none (1 GPU)"},
        "tokens_per_s": round(c.num_seqs / (ms_step * 1e-3), 1),
        "hbm_peak_frac_step": round(by["kv_logical"] / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                    4),
        "kernels_ms": {"reshape_and_cache": round(statistics.mean(t["write"]), 5),
                       "decode": round(main_ms, 5), "reduce": round(red_ms, 5),
                       "step_events": round(statistics.mean(t["step"]), 5),
                       "decode_cold_l2": round(statistics.median(t["cold"]), 5),
                       "decode_p10": round(float(np.percentile(t["main"], 10)), 5),
                       "decode_p90": round(float(np.percentile(t["main"], 90)), 5)},
        "bytes": by,
        "roofline": roof,
    }


def bench_copy_blocks(run, torch):
    """pa_copy_blocks on up to 4096 pairs, each from a block the tables use
    into one they do not (the decode inputs stay intact)."""
    c, pa = run.c, run.pa
    stream = torch.cuda.current_stream()
    used = np.unique(run.w.tables_at(0)[run.w.tables_at(0) >= 0])
    free_blocks = np.setdiff1d(np.arange(c.num_blocks), used)
    rng = np.random.default_rng(1234)
    n_cp = int(min(4096, len(free_blocks)))
    if n_cp == 0:
        return None
    pairs = np.stack([rng.choice(used, size=n_cp), rng.permutation(free_blocks)[:n_cp]],
                     axis=1).astype(np.int32)
    pairs_d = run.dev_t(pairs)
    for _ in range(3):
        pa.pa_copy_blocks(run.k_cache, run.v_cache, pairs_d, stream=stream)
    cp_ms = []
    for _ in range(20):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        pa.pa_copy_blocks(run.k_cache, run.v_cache, pairs_d, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        cp_ms.append(e0.elapsed_time(e1))
    block_bytes = c.num_kv_heads * c.block_size * c.head_dim * (2 if c.dtype == "bf16" else 4)
    cp_bytes = 4 * n_cp * block_bytes                 # read + write, K and V
    cp_t = statistics.median(cp_ms)
    return {"pairs": n_cp, "ms": round(cp_t, 5), "bytes": cp_bytes,
            "GBs": round(cp_bytes / (cp_t * 1e-3) / 1e9, 1),
            "frac": round(cp_bytes / (cp_t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "kernel": "copy_blocks_kernel"}


def bench_stream_read(torch, pa, dev):
    """A plain streaming read of a 2 GiB buffer (the calibration kernel of
    libpa.so), with the non-temporal hint the decode kernels use and with the
    default policy: the practical read ceiling of this GPU, as context."""
    nbytes = 2 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.empty(pa.MEASURE_SINK_WORDS, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    rec = {"bytes": nbytes, "kernel": "stream_read_kernel", "runs": 20}
    for nt in (True, False):
        for _ in range(3):
            pa.pa_measure_stream_read(buf, sink, nontemporal=nt, stream=stream)
        ms = []
        for _ in range(20):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            pa.pa_measure_stream_read(buf, sink, nontemporal=nt, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        rec["nontemporal_GBs" if nt else "default_GBs"] = round(
            nbytes / (statistics.median(ms) * 1e-3) / 1e9, 1)
    del buf, sink
    torch.cuda.empty_cache()
    return rec


# The other bf16 GQA decode workloads, timed in the same run as the default
# one (each with its own launch configuration and roofline).
EXTRA_WORKLOADS = ["shared_prefix_bf16", "long_split_bf16"]


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"metric": METRIC, "error": "the benchmark measures one GPU: the "
                          "decode path has no multi-GPU mode; run with --gpus 1"}))
        sys.exit(2)

    import torch
    from paged_kv_cache_261_amd import pa
    from paged_kv_cache_261_amd import synthetic as S

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    algo = {"auto": pa.PA_ALGO_AUTO, "vector": pa.PA_ALGO_VECTOR, "mfma": pa.PA_ALGO_MFMA}[args.algo]

    if args.config in S.PREFILL_CONFIGS:
        return bench_prefill(args, torch, pa, S, dev)

    def make(name):
        return BeamLastStep(S.make_beam_workload(name)) if name in S.BEAM_CONFIGS \
            else S.make_workload(name)

    log(f"building workload {args.config}")
    w = make(args.config)
    part_req = w.cfg.partition_size if args.partition is None else args.partition
    run = DecodeRun(w, torch, pa, dev, algo, args.algo, part_req)
    log(f"workload ready: batch {w.cfg.num_seqs}, sum ctx {int(run.ctx_h.sum())}, "
        f"partition {run.part}, algo {args.algo}")
    t = run.time(args.steps, args.warmup)
    log(f"timed {args.steps} steps: {t['wall_ms']:.2f} ms")
    rec = decode_record(run, t, args.steps, args)
    copy_rec = bench_copy_blocks(run, torch)
    run.free()

    result = {"metric": METRIC, "value": rec["value"], "unit": "GB/s", "n_gpus": 1,
              "steps": args.steps, "warmup": args.warmup, "ms_per_step": rec["ms_per_step"],
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
              "dtype": w.cfg.dtype, "data": "synthetic"}
    for key in ("config", "tokens_per_s", "hbm_peak_frac_step", "kernels_ms", "bytes",
                "roofline"):
        result[key] = rec[key]
    result["copy_blocks"] = copy_rec

    default_run = args.config == DEFAULT_CONFIG and args.partition is None and \
        args.algo == "auto" and not args.no_extra_workloads
    if default_run:
        result["workloads"] = {}
        for name in EXTRA_WORKLOADS:
            log(f"building workload {name}")
            wx = make(name)
            rx = DecodeRun(wx, torch, pa, dev, algo, args.algo, wx.cfg.partition_size)
            tx = rx.time(args.steps, args.warmup)
            log(f"timed {args.steps} steps of {name}: {tx['wall_ms']:.2f} ms")
            result["workloads"][name] = decode_record(rx, tx, args.steps, args)
            rx.free()
            del wx
        log("streaming-read ceiling")
        result["stream_read"] = bench_stream_read(torch, pa, dev)
        nt = result["stream_read"]["nontemporal_GBs"]
        result["roofline"]["frac_of_stream_read"] = round(result["roofline"]["achieved"] / nt, 4)
        for r in result["workloads"].values():
            r["roofline"]["frac_of_stream_read"] = round(r["roofline"]["achieved"] / nt, 4)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
