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
with HIP events on the launch stream.  `cpu_baseline` times the CPU oracle
(float64 concatenate-then-attend plus the slot write) on a bounded sample of
the same workload on this host's cores.
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


def cpu_baseline(w, target_seconds):
    """Time the oracle (slot write of the step's tokens + float64
    concatenate-then-attend) on a bounded prefix of the batch, all cores."""
    from oracle import pao
    c = w.cfg
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
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

    # all cores: grow the prefix until one run takes a quarter of the budget
    # (or the batch is whole), then repeat it within the budget; median
    n = min(c.num_seqs, max(1, cores))
    dt = run(n, cores)
    while n < c.num_seqs and dt < target_seconds / 4:
        n = min(c.num_seqs, n * 2)
        dt = run(n, cores)
    times = [dt]
    while sum(times) < target_seconds and len(times) < 40:
        times.append(run(n, cores))
    dt = statistics.median(times)
    # one core, on a prefix about 1/cores as long
    n1 = max(1, n // cores)
    t1 = run(n1, 1)
    return {"value": round(kv_bytes(n) / dt / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"first {n} of {c.num_seqs} sequences of {c.name} "
                      f"(sum ctx {int(ctx[:n].sum())}), one step, median of {len(times)} "
                      f"runs, {dt:.3f} s each",
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
    log(f"building workload {args.config}")
    w = BeamLastStep(S.make_beam_workload(args.config)) if args.config in S.BEAM_CONFIGS \
        else S.make_workload(args.config)
    c = w.cfg
    tdt = torch.bfloat16 if c.dtype == "bf16" else torch.float32

    def dev_t(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    shape = (c.num_blocks, c.num_kv_heads, c.block_size, c.head_dim)
    k_cache = torch.zeros(shape, dtype=tdt, device=dev)
    v_cache = torch.zeros(shape, dtype=tdt, device=dev)
    pa.pa_reshape_and_cache(dev_t(w.prefill_k), dev_t(w.prefill_v), k_cache, v_cache,
                            dev_t(w.prefill_slots))
    for st in getattr(w, "earlier_steps", []):   # beam workloads: the steps before the last
        if len(st.cow):
            pa.pa_copy_blocks(k_cache, v_cache, dev_t(st.cow))
        pa.pa_reshape_and_cache(dev_t(st.k), dev_t(st.v), k_cache, v_cache, dev_t(st.slots))
    cow_h = getattr(w, "cow", np.zeros((0, 2), dtype=np.int32))
    cow = dev_t(cow_h) if len(cow_h) else None
    q = dev_t(w.q[0])
    new_k, new_v = dev_t(w.step_k[0]), dev_t(w.step_v[0])
    slots = dev_t(w.step_slots[0])
    ctx_h = w.ctx_at(0)
    tables = dev_t(w.tables_at(0))
    ctx = dev_t(ctx_h)
    max_ctx = int(ctx_h.max())
    out = torch.empty_like(q)
    part_req = c.partition_size if args.partition is None else args.partition
    part = (pa.pa_decode_auto_partition(c.num_seqs, c.num_q_heads, c.num_kv_heads, c.head_dim,
                                        c.block_size, max_ctx, pa.dtype_code(q))
            if part_req == -1 else part_req)
    if part == pa.PA_PARTITION_BALANCED and args.algo == "vector":
        part = 512
    ws = pa.workspace_for(q, k_cache, max_ctx, part)
    torch.cuda.synchronize()
    log(f"workload ready: batch {c.num_seqs}, sum ctx {int(ctx_h.sum())}, partition {part}, "
        f"algo {args.algo}")

    stream = torch.cuda.current_stream()

    def step(evs=None):
        if evs is not None:
            evs[0].record(stream)
        if cow is not None:         # the step's copy-on-write copies, then its writes
            pa.pa_copy_blocks(k_cache, v_cache, cow, stream=stream)
        pa.pa_reshape_and_cache(new_k, new_v, k_cache, v_cache, slots, stream=stream)
        if evs is not None:
            evs[1].record(stream)
        if part == 0:
            pa.pa_decode(out, q, k_cache, v_cache, tables, ctx, c.scale, max_ctx, 0, None, algo,
                         stream=stream)
            if evs is not None:
                evs[2].record(stream)
                evs[3].record(stream)
        else:
            pa.pa_decode_partitions(out, q, k_cache, v_cache, tables, ctx, c.scale, max_ctx, part,
                                    ws, algo, stream=stream)
            if evs is not None:
                evs[2].record(stream)
            pa.pa_decode_reduce(out, ctx, c.num_kv_heads, max_ctx, part, ws, stream=stream)
            if evs is not None:
                evs[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # (1) wall clock over exactly K steps
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"timed {args.steps} steps: {wall * 1e3:.2f} ms")

    # (2) per-kernel durations with HIP events on the launch stream
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    t_write = [e[0].elapsed_time(e[1]) for e in evs]
    t_main = [e[1].elapsed_time(e[2]) for e in evs]
    t_reduce = [e[2].elapsed_time(e[3]) for e in evs]
    t_step = [e[0].elapsed_time(e[3]) for e in evs]

    # (4) copy-on-write block copies (pa_copy_blocks): up to 4096 pairs, each
    # from a block the tables use into one they do not (the decode inputs
    # stay intact)
    used = np.unique(w.tables_at(0)[w.tables_at(0) >= 0])
    free_blocks = np.setdiff1d(np.arange(c.num_blocks), used)
    rng = np.random.default_rng(1234)
    n_cp = int(min(4096, len(free_blocks)))
    copy_rec = None
    if n_cp > 0:
        pairs = np.stack([rng.choice(used, size=n_cp), rng.permutation(free_blocks)[:n_cp]],
                         axis=1).astype(np.int32)
        pairs_d = dev_t(pairs)
        for _ in range(3):
            pa.pa_copy_blocks(k_cache, v_cache, pairs_d, stream=stream)
        cp_ms = []
        for _ in range(20):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            pa.pa_copy_blocks(k_cache, v_cache, pairs_d, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            cp_ms.append(e0.elapsed_time(e1))
        block_bytes = c.num_kv_heads * c.block_size * c.head_dim * (2 if c.dtype == "bf16" else 4)
        cp_bytes = 4 * n_cp * block_bytes                 # read + write, K and V
        cp_t = statistics.median(cp_ms)
        copy_rec = {"pairs": n_cp, "ms": round(cp_t, 5), "bytes": cp_bytes,
                    "GBs": round(cp_bytes / (cp_t * 1e-3) / 1e9, 1),
                    "frac": round(cp_bytes / (cp_t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "kernel": "copy_blocks_kernel"}

    es = 2 if c.dtype == "bf16" else 4
    kv_logical = w.kv_logical_bytes(0)
    kv_unique = w.kv_unique_bytes(0)
    qo_bytes = 2 * c.num_seqs * c.num_q_heads * c.head_dim * es
    table_bytes = int(((ctx_h + c.block_size - 1) // c.block_size).sum()) * 4 + 4 * c.num_seqs
    decode_alg = kv_unique + qo_bytes + table_bytes
    ms_step = wall / args.steps * 1e3
    main_ms = statistics.mean(t_main)
    achieved = decode_alg / (main_ms * 1e-3) / 1e9
    algo_name = args.algo
    traffic = load_traffic(args.config, algo_name, part)
    kernel_name = decode_kernel_name(c, part, args.algo)

    # (3) the decode phase with caches cold: reading a 1 GiB buffer between
    # launches evicts L2 and the MALL (not timed; a read leaves no dirty
    # lines to write back during the decode)
    flush = torch.ones(1 << 27, dtype=torch.int64, device=dev)
    cold = []
    for _ in range(min(args.steps, 20)):
        flush.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        if part == 0:
            pa.pa_decode(out, q, k_cache, v_cache, tables, ctx, c.scale, max_ctx, 0, None, algo,
                         stream=stream)
        else:
            pa.pa_decode_partitions(out, q, k_cache, v_cache, tables, ctx, c.scale, max_ctx, part,
                                    ws, algo, stream=stream)
        e1.record(stream)
        if part != 0:
            pa.pa_decode_reduce(out, ctx, c.num_kv_heads, max_ctx, part, ws, stream=stream)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    del flush

    result = {
        "metric": METRIC,
        "value": round(kv_logical / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c.dtype,
        "data": "synthetic",
        "config": {"workload": c.name, "description": c.description, "batch": c.num_seqs,
                   "num_q_heads": c.num_q_heads, "num_kv_heads": c.num_kv_heads,
                   "head_dim": c.head_dim, "block_size": c.block_size,
                   "sum_context": int(ctx_h.sum()), "max_context": max_ctx,
                   "partition_size": part, "algo": algo_name, "parallelism": "none (1 GPU)"},
        "tokens_per_s": round(c.num_seqs / (ms_step * 1e-3), 1),
        "hbm_peak_frac_step": round(kv_logical / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "kernels_ms": {"reshape_and_cache": round(statistics.mean(t_write), 5),
                       "decode": round(main_ms, 5),
                       "reduce": round(statistics.mean(t_reduce), 5),
                       "step_events": round(statistics.mean(t_step), 5),
                       "decode_cold_l2": round(statistics.median(cold), 5),
                       "decode_p10": round(float(np.percentile(t_main, 10)), 5),
                       "decode_p90": round(float(np.percentile(t_main, 90)), 5)},
        "bytes": {"kv_logical": kv_logical, "kv_unique": kv_unique,
                  "decode_algorithmic": decode_alg},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": kernel_name},
        "copy_blocks": copy_rec,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
