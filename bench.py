#!/usr/bin/env python3
"""Benchmark of one packed engine step (append + paged attention) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config {2,3,4,5}] [--gpus 1]

A step is pkv_append of the step's new K/V rows followed by pkv_attention over
the whole batch, on synthetic N(0,1) data already resident in HBM.  The
default workload is the 128-sequence large decode batch (contexts uniform in
[4096, 32768], 64 query / 8 kv heads, head_dim 128, page size 16, bf16): its
9.7 GB of keys and values cannot stay in the 256 MB Infinity Cache, so back to
back steps read HBM.  One JSON line is printed:

  value      decode KV-read GB/s = valid K/V bytes of the step / step time
  roofline   the decode pass (split-key partial + merge kernels) against the
             8 TB/s HBM peak, timed with HIP events on the launch stream
  cpu_baseline  the float64 oracle on the host cores over a bounded sample
  extra      the mixed chunked-prefill step: packed-step tokens/s and the
             prefill kernel's MFMA utilisation against 2.5 PFLOP/s dense bf16;
             a step of 4-token speculative-verify windows against the plain
             decode step over the same contexts
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import paged_kv_attention_03_amd as pkv  # noqa: E402
from paged_kv_attention_03_amd import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_DENSE_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak, published
METRIC = "decode KV-read GB/s (% HBM peak) + packed-step tokens/s; prefill MFMA util"
KERNEL_SOURCES = ["decode.hpp", "pkv_device.hpp"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kv_bytes(st) -> int:
    """Valid K+V bytes a step reads: sum over sequences of (keys - kv_start)
    * 2 (K and V) * Hkv * D * element size."""
    e = 2 if st.dtype == torch.bfloat16 else 4
    return int(sum(st.real_lens) * 2 * st.num_kv_heads * st.head_dim * e)


def prefill_flops(st) -> float:
    """QK^T and PV multiply-adds (2 flops each) over every visible
    (query token, key) pair of the prefill sequences, for all query heads."""
    pairs = 0
    for L, n in zip(st.real_lens, st.q_lens):
        if n >= 2:
            pairs += sum(L - n + i + 1 for i in range(n))
    return 4.0 * st.head_dim * st.num_q_heads * pairs


class Step:
    """Resident device state of one workload: pools, metadata, the step's
    rows, q, out and workspace."""

    def __init__(self, st, gen_device="cuda"):
        self.st = st
        self.kp, self.vp = st.new_pool("cuda", poison=False)
        k, v, s = st.rows("fill", "cuda", gen_device=gen_device)
        if k.shape[0]:
            pkv.pkv_append(k, v, self.kp, self.vp, s)
        del k, v, s
        self.k_new, self.v_new, self.slots = st.rows("step", "cuda", gen_device=gen_device)
        md = st.metadata("cuda")
        self.bt, self.sl, self.qsl, self.ks = (md["block_tables"], md["seq_lens"],
                                               md["query_start_loc"], md["kv_start"])
        self.q = st.make_q("cuda", gen_device=gen_device)
        self.out = torch.empty_like(self.q)
        need = pkv.pkv_attention_workspace_size(st.num_seqs, st.total_q, st.max_seqlen_q,
                                                st.max_seqlen_k, st.num_q_heads,
                                                st.num_kv_heads, st.head_dim, 16, st.dtype)
        self.ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        # the step's two calls, checked once and re-issued each step
        self.append = pkv.prepare_append(self.k_new, self.v_new, self.kp, self.vp, self.slots)
        self.attention = pkv.prepare_attention(
            self.q, self.kp, self.vp, self.bt, self.sl, self.qsl, st.scale,
            max_seqlen_q=st.max_seqlen_q, max_seqlen_k=st.max_seqlen_k, kv_start=self.ks,
            out=self.out, workspace=self.ws)
        torch.cuda.synchronize()

    def append_plain(self):
        pkv.pkv_append(self.k_new, self.v_new, self.kp, self.vp, self.slots)

    def attention_plain(self):
        st = self.st
        pkv.pkv_attention(self.q, self.kp, self.vp, self.bt, self.sl, self.qsl, st.scale,
                          max_seqlen_q=st.max_seqlen_q, max_seqlen_k=st.max_seqlen_k,
                          kv_start=self.ks, out=self.out, workspace=self.ws)


def time_steps(step: Step, steps: int, warmup: int, flush_bytes: int = 0):
    """Whole-step wall time over ``steps`` steps, and the attention call's
    average duration from HIP events recorded on the launch stream."""
    flush = torch.ones(flush_bytes // 4, dtype=torch.float32, device="cuda") if flush_bytes else None
    for _ in range(warmup):
        step.append()
        step.attention()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    if flush is None:
        t0 = time.perf_counter()
        for a, b in ev:
            step.append()
            a.record()
            step.attention()
            b.record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
    else:
        # caches are cleared before every step by reading a buffer larger than
        # L2 + Infinity Cache (a read leaves no dirty lines whose write-back
        # would be charged to the step); the wall time then excludes the
        # clearing by summing per-step event pairs around append + attention
        wall_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(steps)]
        for (a, b), (c, d) in zip(ev, wall_ev):
            sink = flush.sum()  # noqa: F841
            c.record()
            step.append()
            a.record()
            step.attention()
            b.record()
            d.record()
        torch.cuda.synchronize()
        wall = float(np.mean([c.elapsed_time(d) for c, d in wall_ev])) / 1e3
    attn = [a.elapsed_time(b) / 1e3 for a, b in ev]
    return wall, float(np.mean(attn)), float(np.median(attn)), float(np.min(attn))


def device_copy_gbs(nbytes: int = 1 << 31, reps: int = 5) -> float:
    """Bandwidth of a plain device-to-device copy of ``nbytes`` (bytes read +
    bytes written per second): the box's practical HBM ceiling, and the
    known-size kernel that calibrates the HBM byte counters."""
    src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    sec = a.elapsed_time(b) / 1e3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / sec / 1e9


def source_hash() -> str:
    """Hash of the decode kernels' code: their sources with comments and
    whitespace removed, so that a counter record outlives edits of comments
    but not of code."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_attention_03_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(name: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(st, budget_s: float = 10.0):
    """The float64 oracle on the host cores over the first sequences of the
    workload (up to ``budget_s`` seconds for one pass), batched 16 sequences
    per call; the pass is repeated until about ``budget_s`` seconds of oracle
    time (3 to 10 passes) and the median pass is reported.  Only the oracle
    calls are timed (page gather + math)."""
    import oracle
    q_dev = st.make_q("cuda")
    qsl = st.query_start_loc()
    batches, covered, seqs, first = [], 0, 0, 0.0
    while seqs < st.num_seqs and first < budget_s:
        batch = list(range(seqs, min(seqs + 16, st.num_seqs)))
        ks, vs, bts, lens, qs, qls = [], [], [], [], [], []
        page0 = 0
        for s in batch:
            k, v = st.seq_kv(s, "cuda")
            L = k.shape[0]
            npg = (L + 15) // 16
            pad = npg * 16 - L
            shp = (pad, st.num_kv_heads, st.head_dim)
            ks.append(torch.cat([k, torch.zeros(shp, dtype=k.dtype, device=k.device)]).cpu())
            vs.append(torch.cat([v, torch.zeros(shp, dtype=v.dtype, device=v.device)]).cpu())
            bts.append(np.arange(page0, page0 + npg, dtype=np.int32))
            page0 += npg
            lens.append(L)
            qs.append(q_dev[qsl[s]:qsl[s + 1]].cpu())
            qls.append(qsl[s + 1] - qsl[s])
        kpool = torch.cat(ks).view(page0, 16, st.num_kv_heads, st.head_dim).transpose(1, 2).contiguous()
        vpool = torch.cat(vs).view(page0, 16, st.num_kv_heads, st.head_dim).transpose(1, 2).contiguous()
        width = max(len(b) for b in bts)
        bt = np.zeros((len(batch), width), np.int32)
        for i, b in enumerate(bts):
            bt[i, :len(b)] = b
        args = (torch.cat(qs), kpool, vpool, bt, lens,
                np.concatenate([[0], np.cumsum(qls)]).astype(np.int32), st.scale)
        t0 = time.perf_counter()
        oracle.oracle_attention(*args)
        first += time.perf_counter() - t0
        batches.append(args)
        covered += sum(lens)
        seqs += len(batch)
    passes, spent = [first], first
    while len(passes) < 10 and (len(passes) < 3 or spent < budget_s):
        t0 = time.perf_counter()
        for args in batches:
            oracle.oracle_attention(*args)
        passes.append(time.perf_counter() - t0)
        spent += passes[-1]
    del batches
    med = float(np.median(passes))
    e = 2 if st.dtype == torch.bfloat16 else 4
    kvb = covered * 2 * st.num_kv_heads * st.head_dim * e
    return {"value": kvb / med / 1e9, "unit": "GB/s", "cores": oracle.max_threads(),
            "kind": "oracle", "tokens_per_s": seqs / med, "cpu_model": cpu_model(),
            "host_cpus": os.cpu_count(), "small_configs": oracle_small_configs(),
            "sample": f"first {seqs} of {st.num_seqs} sequences ({covered} keys, "
                      f"{kvb / 1e9:.2f} GB of K/V); median of {len(passes)} passes, "
                      f"{spent:.1f} s of oracle time"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_small_configs(reps: int = 3):
    """The oracle on the tiny decode step (config 1) and the 16-sequence
    decode step (config 2), whole step, with all host threads and with one:
    median of ``reps`` calls (page gather + math; inputs prepared before)."""
    import oracle
    res = {}
    for k in (1, 2):
        st = W.config_step(k, poison=False)
        q = st.make_q("cpu")
        kp, vp = st.new_pool("cpu")
        for which in ("fill", "step"):
            kr, vr, sl = st.rows(which, "cpu")
            kp, vp = oracle.oracle_append(kp, vp, kr, vr, sl)
        md = st.metadata("cpu")
        args = (q, kp, vp, md["block_tables"], md["seq_lens"], md["query_start_loc"], st.scale)
        e = 2 if st.dtype == torch.bfloat16 else 4
        kvb = sum(st.real_lens) * 2 * st.num_kv_heads * st.head_dim * e
        rec = {"workload": st.name, "kv_bytes": kvb}
        for name, th in (("all_threads", 0), ("one_thread", 1)):
            ts = []
            for _ in range(reps):
                t0 = time.perf_counter()
                oracle.oracle_attention(*args, threads=th)
                ts.append(time.perf_counter() - t0)
            t = float(np.median(ts))
            rec[name] = {"ms": t * 1e3, "tokens_per_s": st.total_q / t, "kv_gbs": kvb / t / 1e9,
                         "threads": oracle.max_threads() if th == 0 else 1}
        res[st.name] = rec
    return res


def launch_latency(reps: int = 50):
    """The tiny decode step (config 1: 4 sequences, 214 keys, fp32): a step
    whose bytes take nanoseconds, so its time is launch latency.  Per rep:
    the attention call's device time (HIP events around it on the launch
    stream), the host time to enqueue it, and the wall time of append +
    attention + synchronize; through prepared calls (arguments checked once),
    through the plain binding calls, and as one HIP graph replay of the
    captured step.  Median and min over ``reps``."""
    st = W.config_step(1, poison=False)
    step = Step(st, gen_device="cuda")
    stat = lambda xs: {"median": float(np.median(xs)), "min": float(np.min(xs))}
    res = {"workload": st.name, "reps": reps, "unit": "us"}
    for form, append, attention in (("prepared", step.append, step.attention),
                                    ("plain", step.append_plain, step.attention_plain)):
        for _ in range(10):
            append()
            attention()
        torch.cuda.synchronize()
        dev, host, wall = [], [], []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            append()
            a.record()
            t1 = time.perf_counter()
            attention()
            t2 = time.perf_counter()
            b.record()
            torch.cuda.synchronize()
            t3 = time.perf_counter()
            dev.append(a.elapsed_time(b) * 1e3)
            host.append((t2 - t1) * 1e6)
            wall.append((t3 - t0) * 1e6)
        res[form] = {"attention_device_us": stat(dev), "attention_enqueue_host_us": stat(host),
                     "step_wall_us": stat(wall)}
    # The same step captured once in a HIP graph and replayed, as a serving loop
    # that captures its decode step runs it (plain calls: a prepared call holds
    # the stream it was prepared on, not the capturing one).
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step.append_plain()
        step.attention_plain()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step.append_plain()
        step.attention_plain()
    for _ in range(10):
        graph.replay()
    torch.cuda.synchronize()
    dev, wall = [], []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        a.record()
        graph.replay()
        b.record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        dev.append(a.elapsed_time(b) * 1e3)
        wall.append((t1 - t0) * 1e6)
    res["graph"] = {"step_device_us": stat(dev), "step_wall_us": stat(wall)}
    del graph, step
    torch.cuda.empty_cache()
    best = min(("prepared", "graph"), key=lambda f: res[f]["step_wall_us"]["median"])
    res["launch_form"] = best
    res["step_wall_us"] = res[best]["step_wall_us"]
    res["note"] = ("device: HIP events around the attention call (decode kernel, and the "
                   "merge kernel when a segment is cut; graph: around the replayed append + "
                   "attention); host: the enqueue of that call (prepared: the C call alone; "
                   "plain: the binding's checks and conversions too); wall: append + "
                   "attention + synchronize (graph: one replay + synchronize); step_wall_us "
                   "is the faster of the prepared and graph forms")
    return res


def with_mixed_step(mode, fn):
    """Runs fn with the library's mixed-step launch set to ``mode`` (fused: one
    launch for decode waves and prefill tiles; split: separate launches)."""
    old = os.environ.get("PKV_MIXED_STEP")
    os.environ["PKV_MIXED_STEP"] = mode
    try:
        return fn()
    finally:
        if old is None:
            os.environ.pop("PKV_MIXED_STEP", None)
        else:
            os.environ["PKV_MIXED_STEP"] = old


def extra_prefill(steps: int, warmup: int):
    """Mixed chunked-prefill workload (16 sequences: two 512-token chunks at
    offsets 4608 and 4601 plus 14 decodes): packed-step tokens/s with the
    library's default launch, the same step with one launch (fused) and with
    separate decode and prefill launches (split), and the prefill kernel alone
    (the two chunks as their own step) against the dense bf16 matrix peak."""
    mixed = W.config_step(3, poison=False)
    sm = Step(mixed, gen_device="cuda")
    # The three forms are timed in the order default, fused, split, split,
    # fused, default and each is averaged over its two passes, so that a drift
    # of the clocks over the sequence (the first pass after the large batch
    # runs slower) weighs on all three alike.
    passes = {"default": [], "fused": [], "split": []}
    time_steps(sm, steps, warmup, flush_bytes=1 << 30)  # untimed: settles the clocks
    for mode in ("default", "fused", "split", "split", "fused", "default"):
        timed = lambda: time_steps(sm, steps, warmup, flush_bytes=1 << 30)
        passes[mode].append(timed() if mode == "default" else with_mixed_step(mode, timed))
    mean = lambda mode, i: float(np.mean([r[i] for r in passes[mode]]))
    wall, attn = mean("default", 0), mean("default", 1)
    res = {"workload": mixed.name, "packed_step_tokens_per_s": mixed.total_q / wall,
           "step_ms": wall * 1e3, "attention_ms": attn * 1e3}
    for mode in ("fused", "split"):
        res[f"{mode}_step_ms"] = mean(mode, 0) * 1e3
        res[f"{mode}_attention_ms"] = mean(mode, 1) * 1e3
    log(f"mixed step: attention {attn * 1e3:.4f} ms (default), fused {res['fused_attention_ms']:.4f}"
        f" ms, split {res['split_attention_ms']:.4f} ms")
    del sm
    torch.cuda.empty_cache()
    res.update(prefill_chunks(steps, warmup))
    return res


def prefill_chunks(steps: int, warmup: int):
    """The mixed workload's two 512-token chunks as a step of their own: the
    prefill kernel alone against the dense bf16 matrix peak."""
    mixed = W.config_step(3, poison=False)
    idx = [i for i, n in enumerate(mixed.q_lens) if n > 1]
    pre = W.build_step("mixed-prefill-chunks", [mixed.seq_lens[i] for i in idx],
                       [mixed.q_lens[i] for i in idx], 32, 8, 128, torch.bfloat16, 3000,
                       poison=False)
    sp = Step(pre, gen_device="cuda")
    _, pattn, pmed, _ = time_steps(sp, steps, warmup, flush_bytes=1 << 30)
    fl = prefill_flops(pre)
    res = {"prefill_gflop": fl / 1e9, "prefill_ms": pattn * 1e3,
           "prefill_tflops": fl / pattn / 1e12,
           "prefill_mfma_util": fl / pattn / 1e12 / BF16_DENSE_TFLOPS}
    del sp
    torch.cuda.empty_cache()
    return res


def extra_windows(steps: int, warmup: int):
    """Speculative-verify windows on the 16-sequence decode shape (contexts
    uniform in [1024, 4096], 16 query / 8 kv heads): every sequence verifies a
    4-token window (3 draft tokens) through the decode path, timed against the
    plain one-token decode step over the same contexts; caches cleared before
    every step."""
    lens = np.random.default_rng(2000).integers(1024, 4096, size=16, endpoint=True).tolist()
    res = {"workload": "verify-window-16seq", "window_tokens": 4}
    for name, n in (("window", 4), ("decode", 1)):
        st = W.build_step(f"{name}-16seq", lens, [n] * 16, 16, 8, 128, torch.bfloat16, 2100,
                          poison=False)
        sm = Step(st, gen_device="cuda")
        wall, attn, _, _ = time_steps(sm, steps, warmup, flush_bytes=1 << 30)
        res[f"{name}_step_ms"] = wall * 1e3
        res[f"{name}_attention_ms"] = attn * 1e3
        res[f"{name}_tokens_per_s"] = st.total_q / wall
        res[f"{name}_kv_gbs"] = kv_bytes(st) / wall / 1e9
        del sm
        torch.cuda.empty_cache()
    return res


def extra_pool(steps: int = 2000):
    """Host-side pool manager on the large decode batch's shape: 128 sequences
    of U[4096, 32768] tokens in a pool of 1.25x their pages.  Host time
    (microseconds, one thread) of one step's slots (one slot per sequence) and
    of exporting all 128 block-table rows."""
    lens = np.random.default_rng(5000).integers(4096, 32768, size=128, endpoint=True)
    bs = 16
    width = int((lens.max() + steps + bs - 1) // bs) + 1
    nb = int(1.25 * sum((int(x) + steps + bs - 1) // bs for x in lens))
    pool = pkv.PagePool(nb, bs, 128, width)
    for s_, n in enumerate(lens):
        pool.add_seq(s_)
        pool.append(s_, int(n))
    seqs = list(range(128))
    ones = [1] * 128
    t0 = time.perf_counter()
    for _ in range(steps):
        pool.append_batch(seqs, ones)
    t_app = (time.perf_counter() - t0) / steps
    t0 = time.perf_counter()
    for _ in range(steps // 10):
        pool.block_tables(seqs, width)
    t_bt = (time.perf_counter() - t0) / (steps // 10)
    pool.close()
    return {"workload": "pool-manager-128seq", "append_us_per_step": t_app * 1e6,
            "block_tables_us": t_bt * 1e6, "table_width": width,
            "note": "host time through the Python binding: one pkv_pool_append_batch per "
                    "step (128 slots); one full pkv_pool_block_tables export"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=5, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--mixed-step", choices=["default", "fused", "split"], default="default",
                    help="launch form of steps with prefill chunks (for profiling one form)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the two prefill chunks of the mixed workload (for profiling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.manual_seed(0)
    if args.mixed_step != "default":
        os.environ["PKV_MIXED_STEP"] = args.mixed_step
    if args.prefill_only:
        print(json.dumps({"workload": "mixed-prefill-chunks", **prefill_chunks(args.steps, args.warmup)}),
              flush=True)
        return
    k = args.config
    if k == 1:
        lat = launch_latency(max(args.steps, 20))
        print(json.dumps({"metric": "launch latency of the tiny decode step", "unit": "us",
                          "value": lat["step_wall_us"]["median"], "higher_is_better": False,
                          "n_gpus": 1, "steps": lat["reps"], "warmup": 10, "dtype": "f32",
                          "data": "synthetic N(0,1), seeded",
                          "config": {"workload": lat["workload"], "launch_form": lat["launch_form"]},
                          "detail": lat}), flush=True)
        return
    if k == 4:
        run_main = bench_agent
    else:
        run_main = bench_single
    rec = run_main(k, args)
    print(json.dumps(rec), flush=True)


def bench_single(k, args):
    st = W.config_step(k, poison=False)
    log(f"workload {st.name}: {st.num_seqs} seqs, {sum(st.real_lens)} keys, "
        f"{kv_bytes(st) / 1e9:.3f} GB K/V")
    copy_gbs = device_copy_gbs()
    log(f"device copy: {copy_gbs:.0f} GB/s (read + write)")
    step = Step(st, gen_device="cuda")
    flush = 0 if k == 5 else (1 << 30)   # the large batch outgrows every cache by itself
    wall, attn_mean, attn_med, attn_min = time_steps(step, args.steps, args.warmup, flush)
    kvb = kv_bytes(st)
    gbs = kvb / wall / 1e9
    achieved = kvb / attn_mean / 1e9
    log(f"step {wall * 1e3:.3f} ms, attention mean {attn_mean * 1e3:.3f} ms "
        f"(median {attn_med * 1e3:.3f}, min {attn_min * 1e3:.3f}) -> {achieved:.0f} GB/s")
    rec = {
        "metric": METRIC, "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if st.dtype == torch.bfloat16 else "f32",
        "data": "synthetic N(0,1) K/V/q, seeded; pool pages shuffled",
        "config": {"workload": st.name, "num_seqs": st.num_seqs,
                   "context_keys_total": int(sum(st.real_lens)), "max_seqlen_k": st.max_seqlen_k,
                   "q_heads": st.num_q_heads, "kv_heads": st.num_kv_heads,
                   "head_dim": st.head_dim, "page_size": st.block_size,
                   "tokens_per_step": st.total_q, "kv_bytes_per_step": kvb,
                   "cache_flush_between_steps": bool(flush)},
        "hbm_peak_frac": gbs / HBM_PEAK_GBS,
        "device_copy_gbs": copy_gbs,
        "copy_frac": gbs / copy_gbs,
        "packed_step_tokens_per_s": st.total_q / wall,
        "roofline": {"bound": "hbm", "kernel": "decode pass (decode_kernel + merge_kernel)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(f"decode_{st.name}"),
                     "launch_ms_mean": attn_mean * 1e3, "launch_ms_median": attn_med * 1e3,
                     "algorithmic_bytes_per_launch": kvb},
    }
    if k == 3:
        # the same step with one launch (decode waves and prefill tiles in
        # one grid) and with separate launches
        modes = {}
        for mode in ("fused", "split"):
            mw, ma, amed, amin = with_mixed_step(mode, lambda: time_steps(step, args.steps,
                                                                          args.warmup, flush))
            modes[mode] = {"step_ms": mw * 1e3, "attention_ms_mean": ma * 1e3,
                           "attention_ms_median": amed * 1e3, "attention_ms_min": amin * 1e3}
        rec["single_launch"] = modes
        log(f"mixed step attention: fused {modes['fused']['attention_ms_mean']:.4f} ms, split "
            f"{modes['split']['attention_ms_mean']:.4f} ms")
    del step
    torch.cuda.empty_cache()
    if not args.no_extra and k != 3:
        rec["extra"] = extra_prefill(min(args.steps, 20), args.warmup)
        rec["extra"]["verify_windows"] = extra_windows(min(args.steps, 20), args.warmup)
        rec["extra"]["pool_manager"] = extra_pool()
        rec["extra"]["launch_latency"] = launch_latency()
    if not args.no_extra and k == 3:
        rec["extra"] = {"split_parts": split_parts(min(args.steps, 20), args.warmup)}
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(st)
    return rec


def split_parts(steps: int, warmup: int):
    """The mixed step's decode part and its prefill chunks as two calls: back
    to back on one stream, and at once on two streams (whether running the
    HBM-bound and the MFMA-bound parts concurrently would pay)."""
    mixed = W.config_step(3, poison=False)
    ip = [i for i, n in enumerate(mixed.q_lens) if n > 1]
    idc = [i for i, n in enumerate(mixed.q_lens) if n == 1]
    pre = W.build_step("mixed-prefill-chunks", [mixed.seq_lens[i] for i in ip],
                       [mixed.q_lens[i] for i in ip], 32, 8, 128, torch.bfloat16, 3000, poison=False)
    dec = W.build_step("mixed-decode-part", [mixed.seq_lens[i] for i in idc], [1] * len(idc),
                       32, 8, 128, torch.bfloat16, 3001, poison=False)
    sp, sd = Step(pre, gen_device="cuda"), Step(dec, gen_device="cuda")
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()

    def timed(fn):
        ts = []
        for r in range(steps + warmup):
            flush.sum()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            if r >= warmup:
                ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    def serial():
        sd.attention()
        sp.attention()

    def concurrent():
        cur = torch.cuda.current_stream()
        e = torch.cuda.Event()
        e.record(cur)
        s1.wait_event(e)
        s2.wait_event(e)
        with torch.cuda.stream(s1):
            sd.attention_plain()  # (the plain call launches on the current stream)
        with torch.cuda.stream(s2):
            sp.attention_plain()
        cur.wait_stream(s1)
        cur.wait_stream(s2)

    res = {"decode_part_ms": timed(sd.attention), "prefill_part_ms": timed(sp.attention),
           "back_to_back_ms": timed(serial), "two_streams_ms": timed(concurrent)}
    log(f"split mixed step: decode part {res['decode_part_ms']:.4f} ms, prefill part "
        f"{res['prefill_part_ms']:.4f} ms, back to back {res['back_to_back_ms']:.4f} ms, "
        f"two streams {res['two_streams_ms']:.4f} ms")
    del sp, sd, flush
    torch.cuda.empty_cache()
    return res


def agent_loop(run, share_prefix: bool = True, prefix_pass=None, graphs: bool = False,
               lookahead: int = 1):
    """The agent loop as an engine runs it: each of the 70 steps plans its
    metadata on the host (pool manager: one slot per sequence, copy-on-write
    check, block-table export), uploads it, appends one token per sequence
    and attends.  A first loop warms up (a fresh pool each time, the manager
    being stateful).  With ``graphs`` each step's device work is a replayed
    HIP graph (captured before the timed loop; the planning stays in it);
    ``lookahead`` K plans K steps at a time and uploads them with one copy.
    Returns wall time per step (host planning included), attention time per
    step (HIP events on the launch stream; None with graphs), the logical
    K/V bytes per step and the host planning time per step."""
    from paged_kv_attention_03_amd.engine import AgentLoop, AgentPlanner

    def make():
        planner = AgentPlanner(run, share_prefix=share_prefix)
        return AgentLoop(run, planner, poison=False, gen_device="cuda", prefix_pass=prefix_pass,
                         graphs=graphs, lookahead=lookahead)

    lp = make()
    for i in range(run.steps):
        lp.step(i)
    torch.cuda.synchronize()
    lp.plan.close()
    del lp
    lp = make()
    ev = [None if graphs or lookahead > 1 else
          (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(run.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(run.steps):
        lp.step(i, ev[i])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / run.steps
    attn = None if ev[0] is None else float(np.mean([a.elapsed_time(c) for a, c in ev])) / 1e3
    lp.plan.close()
    del lp
    torch.cuda.empty_cache()
    # host planning alone, on a fresh manager (no device work)
    planner = AgentPlanner(run, share_prefix=share_prefix)
    planner.prefill()
    t0 = time.perf_counter()
    for i in range(run.steps):
        planner.step(i)
    host = (time.perf_counter() - t0) / run.steps
    planner.close()
    logical = float(np.mean([sum(run.seq_lens_at(i)) for i in range(run.steps)])) * \
        2 * run.num_kv_heads * run.head_dim * 2
    return wall, attn, logical, host


def bench_agent(k, args):
    run = W.AgentRun()
    wall, attn, logical, host = agent_loop(run)
    unique = logical - (run.num_seqs - 1) * run.shared_prefix * 2 * run.num_kv_heads * \
        run.head_dim * 2
    # the same loop with the prefix stored once per sequence: what the shared
    # pages save through the caches as it is (the bound on a prefix pass)
    dwall, dattn, _, _ = agent_loop(W.AgentRun(), share_prefix=False)
    # the same loop with each step's device work replayed from a HIP graph,
    # and with the host planning 8 steps per metadata upload
    gwall, _, _, _ = agent_loop(W.AgentRun(), graphs=True)
    awall, _, _, _ = agent_loop(W.AgentRun(), lookahead=8)
    forms = {"step by step": wall, "graph-replayed": gwall, "8 steps per upload": awall}
    best = min(forms, key=forms.get)
    bwall = forms[best]
    log(f"agent step {wall * 1e3:.4f} ms (host planning {host * 1e6:.1f} us), attention "
        f"{attn * 1e3:.4f} ms; graph-replayed step {gwall * 1e3:.4f} ms; 8 steps per upload "
        f"{awall * 1e3:.4f} ms; duplicated prefix: step {dwall * 1e3:.4f} ms, attention "
        f"{dattn * 1e3:.4f} ms")
    # the shared-prefix entry point on the same loop (routed by the library,
    # and with the prefix pass forced), and on a loop whose shared prefix is
    # long (8192 keys) next to short private suffixes
    _, sattn, _, _ = agent_loop(W.AgentRun(), prefix_pass="auto")
    _, fattn, _, _ = agent_loop(W.AgentRun(), prefix_pass="always")
    long_kw = dict(shared_prefix=8192, prompt_lens=[8192 + 256 + 48 * s for s in range(16)])
    lwall, lattn, llog, _ = agent_loop(W.AgentRun(**long_kw))
    lswall, lsattn, _, _ = agent_loop(W.AgentRun(**long_kw), prefix_pass="auto")
    log(f"shared-prefix entry point: agent attention {sattn * 1e3:.4f} ms (auto), "
        f"{fattn * 1e3:.4f} ms (prefix pass forced); 8192-key prefix: plain {lattn * 1e3:.4f} ms, "
        f"shared-prefix (auto) {lsattn * 1e3:.4f} ms")
    return {
        "metric": METRIC, "value": unique / bwall / 1e9, "unit": "GB/s", "n_gpus": 1,
        "steps": run.steps, "warmup": run.steps, "ms_per_step": bwall * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic N(0,1), seeded; 512-token prefix in shared pages; pages from the "
                "host pool manager (shuffled free list)",
        "config": {"workload": run.name, "num_seqs": run.num_seqs, "decode_steps": run.steps,
                   "q_heads": run.num_q_heads, "kv_heads": run.num_kv_heads,
                   "head_dim": run.head_dim, "page_size": 16, "logical_kv_bytes_per_step": logical,
                   "unique_kv_bytes_per_step": unique,
                   "step": "host planning (pool manager) + metadata upload + append + attention",
                   "launch_form": best},
        "packed_step_tokens_per_s": run.num_seqs / bwall,
        "host_planning_us_per_step": host * 1e6,
        "roofline": {"bound": "hbm", "kernel": "decode pass (decode_kernel + merge_kernel)",
                     "achieved": unique / attn / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": unique / attn / 1e9 / HBM_PEAK_GBS, "traffic": None,
                     "launch_ms_mean": attn * 1e3, "algorithmic_bytes_per_launch": unique},
        "extra": {"launch_forms_step_ms": {k: v * 1e3 for k, v in forms.items()},
                  "launch_forms_note": "step by step: each step planned, uploaded and launched "
                                       "through prepared calls; graph-replayed: upload, append "
                                       "and attention of a step in one HIP graph; 8 steps per "
                                       "upload: the host plans 8 steps, uploads their metadata "
                                       "in one copy, then launches each step",
                  "duplicated_prefix": {"step_ms": dwall * 1e3, "attention_ms": dattn * 1e3,
                                        "note": "same steps, prefix stored per sequence"},
                  "shared_prefix_entry_point": {
                      "agent_attention_ms_auto": sattn * 1e3,
                      "agent_attention_ms_prefix_pass_forced": fattn * 1e3,
                      "long_prefix": {
                          "workload": "16 seqs, 8192-key shared prefix + 256..976 own keys, "
                                      "70 decode steps, 40 q / 8 kv heads",
                          "logical_kv_bytes_per_step": llog,
                          "plain_attention_ms": lattn * 1e3, "plain_step_ms": lwall * 1e3,
                          "shared_prefix_attention_ms_auto": lsattn * 1e3,
                          "shared_prefix_step_ms_auto": lswall * 1e3}}},
    }


if __name__ == "__main__":
    main()
