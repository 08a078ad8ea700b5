#!/usr/bin/env python3
"""Throughput of the paged MQA-logits hot path on one MI355X.

One step = the whole decode path over one batch of synthetic input:
schedule (paged_mqa_logits_metadata) -> paged logits (fp8_fp4_paged_mqa_logits)
-> per-row top-k (top_k_per_row). The workload is the varlen speculative-decode
batch: 40 requests with contexts U[100K, 128K] tokens and accepted draft lengths
U{1..6}, flattened into rows that share K reads per request, fp8 K cache with
block_kv 64, H = 64, D = 128, top-k 2048.

Inputs are resident in HBM before the timed region. Steps rotate over
independent copies of the key cache (together larger than the 256 MB last-level
cache), so each step streams its keys from HBM. HIP events on the launch stream
time every kernel inside the timed region; the JSON line reports the whole-step
rate (HIP-graph replays), per-kernel mean / median / min (eager launches), the
logits call against the HBM roofline, the same rows scored without request
grouping (indices = arange(rows), each row reading its keys alone), and the CPU
oracle timed on a bounded sample of this workload and on each other workload,
with the host's core count and CPU model.

  python bench.py [--steps K] [--warmup W] [--all]

--all adds one line per further workload, each timed the same way: uniform
decode, MXFP4 keys, MXFP4 keys with fp4 q, the tiny decode, the 120K decode
with bf16 logits (the top-k reads them directly; the valid-span upcast to fp32 is
timed beside the step), the fused logits + top-k call, the exact
top-k merge over 8 context-parallel ranks, and ragged prefill logits.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import paged_mqa_logits_amd as pml  # noqa: E402
import pml_synth as syn  # noqa: E402

PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_FP4_TFLOPS = 10100.0   # MI355X dense fp4 MFMA (both operands e2m1)
BYTES_PER_TOKEN = {syn.KV_FP8: 132, syn.KV_FP4: 68}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "paged_logits_fp8_varlen120k_traffic.md")


def measured_traffic():
    """HBM bytes per launch of the fp8 decode-logits kernel on this workload, from the
    committed FETCH_SIZE + WRITE_SIZE summary; None when the kernel sources have changed
    since the counters were taken (or there is no summary)."""
    import profsum
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    for ln in text.splitlines():
        f = ln.strip("` ").split()
        if len(f) == 4 and f[0] == "traffic_bytes_per_launch" and f[2] == "digest":
            return int(f[1]) if f[3] == profsum.source_digest() else None
    return None


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=3, help="key-cache copies rotated over the steps")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-grouping", action="store_true",
                    help="skip the run without request grouping (profiles of the headline step alone)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches instead of HIP-graph replays of the step")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="after timing, run one device-to-device copy of BYTES bytes (a known-size "
                         "reference for the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--all", action="store_true",
                    help="also time the other workloads (one JSON line each on stderr)")
    ap.add_argument("--workload", choices=sorted(OTHERS), default=None,
                    help="time only this other workload (its JSON line on stdout; for profiling one "
                         "workload at a time)")
    return ap.parse_args()


class PagedBench:
    """Device copies of one paged case and the three calls of one step. With bf16,
    the logits are written as bf16 and the top-k reads them as they are."""

    def __init__(self, case: syn.PagedCase, copies: int, num_cus: int | None = None, bf16: bool = False,
                 fused: bool = False):
        d = torch.device("cuda:0")
        self.case = case
        self.q = case.q.to(d)
        self.q_scale = None if case.q_scale is None else case.q_scale.to(d)
        self.w = case.weights.to(d)
        self.lens = case.context_lens.to(d)
        self.bt = case.block_table.to(d)
        self.indices = None if case.indices is None else case.indices.to(d)
        self.kv = [case.kv_cache.to(d) for _ in range(max(1, copies))]
        self.num_cus = num_cus or pml.default_num_workers()
        self.sched = torch.empty(pml.schedule_rows(self.num_cus), 2, dtype=torch.int32, device=d)
        self.ws = torch.empty(pml.logits_workspace_size(case.rows, self.num_cus), dtype=torch.uint8, device=d)
        self.logits = torch.empty(case.rows, pml.logits_ld(case.max_ctx), dtype=torch.float32, device=d)
        self.bf16 = bf16
        self.fused = fused
        self.nev = 3 if fused else 4
        if fused:
            need = pml.fused_topk_workspace_size(case.rows, case.max_ctx, case.block_kv, case.topk, self.num_cus)
            self.ws = torch.empty(need, dtype=torch.uint8, device=d)
        if bf16:
            assert case.next_n == 1
            ld = (case.max_ctx + 7) // 8 * 8
            self.logits_bf16 = torch.empty(case.rows, ld, dtype=torch.bfloat16, device=d)
        self.topk = torch.empty(case.rows, case.topk, dtype=torch.int32, device=d)
        self.req_tokens = int(sum(case.req_ctx))
        self.pairs = syn.scored_pairs(case)

    def step(self, i: int, ev=None):
        c = self.case
        if ev is not None:
            ev[0].record()
        pml.paged_mqa_logits_metadata(self.lens, c.block_kv, self.num_cus, indices=self.indices,
                                      next_n=c.next_n, out=self.sched)
        if ev is not None:
            ev[1].record()
        if self.fused:
            pml.fp8_fp4_paged_mqa_logits_topk(self.q, self.kv[i % len(self.kv)], self.w, self.lens, self.bt,
                                              self.sched, c.max_ctx, c.topk, self.indices, kv_format=c.kv_format,
                                              block_kv=c.block_kv, next_n=c.next_n, logits=self.logits,
                                              out=self.topk, workspace=self.ws)
            if ev is not None:
                ev[2].record()
            return
        pml.fp8_fp4_paged_mqa_logits(self.q, self.kv[i % len(self.kv)], self.w, self.lens, self.bt, self.sched,
                                     c.max_ctx, self.indices, kv_format=c.kv_format, block_kv=c.block_kv,
                                     next_n=c.next_n, logits=self.logits_bf16 if self.bf16 else self.logits,
                                     q_scale=self.q_scale, workspace=self.ws)
        if ev is not None:
            ev[2].record()
        pml.top_k_per_row(self.logits_bf16 if self.bf16 else self.logits, self.lens, c.topk, next_n=c.next_n,
                          max_width=c.max_ctx, out=self.topk)
        if ev is not None:
            ev[self.nev - 1].record()


class RaggedBench:
    def __init__(self, case: syn.RaggedCase):
        d = torch.device("cuda:0")
        self.case = case
        self.q, self.k, self.ksc = case.q.to(d), case.k.to(d), case.k_scale.to(d)
        self.w, self.ks, self.ke = case.weights.to(d), case.ks.to(d), case.ke.to(d)
        self.logits = torch.empty(case.M, pml.logits_ld(case.N), dtype=torch.float32, device=d)
        self.topk = torch.empty(case.M, case.topk, dtype=torch.int32, device=d)
        self.pairs = int((case.ke - case.ks).clamp_min(0).sum())
        self.max_width = int((case.ke - case.ks).clamp_min(0).max())

    def step(self, i: int, ev=None):
        c = self.case
        if ev is not None:
            ev[0].record()
            ev[1].record()
        pml.mqa_logits(self.q, self.k, self.ksc, self.w, self.ks, self.ke, logits=self.logits)
        if ev is not None:
            ev[2].record()
        pml.top_k_per_row(self.logits, self.ke, c.topk, ks=self.ks, max_width=self.max_width, out=self.topk)
        if ev is not None:
            ev[3].record()


class DcpBench:
    """One rank's share of a decode step split over `world` context-parallel ranks,
    after its logits: local top_k_per_row on its 1/world of the columns, the pack
    into (score, global id) pairs, and the merge of all ranks' gathered pairs
    (the all-gather itself is not part of one GPU's work)."""

    def __init__(self, case: syn.PagedCase, world: int = 8, interleave: int = 1):
        d = torch.device("cuda:0")
        self.world, self.interleave, self.k = world, interleave, case.topk
        self.rows = case.rows
        T = case.max_ctx
        self.local_w = -(-T // world)
        ld = (self.local_w + 3) // 4 * 4
        vis = syn.vis_per_row(case)
        g = torch.Generator(device=d)
        g.manual_seed(77)
        self.local = [torch.randn(self.rows, ld, device=d, generator=g) for _ in range(world)]
        # rank r holds the tokens t < vis with (t // interleave) % world == r
        ke = []
        for r in range(world):
            full_runs = vis // (world * interleave)
            rem = vis - full_runs * world * interleave
            n_r = full_runs * interleave + np.clip(rem - r * interleave, 0, interleave)
            ke.append(torch.from_numpy(n_r.astype(np.int32)).to(d))
        self.ke = ke
        self.loc = [pml.top_k_per_row(self.local[r], ke[r], self.k, max_width=self.local_w) for r in range(world)]
        self.gathered = torch.stack([pml.pack_dcp_topk_candidates(self.local[r], self.loc[r], r, world, interleave)
                                     for r in range(world)])
        self.out = torch.empty(self.rows, self.k, dtype=torch.int32, device=d)
        torch.cuda.synchronize()

    def step(self, i: int, ev=None):
        if ev:
            ev[0].record()
        pml.top_k_per_row(self.local[0], self.ke[0], self.k, max_width=self.local_w, out=self.loc[0])
        if ev:
            ev[1].record()
        pml.pack_dcp_topk_candidates(self.local[0], self.loc[0], 0, self.world, self.interleave,
                                     out=self.gathered[0])
        if ev:
            ev[2].record()
        pml.stable_topk_from_gathered_candidates(self.gathered, self.k, out=self.out)
        if ev:
            ev[3].record()


def run_timed(b, steps: int, warmup: int):
    """Warm up, then time exactly `steps` steps; per-kernel times from events."""
    for i in range(warmup):
        b.step(i)
    torch.cuda.synchronize()
    nev = getattr(b, "nev", 4)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        b.step(warmup + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(nev - 1)] for e in evs])
    return wall, per  # per: [steps, nev - 1] ms of (schedule, logits, [upcast,] top-k)


def capture_steps(b) -> list:
    """One HIP graph per key-cache copy holding the whole step (schedule, logits,
    top-k). The calls allocate nothing and never synchronise, so they capture."""
    graphs = []
    for i in range(len(b.kv)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            b.step(i)
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def run_graphs(graphs: list, steps: int, warmup: int) -> float:
    """Warm up, then time exactly `steps` replays (rotating over the copies); wall seconds."""
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        graphs[(warmup + i) % len(graphs)].replay()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def _host() -> dict:
    """Cores this process may run on, and the host CPU model."""
    model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": len(os.sched_getaffinity(0)), "cpu_model": model}


def cpu_baseline(case: syn.PagedCase, target_s: float) -> dict:
    """The oracle (as it stands) on a bounded sample of rows of the same workload."""
    import oracle
    vis = oracle.visible_lengths(case)
    rng = np.random.default_rng(0)
    order = rng.permutation(case.rows)
    # calibrate on one row, then take rows until the estimate reaches target_s
    t0 = time.perf_counter()
    oracle.paged_logits(case, rows=order[:1])
    rate = max(1.0, vis[order[0]]) / max(1e-6, time.perf_counter() - t0)
    n, acc = 0, 0.0
    while n < case.rows and acc < target_s * rate:
        acc += vis[order[n]]
        n += 1
    rows = np.sort(order[:max(1, n)])
    t0 = time.perf_counter()
    sc = oracle.paged_logits(case, rows=rows)
    oracle.topk(sc, vis[rows], case.topk)
    dt = time.perf_counter() - t0
    pairs = int(vis[rows].sum())
    return {"value": round(pairs / dt / 1e3, 3), "unit": "K tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{len(rows)} of {case.rows} rows ({pairs} scored pairs) of the same workload, "
                      f"fp64 logits + top-k, {dt:.1f} s"}


def _oracle_paged(case, rows=None) -> tuple[float, int]:
    """Seconds for the oracle's logits + top-k of `rows` (all by default), and the pairs scored."""
    import oracle
    vis = oracle.visible_lengths(case)
    rows = np.arange(case.rows) if rows is None else np.asarray(rows)
    t0 = time.perf_counter()
    sc = oracle.paged_logits(case, rows=rows)
    oracle.topk(sc, vis[rows], case.topk)
    return time.perf_counter() - t0, int(vis[rows].sum())


def cpu_baseline_configs() -> dict:
    """The oracle on each of the other workloads (whole, or a stated sample of it):
    the tiny decode as the median of 5 runs plus one run on a single thread, the
    uniform decode whole, 8 of the 64 MXFP4 requests (generated with the same
    distributions), and 1024 of the 32768 ragged prefill rows."""
    import oracle
    out = {}
    nthr = oracle.num_threads()
    c1 = syn.config_tiny_decode()
    ts = []
    for _ in range(5):
        dt, pairs = _oracle_paged(c1)
        ts.append(dt)
    oracle.set_num_threads(1)
    try:
        dt1, _ = _oracle_paged(c1)
    finally:
        oracle.set_num_threads(nthr)
    med = float(np.median(ts))
    out["tiny_decode"] = {"value": round(pairs / med / 1e3, 3), "unit": "K tokens/s", "cores": nthr,
                          "seconds_median_of_5": round(med, 4), "seconds_1_thread": round(dt1, 4),
                          "value_1_thread": round(pairs / dt1 / 1e3, 3), "sample": f"all {c1.rows} rows"}
    c2 = syn.config_uniform_decode()
    dt, pairs = _oracle_paged(c2)
    out["uniform_decode_32k"] = {"value": round(pairs / dt / 1e3, 3), "unit": "K tokens/s", "cores": nthr,
                                 "seconds": round(dt, 3), "sample": f"all {c2.rows} rows"}
    c4 = syn.config_varlen_fp4(R=8)
    dt, pairs = _oracle_paged(c4)
    out["varlen_mxfp4_64k"] = {"value": round(pairs / dt / 1e3, 3), "unit": "K tokens/s", "cores": nthr,
                               "seconds": round(dt, 3),
                               "sample": f"8 of 64 requests ({c4.rows} rows) drawn from the same distributions"}
    c5 = syn.config_ragged_prefill()
    rows = np.sort(np.random.default_rng(0).choice(c5.M, 1024, replace=False))
    ks, ke = c5.ks.numpy(), c5.ke.numpy()
    t0 = time.perf_counter()
    sc = oracle.ragged_logits(c5, rows=rows)
    oracle.topk(sc, ke[rows], c5.topk, ks=ks[rows])
    dt = time.perf_counter() - t0
    pairs = int(np.maximum(ke[rows] - ks[rows], 0).sum())
    out["ragged_prefill_4x8192"] = {"value": round(pairs / dt / 1e3, 3), "unit": "K tokens/s", "cores": nthr,
                                    "seconds": round(dt, 3), "sample": f"1024 of {c5.M} rows"}
    return out


def grouping_comparison(case: syn.PagedCase, steps: int, warmup: int, copies: int) -> dict:
    """The same rows scored with and without the request-id grouping: with
    indices = arange(rows) every row is its own piece and reads its keys alone.
    Schedule + logits only, eager launches with HIP events."""
    out = {}
    for name, idx in (("grouped", case.indices), ("arange", torch.arange(case.rows, dtype=torch.int32))):
        c = syn.PagedCase(**{**case.__dict__, "indices": idx})
        b = PagedBench(c, copies)
        _, per = run_timed(b, steps, warmup)
        t = per[:, 1]
        # keys read: each request's tokens once when grouped, each row's own when not
        tokens = int(syn.vis_per_row(c).sum()) if name == "arange" else b.req_tokens
        kbytes = tokens * BYTES_PER_TOKEN[c.kv_format]
        out[name] = {"ms_logits_mean": round(float(t.mean()), 4), "ms_logits_median": round(float(np.median(t)), 4),
                     "ms_logits_min": round(float(t.min()), 4), "key_bytes_read": kbytes,
                     "hbm_GBs": round(kbytes / (float(t.mean()) * 1e-3) / 1e9, 1)}
        del b
    out["speedup_of_grouping"] = round(out["arange"]["ms_logits_mean"] / out["grouped"]["ms_logits_mean"], 3)
    return out


def stats(x: np.ndarray) -> dict:
    return {"mean": round(float(x.mean()), 4), "median": round(float(np.median(x)), 4), "min": round(float(x.min()), 4)}


def describe(case: syn.PagedCase) -> dict:
    return {"rows": case.rows, "requests": len(case.req_ctx), "req_tokens": int(sum(case.req_ctx)),
            "scored_pairs": syn.scored_pairs(case), "max_ctx": case.max_ctx, "block_kv": case.block_kv,
            "kv": "fp8" if case.kv_format == syn.KV_FP8 else "mxfp4", "heads": case.H, "head_dim": case.D,
            "topk": case.topk}


def paged_summary(name: str, b: PagedBench, wall: float, per: np.ndarray, steps: int) -> dict:
    c = b.case
    t_log = float(per[:, 1].mean()) * 1e-3
    kbytes = b.req_tokens * BYTES_PER_TOKEN[c.kv_format]
    return {"workload": name, "ms_per_step": wall / steps * 1e3,
            "ms_schedule": float(per[:, 0].mean()), "ms_logits": t_log * 1e3, "ms_topk": float(per[:, 2].mean()),
            "scored_Ktok_s": b.pairs / (wall / steps) / 1e3,
            "logits_hbm_GBs": kbytes / t_log / 1e9, "logits_hbm_frac": kbytes / t_log / 1e9 / PEAK_HBM_GBS,
            "logits_mfma_frac": b.pairs * 2 * c.H * c.D / t_log / 1e12 /
                                (PEAK_FP4_TFLOPS if c.q_scale is not None else PEAK_FP8_TFLOPS),
            "logits_out_bytes": c.rows * c.max_ctx * 4, **describe(c)}


def _paged_other(mk, copies_mult: int = 2):
    def run(args):
        ob = PagedBench(mk(), args.copies * copies_mult)
        w2, p2 = run_timed(ob, args.steps, args.warmup)
        if not args.no_graph:
            w2 = run_graphs(capture_steps(ob), args.steps, args.warmup)
        return ob, w2, p2
    return run


def run_uniform(args):
    ob, w2, p2 = _paged_other(syn.config_uniform_decode)(args)
    return paged_summary("uniform_decode_fp8_32k", ob, w2, p2, args.steps)


def run_mxfp4(args):
    ob, w2, p2 = _paged_other(syn.config_varlen_fp4)(args)
    return paged_summary("varlen_spec_decode_mxfp4_64k", ob, w2, p2, args.steps)


def run_mxfp4_fp4q(args):
    ob, w2, p2 = _paged_other(lambda: syn.config_varlen_fp4(q_fp4=True))(args)
    return paged_summary("varlen_spec_decode_mxfp4_64k_fp4q", ob, w2, p2, args.steps)


def run_tiny(args):
    ob, w2, p2 = _paged_other(syn.config_tiny_decode, 0)(args)
    return paged_summary("tiny_decode_fp8", ob, w2, p2, args.steps)


def run_bf16(args):
    ob = PagedBench(syn.config_varlen_fp8(), args.copies, bf16=True)
    w2, p2 = run_timed(ob, args.steps, args.warmup)
    if not args.no_graph:
        w2 = run_graphs(capture_steps(ob), args.steps, args.warmup)
    c = ob.case
    t_log = float(p2[:, 1].mean()) * 1e-3
    kbytes = ob.req_tokens * BYTES_PER_TOKEN[c.kv_format]
    # The valid-span upcast of the same bf16 logits, outside the step (the
    # step's top-k reads bf16 directly): 2 bytes read and 4 written per column
    # below each row's end.
    lb = ob.logits_bf16
    up = torch.empty_strided(lb.shape, (lb.stride(0), 1), dtype=torch.float32, device=lb.device)
    for _ in range(max(args.warmup, 1)):
        pml.as_fp32_logits(lb, ob.lens, out=up, cols=c.max_ctx)
    uev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1 in uev:
        e0.record()
        pml.as_fp32_logits(lb, ob.lens, out=up, cols=c.max_ctx)
        e1.record()
    torch.cuda.synchronize()
    t_up = float(np.mean([e0.elapsed_time(e1) for e0, e1 in uev])) * 1e-3
    ubytes = 6 * int(ob.lens.clamp(0, c.max_ctx).sum())
    return {"workload": "varlen_spec_decode_fp8_120k_bf16_logits", "ms_per_step": w2 / args.steps * 1e3,
            "ms_schedule": float(p2[:, 0].mean()), "ms_logits": t_log * 1e3,
            "ms_topk": float(p2[:, 2].mean()),
            "scored_Ktok_s": ob.pairs / (w2 / args.steps) / 1e3,
            "logits_hbm_GBs": kbytes / t_log / 1e9, "logits_hbm_frac": kbytes / t_log / 1e9 / PEAK_HBM_GBS,
            "logits_out_bytes": c.rows * c.max_ctx * 2,
            "ms_upcast": t_up * 1e3, "upcast_bytes": ubytes, "upcast_GBs": ubytes / t_up / 1e9,
            "upcast_hbm_frac": ubytes / t_up / 1e9 / PEAK_HBM_GBS}


def run_fused(args):
    ob = PagedBench(syn.config_varlen_fp8(), args.copies, fused=True)
    w2, p2 = run_timed(ob, args.steps, args.warmup)
    if not args.no_graph:
        w2 = run_graphs(capture_steps(ob), args.steps, args.warmup)
    return {"workload": "varlen_spec_decode_fp8_120k_fused_logits_topk",
            "ms_per_step": w2 / args.steps * 1e3, "ms_schedule": float(p2[:, 0].mean()),
            "ms_fused_logits_topk": float(p2[:, 1].mean()),
            "scored_Ktok_s": ob.pairs / (w2 / args.steps) / 1e3}


def run_dcp(args):
    db = DcpBench(syn.config_varlen_fp8())
    w2, p2 = run_timed(db, args.steps, args.warmup)
    t_m = float(p2[:, 2].mean()) * 1e-3
    mbytes = db.world * db.rows * db.k * 8 + db.rows * db.k * 4
    return {"workload": "dcp_topk_merge_8ranks_varlen120k", "rows": db.rows, "k": db.k,
            "world": db.world, "local_width": db.local_w,
            "ms_local_topk": float(p2[:, 0].mean()), "ms_pack": float(p2[:, 1].mean()),
            "ms_merge": t_m * 1e3, "merge_bytes": mbytes,
            "merge_GBs": mbytes / t_m / 1e9, "merge_hbm_frac": mbytes / t_m / 1e9 / PEAK_HBM_GBS}


def run_ragged(args):
    rb = RaggedBench(syn.config_ragged_prefill())
    n = max(3, args.steps // 4)
    w2, p2 = run_timed(rb, n, 2)
    t_log = float(p2[:, 1].mean()) * 1e-3
    return {"workload": "ragged_prefill_4x8192", "ms_per_step": w2 / n * 1e3,
            "ms_logits": t_log * 1e3, "ms_topk": float(p2[:, 2].mean()),
            "ms_logits_median": float(np.median(p2[:, 1])), "ms_logits_min": float(p2[:, 1].min()),
            "scored_Ktok_s": rb.pairs / (w2 / n) / 1e3,
            "logits_mfma_frac": rb.pairs * 2 * 64 * 128 / t_log / 1e12 / PEAK_FP8_TFLOPS,
            "logits_write_GBs": rb.case.M * rb.case.N * 4 / t_log / 1e9}


def calibration_copy(nbytes: int) -> None:
    """One device-to-device copy of nbytes (a known-size reference for the byte counters)."""
    if nbytes <= 0:
        return
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[bench] calibration copy of {nbytes} bytes done", file=sys.stderr, flush=True)
    del src, dst


def copy_bandwidth(nbytes: int = 1 << 30, reps: int = 10) -> dict:
    """The achievable HBM rate on this machine: a device-to-device copy of nbytes
    (larger than the 256 MB MALL), bytes read plus written over the median time."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record()
        dst.copy_(src)
        e1.record()
    torch.cuda.synchronize()
    ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))
    del src, dst
    return {"copy_GBs": round(2 * nbytes / ms / 1e6, 1), "copy_bytes": nbytes, "ms_median": round(ms, 4),
            "note": "device-to-device copy, read + write bytes over the median of %d events" % reps}


OTHERS = {"uniform_decode_fp8_32k": run_uniform, "varlen_spec_decode_mxfp4_64k": run_mxfp4,
          "varlen_spec_decode_mxfp4_64k_fp4q": run_mxfp4_fp4q, "tiny_decode_fp8": run_tiny,
          "varlen_spec_decode_fp8_120k_bf16": run_bf16, "varlen_spec_decode_fp8_120k_fused": run_fused,
          "dcp_merge_8ranks": run_dcp, "ragged_prefill_4x8192": run_ragged}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    pml.lib()  # fail loudly before generating data if the library is missing
    if args.workload:
        print(f"[bench] {args.workload}", file=sys.stderr, flush=True)
        res = OTHERS[args.workload](args)
        calibration_copy(args.copy_calibration)
        print(json.dumps(res), flush=True)
        return

    print("[bench] generating the varlen speculative-decode workload", file=sys.stderr, flush=True)
    case = syn.config_varlen_fp8()
    b = PagedBench(case, args.copies)
    print(f"[bench] {case.rows} rows, {len(case.req_ctx)} requests, {b.pairs} scored pairs; timing",
          file=sys.stderr, flush=True)
    # per-kernel times: eager launches bracketed by HIP events on the launch stream
    wall, per = run_timed(b, args.steps, args.warmup)
    timing = "eager launches"
    if not args.no_graph:
        # whole-step throughput: the same steps replayed as HIP graphs (no launch gaps)
        wall = run_graphs(capture_steps(b), args.steps, args.warmup)
        timing = "HIP-graph replay of the step; per-kernel times from eager launches with HIP events"
    s = paged_summary("varlen_spec_decode_fp8_120k", b, wall, per, args.steps)

    line = {
        "metric": "scored K tokens/s + achieved HBM GB/s (paged MQA logits + top-k), 1xMI355X",
        "value": round(s["scored_Ktok_s"], 1),
        "unit": "K tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(s["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "timing": timing,
        "config": {"workload": "varlen speculative decode: 40 requests, ctx U[100K,128K], accepted lengths "
                               "U{1..6} flattened to rows, fp8 K cache block_kv 64, H 64, D 128, top-k 2048",
                   **describe(case), "parallelism": "single GPU", "num_workers": b.num_cus,
                   "kv_copies_rotated": len(b.kv)},
        "breakdown_ms": {"schedule": round(s["ms_schedule"], 4), "logits": round(s["ms_logits"], 4),
                         "topk": round(s["ms_topk"], 4)},
        "per_step_ms": {"schedule": stats(per[:, 0]), "logits": stats(per[:, 1]), "topk": stats(per[:, 2]),
                        "step_eager": stats(per.sum(axis=1))},
        "logits_mfma_frac": round(s["logits_mfma_frac"], 4),
        "roofline": {"bound": "hbm", "achieved": round(s["logits_hbm_GBs"], 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(s["logits_hbm_frac"], 4), "traffic": measured_traffic(),
                     "kernel": "fp8_fp4_paged_mqa_logits (u-piece prep + paged_logits_kernel<fp8, block_kv 64>), "
                               "HIP events around the call",
                     "bytes_per_launch": b.req_tokens * BYTES_PER_TOKEN[case.kv_format]},
    }
    calibration_copy(args.copy_calibration)
    del b
    torch.cuda.empty_cache()
    ach = copy_bandwidth()
    line["roofline"]["achievable"] = ach
    line["roofline"]["frac_of_achievable"] = round(line["roofline"]["achieved"] / ach["copy_GBs"], 4)
    if not args.no_grouping:
        print("[bench] the same rows without request grouping (indices = arange)", file=sys.stderr, flush=True)
        line["varlen_grouping"] = grouping_comparison(case, args.steps, args.warmup, args.copies)
        torch.cuda.empty_cache()
        # the ungrouped call reads 3.4x the bytes with the same kernel: its rate shows what this
        # read pattern reaches when nothing else limits it, a higher bar than the copy
        ach["read_GBs_ungrouped_call"] = line["varlen_grouping"]["arange"]["hbm_GBs"]
        line["roofline"]["frac_of_achievable"] = round(
            line["roofline"]["achieved"] / max(ach["copy_GBs"], ach["read_GBs_ungrouped_call"]), 4)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
        line["cpu_baseline"].update(_host())
        print("[bench] timing the CPU oracle on the other workloads", file=sys.stderr, flush=True)
        line["cpu_baseline"]["other_workloads"] = cpu_baseline_configs()

    if args.all:
        for name in OTHERS:
            print(f"[bench] {name}", file=sys.stderr, flush=True)
            print(json.dumps(OTHERS[name](args)), file=sys.stderr, flush=True)
            torch.cuda.empty_cache()

    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
