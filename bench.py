#!/usr/bin/env python3
"""Benchmark of the ODA decode step on one MI355X.

Workload (default): Qwen3-1.7B-shaped attention stack -- 28 layers, 16 query
/ 8 KV heads, head_dim 128 -- batch 4, 131,072-token contiguous bf16 KV
cache per sequence (60 GB), three planted far needles, random Xavier fp32
recall head, threshold tuned so that 12.5% of (sequence, step) decisions
take the full branch.  All inputs are synthetic (seeded generator G, filled
on the device) and resident in HBM before any timing: the cache, and every
step's q / k / v of both branches and embedding.

One step = local attention of all 28 layers, recall score + rule + work
list, conditional full attention of all 28 layers, commit.

Protocol: a calibration pass with theta = +inf (all local) records the
head's scores and sets theta to the midpoint between the k-th and (k+1)-th
largest, k = round(0.125 * B * steps); the state is reset; W warm-up steps.
Each step is captured into its own HIP graph, bound to that step's inputs.
The timed region replays the K graphs in order from one start state, REPEATS
times; the median is the reported warm throughput.  The same K steps are
then replayed as three graphs each (local + score | the L full-attention
launches | commit), the middle one bracketed by a pair of HIP events on its
stream: that gives the dominant kernel's average launch duration and, from
the recorded flags and positions, its algorithmic bytes per launch, t_b *
4096 B (K and V of every key of every flagged sequence, including the staged
current token).  Both passes run the same kernels on the same inputs, so
they follow the same trajectory.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import dataclasses
import json
import math
import os
import statistics
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--repeats", type=int, default=3)
    ap.add_argument("--workload", default="3", help="workload key (default 3: 128K, B=4, 12.5%% recall)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rate-sweep", default="0,0.125,0.25,0.5,1",
                    help="comma list of forced full-branch rates to time as well (per-step graphs, exact counts); "
                         "empty to skip")
    ap.add_argument("--no-always-full", action="store_true",
                    help="skip the always-full baseline (every sequence takes the full branch, no local attention "
                         "and no recall head: the work list, the full attention and the commit)")
    ap.add_argument("--no-first-request", action="store_true",
                    help="skip the first-request timings (a fresh process per measurement: capture plus the "
                         "first K steps, ODA and always-full)")
    ap.add_argument("--first-request-cell", default="", help=argparse.SUPPRESS)  # child: oda | always-full
    ap.add_argument("--pmc-summary", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "BENCH_JSON"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; csv) of a bench run with "
                         "--copy-calibration: HBM bytes per launch of k_attn_full and k_attn_local over the "
                         "split-graph region, each counter scaled by what it reads for the plain 1 GiB copies; prints "
                         "one JSON object (the entries of profiles/hbm_traffic.json) and a markdown table")
    ap.add_argument("--trace-summary", nargs=2, metavar=("TRACE_DIR", "BENCH_JSON"),
                    help="summarise a rocprofv3 --kernel-trace (csv) of a bench run: per-kernel durations over "
                         "the whole run and over the split-graph region its JSON line names (trace_window), and "
                         "the roofline fraction those durations give; prints markdown")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--matrix", action="store_true",
                    help="context x forced recall-rate matrix at batch 1, warm and first-request timings "
                         "(one JSON line per cell, then a summary line)")
    ap.add_argument("--matrix-contexts", default="4096,16384,32768,65536,131072")
    ap.add_argument("--matrix-rates", default="0,0.125,0.25,0.5,1")
    ap.add_argument("--matrix-cell", default="", help=argparse.SUPPRESS)  # child process: CONTEXT:RATE, cold run
    ap.add_argument("--decoder", action="store_true",
                    help="the step with the dense Qwen3-1.7B-shaped decoder around the path (random-init bf16 "
                         "weights): the workload's batch and context, theta tuned to its rate, against always-full")
    ap.add_argument("--decoder-matrix", action="store_true",
                    help="decoder step at batch 1: context x forced recall-rate matrix, warm and first-request")
    ap.add_argument("--decoder-cell", default="", help=argparse.SUPPRESS)  # child process: CONTEXT:RATE, cold run
    ap.add_argument("--hybrid", action="store_true",
                    help="hybrid backbone: 6 attention layers on the ODA path between 18 recurrent (gated delta "
                         "rule) layers whose states go through the save / restore / commit transaction; theta "
                         "tuned to the pages' hybrid call rate, against always-full")
    ap.add_argument("--train", action="store_true",
                    help="one recall-head training step (labels through the tied LM head, then the head's "
                         "forward, Huber loss and backward) on a 4 x 2048-position micro-batch")
    return ap.parse_args()


def main():
    args = parse()
    if args.trace_summary:
        return trace_summary(*args.trace_summary)
    if args.pmc_summary:
        return pmc_summary(*args.pmc_summary)
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the step is timed on one GPU's share "
                                   "of the batch, and runs over several GPUs are not provided", "n_gpus": args.gpus}))
        sys.exit(2)
    if args.matrix:
        return matrix(args)
    if args.decoder_matrix:
        return decoder_matrix(args)
    import torch
    import synth

    if args.matrix_cell:
        ctx, rate = args.matrix_cell.split(":")
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            print(json.dumps(matrix_cell(int(ctx), float(rate), args, stream, torch, cold=True)), flush=True)
        return

    if args.decoder_cell:
        ctx, rate = args.decoder_cell.split(":")
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            print(json.dumps(decoder_cell(int(ctx), float(rate), args, stream, torch, cold=True)), flush=True)
        return

    if args.hybrid:
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            hybrid_bench(args, stream, torch)
        return
    if args.train:
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            train_bench(args, stream, torch)
        return

    wl_key = int(args.workload) if args.workload.isdigit() else args.workload
    wl = synth.workloads()[wl_key]
    if args.decoder:
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            decoder_bench(args, wl, stream, torch)
        return
    if max(args.steps, args.warmup) > wl.steps:
        # more steps than the workload defines: the same workload with room
        # for them (every step's inputs come from the seeded generator)
        wl = wl.replace(steps=max(args.steps, args.warmup))
    stream = torch.cuda.Stream()  # a non-default stream, so the steps can be graph-captured
    with torch.cuda.stream(stream):
        if args.first_request_cell:
            print(json.dumps(first_request_cell(args, wl, stream, torch)), flush=True)
            return
        run(args, wl, stream, torch)


class Session:
    """Device state of one workload: the cache, the workspace, every step's
    synthetic inputs (written into HBM here, before any timing) and one
    StepPlan per step bound to that step's inputs.  ``force_table`` (host
    [steps][B] int8, default all -1: every decision by the head) sets the
    per-step forced flags; each step's plan reads its row of the device copy,
    so rewriting ``force_dev`` changes the schedule of graphs already
    captured."""

    def __init__(self, wl, nsteps, stream, theta, force_table=None):
        import torch
        import synth
        import synth.device as sd
        import conditional_sparse_attention_amd as C
        from conditional_sparse_attention_amd.step import StepBuffers, StepPlan
        self.torch, self.C, self.wl, self.nsteps, self.stream = torch, C, wl, nsteps, stream
        dev = "cuda"
        L, B, Hq, Hkv, d, D = wl.layers, wl.batch, wl.hq, wl.hkv, wl.head_dim, wl.hidden
        self.t0 = torch.from_numpy(wl.t0.astype(np.int32)).to(dev)
        if wl.layout == "paged":
            tables_np, nblocks = synth.paged_block_tables(wl)
            tables = torch.from_numpy(tables_np).to(dev)
            self.dims = C.make_dims(L, B, Hq, Hkv, kv_layout=C.ODA_KV_PAGED, block_size=wl.block_size,
                                    max_blocks_per_seq=tables_np.shape[1], num_blocks=nblocks, sink=wl.sink,
                                    window=wl.window)
            self.K = torch.empty((L, nblocks, Hkv, wl.block_size, d), dtype=torch.int16, device=dev)
        else:
            tables, nblocks = None, 0
            self.dims = C.make_dims(L, B, Hq, Hkv, t_cap=wl.t_cap, sink=wl.sink, window=wl.window)
            self.K = torch.empty((L, B, Hkv, wl.t_cap, d), dtype=torch.int16, device=dev)
        self.V = torch.empty_like(self.K)
        sd.fill_cache(self.K, wl, synth.TAG_K, self.t0, tables=tables, num_blocks=nblocks)
        sd.fill_cache(self.V, wl, synth.TAG_V, self.t0, tables=tables, num_blocks=nblocks)
        self.tables = tables
        self.kv = C.make_kv(self.K, self.V, tables)
        self.ws = torch.zeros(C.oda_workspace_bytes(self.dims), dtype=torch.uint8, device=dev)
        C.oda_workspace_init(self.dims, self.ws)
        self.blob = synth.head_blob(D, wl.head_seed)
        self.h0 = torch.from_numpy(synth.h_prev0(wl).view(np.int16)).to(dev)
        z = lambda *sh, dt=torch.int16: torch.zeros(sh, dtype=dt, device=dev)
        # every step's inputs: [step][L][B][H][d] and [step][B][D]
        self.inp = {"qL": z(nsteps, L, B, Hq, d), "qF": z(nsteps, L, B, Hq, d), "kL": z(nsteps, L, B, Hkv, d),
                    "vL": z(nsteps, L, B, Hkv, d), "kF": z(nsteps, L, B, Hkv, d), "vF": z(nsteps, L, B, Hkv, d),
                    "e": z(nsteps, B, D)}
        pos_j = self.t0.clone()
        for j in range(nsteps):
            pos_j.copy_(self.t0 + j)
            sd.fill_step({k: v[j] for k, v in self.inp.items()}, wl, pos_j, self.t0)
        if force_table is None:
            force_table = np.full((nsteps, B), -1, np.int8)
        self.force_table = np.asarray(force_table, np.int8)
        self.force_dev = torch.from_numpy(self.force_table).to(dev)
        self.state = StepBuffers(pos=self.t0.clone(), qL=None, kL=None, vL=None, qF=None, kF=None, vF=None, emb=None,
                                 h_prev=self.h0.clone(), head_w=torch.from_numpy(self.blob).to(dev),
                                 oL=z(L, B, Hq, d), oF=z(L, B, Hq, d), score=z(B, dt=torch.float32),
                                 flag=z(B, dt=torch.uint8), force=torch.full((B,), -1, dtype=torch.int8, device=dev))
        self.plans = []
        for j in range(nsteps):
            b = dataclasses.replace(self.state, qL=self.inp["qL"][j], kL=self.inp["kL"][j], vL=self.inp["vL"][j],
                                    qF=self.inp["qF"][j], kF=self.inp["kF"][j], vF=self.inp["vF"][j],
                                    emb=self.inp["e"][j],
                                    force=self.force_dev[j])
            self.plans.append(StepPlan(self.dims, self.kv, self.ws, b, theta=theta, stream=stream))
        self.flag_all = torch.ones(B, dtype=torch.uint8, device=dev)
        # one plan on fixed step buffers, for a single graph that serves every
        # step: the step's inputs (and forced flags) are copied into the
        # buffers on the device, selected by pos - t0
        self.buf = {k: torch.zeros_like(v[0]) for k, v in self.inp.items()}
        fb = dataclasses.replace(self.state, qL=self.buf["qL"], kL=self.buf["kL"], vL=self.buf["vL"],
                                 qF=self.buf["qF"], kF=self.buf["kF"], vF=self.buf["vF"], emb=self.buf["e"])
        self.fixed_plan = StepPlan(self.dims, self.kv, self.ws, fb, theta=theta, stream=stream)
        torch.cuda.synchronize()

    def feed_fixed(self):
        """Copy the current step's inputs (and forced flags) from the resident
        per-step table into the fixed step buffers (device-side selection)."""
        torch = self.torch
        j = (self.state.pos[:1] - self.t0[:1]).clamp(0, self.nsteps - 1).long()
        for k, v in self.inp.items():
            torch.index_select(v, 0, j, out=self.buf[k].unsqueeze(0))
        torch.index_select(self.force_dev, 0, j, out=self.state.force.unsqueeze(0))

    def fixed_step(self, always_full=False):
        self.feed_fixed()
        if always_full:
            p = self.fixed_plan
            dp = ctypes.byref(self.dims)
            self.C.check(p._lib.oda_worklist(dp, self.flag_all.data_ptr(), self.state.pos.data_ptr(),
                                             self.ws.data_ptr(), self.ws.numel(), self.stream.cuda_stream),
                         "oda_worklist")
            p.full()
            a = list(p.commit_args)
            a[3] = self.flag_all.data_ptr()
            self.C.check(p._lib.oda_commit(*a), "oda_commit")
        else:
            self.fixed_plan.run()

    def reset(self):
        self.state.pos.copy_(self.t0)
        self.state.h_prev.copy_(self.h0)

    def set_theta(self, theta):
        for p in self.plans + [self.fixed_plan]:
            p.set_theta(theta)

    def always_full_step(self, j):
        """The always-full baseline's step j: every sequence takes the full
        branch; no local attention and no recall head."""
        p = self.plans[j]
        C = self.C
        dp = ctypes.byref(self.dims)
        C.check(p._lib.oda_worklist(dp, self.flag_all.data_ptr(), self.state.pos.data_ptr(), self.ws.data_ptr(),
                                    self.ws.numel(), self.stream.cuda_stream), "oda_worklist")
        p.full()
        a = list(p.commit_args)
        a[3] = self.flag_all.data_ptr()
        C.check(p._lib.oda_commit(*a), "oda_commit")

    def capture(self, fn, count):
        """One HIP graph per step j < count, each capturing fn(j)."""
        torch = self.torch
        graphs = []
        for j in range(count):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=self.stream):
                fn(j)
            graphs.append(g)
        torch.cuda.synchronize()
        return graphs

    def time_graphs(self, graphs, repeats):
        """Median over repeats of the time to replay the graphs in order from
        the start state (ms)."""
        torch = self.torch
        runs = []
        for _ in range(repeats):
            self.reset()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(self.stream)
            for g in graphs:
                g.replay()
            e1.record(self.stream)
            torch.cuda.synchronize()
            runs.append(e0.elapsed_time(e1))
        return statistics.median(runs)

    def error_bits(self):
        return int(self.ws[:4].view(self.torch.int32).item())


BASELINE_METRIC = "ODA decode steps/s + KV HBM GB/s (% peak) at 128K ctx, 12.5% recall, 1 GPU"


def metric_label(wl) -> str:
    """The metric text for a workload: context and recall schedule.  For the
    128K batch of 4 at a 12.5% rate this is exactly the headline metric."""
    if np.all(wl.t0 == wl.t0[0]):
        ctx = f"{int(wl.t0[0]) // 1024}K ctx"
    else:
        ctx = f"ragged {int(np.min(wl.t0)) // 1024}K-{int(np.max(wl.t0)) // 1024}K ctx"
    if wl.rate is not None:
        sched = f"{wl.rate * 100:g}% recall"
    elif wl.bernoulli_odd is not None:
        sched = f"recall by the head (theta {wl.theta:g}) on even and Bernoulli({wl.bernoulli_odd:g}) on odd sequences"
    else:
        sched = f"recall by the head at theta {wl.theta:g}"
    return f"ODA decode steps/s + KV HBM GB/s (% peak) at {ctx}, {sched}, 1 GPU"


def calibrated_theta(S, K, torch):
    """theta for the workload's rate, or the workload's fixed theta; the
    state is reset.  An all-local pass over the K steps (theta = +inf) gives
    a first threshold, then passes of the ODA step itself re-tune it until
    its own trajectory sends round(rate * B * K) decisions to the full
    branch (match_rate).  Returns (theta, calibrated, passes, record)."""
    from conditional_sparse_attention_amd.step import match_rate, tune_theta
    wl = S.wl
    if wl.rate is None:
        return float(wl.theta), False, 0, None
    B = wl.batch
    scores = torch.zeros((K, B), dtype=torch.float32, device="cuda")
    flags = torch.zeros((K, B), dtype=torch.uint8, device="cuda")

    def run_pass(theta):
        S.set_theta(theta)
        S.reset()
        for j in range(K):
            S.plans[j].run()
            scores[j].copy_(S.state.score)
            flags[j].copy_(S.state.flag)
        torch.cuda.synchronize()
        return scores.cpu().numpy(), flags.cpu().numpy()

    theta0 = tune_theta(run_pass(math.inf)[0], wl.rate)
    theta, n, k, passes = match_rate(run_pass, theta0, wl.rate)
    S.reset()
    return theta, True, 1 + passes, {"all_local_theta": theta0, "trajectory_passes": passes,
                                     "full_decisions": n, "target_full_decisions": k}


def run(args, wl, stream, torch):
    import synth
    L, B, Hq, Hkv, d, D = wl.layers, wl.batch, wl.hq, wl.hkv, wl.head_dim, wl.hidden
    t_setup = time.time()
    nsteps = max(args.steps, args.warmup, 1)
    force_table = None
    if wl.bernoulli_odd is not None:
        force_table = np.stack([synth.bernoulli_force(wl, j) for j in range(nsteps)])
    S = Session(wl, nsteps, stream, theta=math.inf, force_table=force_table)
    setup_s = time.time() - t_setup
    K = args.steps

    # ---- calibration: all-local scores -> theta for the target rate
    theta, calibrated, tune_passes, tuning = calibrated_theta(S, K, torch)
    S.set_theta(theta)

    # ---- warm-up
    S.reset()
    for j in range(args.warmup):
        S.plans[j].run()
    torch.cuda.synchronize()

    # ---- timed region: the K per-step graphs replayed in order from the
    # same start state, REPEATS times; the median is the reported throughput
    graphs = S.capture(lambda j: S.plans[j].run(), K)
    ms_total = S.time_graphs(graphs, args.repeats)

    # ---- the same K steps as four graphs per step (the L local launches |
    # score | the L full-attention launches | commit), a pair of HIP events on
    # the stream around the first and the third: the attention kernels'
    # average launch durations, free of host launch gaps; the recorded flags
    # and positions fix their algorithmic bytes
    g_loc = S.capture(lambda j: S.plans[j].local(), K)
    g_score = S.capture(lambda j: S.plans[j].score(), K)
    g_full = S.capture(lambda j: S.plans[j].full(), K)
    g_post = S.capture(lambda j: S.plans[j].commit(), K)
    flags_hist = torch.zeros((K, B), dtype=torch.uint8, device="cuda")
    pos_hist = torch.zeros((K, B), dtype=torch.int32, device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    ev_loc = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    ev_sc = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    S.reset()
    torch.cuda.synchronize()
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    e_start.record(stream)
    for j in range(K):
        pos_hist[j].copy_(S.state.pos)
        l0, l1 = ev_loc[j]
        l0.record(stream)
        g_loc[j].replay()
        l1.record(stream)
        s0, s1 = ev_sc[j]
        s0.record(stream)
        g_score[j].replay()
        s1.record(stream)
        e0, e1 = ev[j]
        e0.record(stream)
        g_full[j].replay()
        e1.record(stream)
        g_post[j].replay()
        flags_hist[j].copy_(S.state.flag)
    e_end.record(stream)
    torch.cuda.synchronize()
    split_ms = e_start.elapsed_time(e_end)
    full_ms = sum(e0.elapsed_time(e1) for e0, e1 in ev)
    local_ms = sum(l0.elapsed_time(l1) for l0, l1 in ev_loc)
    score_ms = sum(s0.elapsed_time(s1) for s0, s1 in ev_sc)
    del g_loc, g_score, g_full, g_post
    fl = flags_hist.cpu().numpy().astype(np.int64)
    ps = pos_hist.cpu().numpy().astype(np.int64)
    full_bytes = float(np.sum(fl * (ps + 1))) * Hkv * d * 2 * 2 * L
    assert S.error_bits() == 0, "device error bits set"

    ms_step = ms_total / K
    steps_per_s = 1000.0 / ms_step
    realised = float(fl.mean())
    kv_local = 0
    for b in range(B):
        for j in range(K):
            t = int(wl.t0[b]) + j + 1
            kv_local += min(t, wl.sink + wl.window)
    kv_bytes_step = (kv_local + float(np.sum(fl * (ps + 1)))) * Hkv * d * 2 * 2 * L / K
    ctx = int(wl.t0[0]) if np.all(wl.t0 == wl.t0[0]) else f"ragged {int(np.min(wl.t0))}-{int(np.max(wl.t0))}, " \
                                                             f"mean {float(np.mean(wl.t0)):.0f}"
    out = {
        "metric": metric_label(wl),
        "value": round(steps_per_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded generator, inputs device-generated into HBM before timing; random-init Xavier "
                "recall head)",
        "config": {"workload": wl.name, "layers": L, "batch": B, "context": ctx, "q_heads": Hq,
                   "kv_heads": Hkv, "head_dim": d, "kv_layout": wl.layout, "recall_rate_target": wl.rate,
                   "recall_rate_realised": realised, "theta": theta, "theta_calibrated": calibrated,
                   "theta_tuning": tuning,
                   "tokens_per_s": round(steps_per_s * B, 1),
                   "repeats": args.repeats, "timing": "per-step hip-graph replay, median of repeats",
                   "split_graph_steps_per_s": round(1000.0 * K / split_ms, 2)},
        "kv_gbs": round(kv_bytes_step / (ms_step * 1e-3) / 1e9, 1),
        "kv_frac_peak": round(kv_bytes_step / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
    }
    if wl.bernoulli_odd is not None:
        even = np.arange(B) % 2 == 0
        out["config"]["recall_rate_realised_head_half"] = round(float(fl[:, even].mean()), 4)
        out["config"]["recall_rate_realised_forced_half"] = round(float(fl[:, ~even].mean()), 4)
    nlaunch = K * L
    avg_us = full_ms * 1e3 / nlaunch
    bytes_per_launch = full_bytes / nlaunch
    achieved = bytes_per_launch / (avg_us * 1e-6) / 1e9
    traffic, traffic_note = measured_traffic(wl.name, bytes_per_launch)
    local_bytes = kv_local * Hkv * d * 2 * 2 * L
    both_gbs = (local_bytes + full_bytes) / ((local_ms + full_ms) * 1e-3) / 1e9
    local_traffic, local_traffic_note = measured_traffic(wl.name, local_bytes / nlaunch, kernel="k_attn_local")
    out["attention_kernels"] = {
        "local_avg_launch_us": round(local_ms * 1e3 / nlaunch, 2),
        "local_algorithmic_bytes_per_launch": int(local_bytes / nlaunch),
        "local_traffic": local_traffic, "local_traffic_note": local_traffic_note,
        "local_gbs": round(local_bytes / (local_ms * 1e-3) / 1e9, 1),
        "local_frac": round(local_bytes / (local_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "full_gbs": round(full_bytes / (full_ms * 1e-3) / 1e9, 1),
        "kv_gbs": round(both_gbs, 1),
        "kv_frac_peak": round(both_gbs / HBM_PEAK_GBS, 4),
        "note": "KV bytes read / summed launch time of the local and the full attention launches (HIP events "
                "around each step's graph of L launches; local includes the per-launch split hand-off)"}
    head_bytes = 4 * synth_head_params(D)
    out["recall_head"] = {"avg_us_per_step": round(score_ms * 1e3 / K, 2),
                          "weight_gbs": round(head_bytes / (score_ms * 1e-3 / K) / 1e9, 1),
                          "frac": round(head_bytes / (score_ms * 1e-3 / K) / 1e9 / HBM_PEAK_GBS, 4),
                          "note": "oda_recall_score per step (HIP events around its graph): fp32 head weights "
                                  "streamed once / time"}
    # dispatch windows of the split region, in this process's launch order,
    # so a kernel trace of the same command can be cut to the same launches
    before = tune_passes * K + args.warmup + args.repeats * K
    out["roofline"] = {"bound": "hbm", "kernel": "k_attn_full (oda_full_attn_if)", "achieved": round(achieved, 1),
                       "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                       "traffic": traffic, "traffic_note": traffic_note, "avg_launch_us": round(avg_us, 2),
                       "algorithmic_bytes_per_launch": int(bytes_per_launch), "launches": nlaunch,
                       "duration_source": "HIP events on the launch stream around each step's graph of the L "
                                          "full-attention launches (empty launches included, with zero bytes)",
                       "attention_kernels_frac": out["attention_kernels"]["kv_frac_peak"],
                       "trace_window": {"k_attn_full": [before * L, nlaunch], "k_attn_local": [before * L, nlaunch],
                                        "pid": os.getpid()}}
    if args.rate_sweep and wl.bernoulli_odd is None:
        out["rate_sweep"] = rate_sweep(args, S, graphs)
    del graphs
    if not args.no_always_full:
        g_af = S.capture(S.always_full_step, K)
        m = S.time_graphs(g_af, args.repeats) / K
        del g_af
        out["always_full"] = {"steps_per_s": round(1000.0 / m, 2), "ms_per_step": round(m, 4),
                              "oda_speedup": round(steps_per_s / (1000.0 / m), 3)}
    out["setup_s"] = round(setup_s, 1)
    out["device_copy"] = device_copy_gbs(torch, stream)
    if args.copy_calibration:
        src = torch.empty(1 << 29, dtype=torch.int16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = 2 * src.numel() * src.element_size()
    blob = S.blob
    del S
    torch.cuda.empty_cache()
    if not args.no_first_request:
        out["first_request"] = first_request(args, wl, theta)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, blob, theta, realised)
    print(json.dumps(out), flush=True)


def synth_head_params(hidden: int) -> int:
    """Recall-head parameter count for input width `hidden` (from the
    library's packed layout)."""
    import conditional_sparse_attention_amd as C
    return C.oda_head_param_count(hidden)


def first_request(args, wl, theta):
    """The pages' first-request protocol (capture included), next to the warm
    one: each measurement runs in a fresh process (setup untimed), capturing
    one graph that serves every step and timing capture plus the first N
    steps, N the workload's decode-step count (one request); the same
    process then times the warm median of REPEATS replays of N steps.  ODA
    with the run's theta, and always-full."""
    import subprocess
    import synth
    key = int(args.workload) if str(args.workload).isdigit() else args.workload
    n = synth.workloads()[key].steps
    res = {"protocol": f"fresh process per measurement; cold = capture + the first {n} steps (the workload's decode "
                       "steps, one request; host clock); warm = median of repeats of the same steps replayed with "
                       "the same single graph; the step's inputs are selected on the device from a resident "
                       "per-step table inside the graph", "steps": n}
    for mode in ("oda", "always-full"):
        cmd = [sys.executable, os.path.abspath(__file__), "--workload", str(args.workload), "--steps",
               str(n), "--warmup", str(args.warmup), "--repeats", str(args.repeats),
               "--first-request-cell", f"{mode}:{theta!r}"]
        cp = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        if cp.returncode != 0:
            raise SystemExit(f"first-request cell {mode} failed ({cp.returncode}): {cp.stderr[-2000:]}")
        res[mode.replace("-", "_")] = json.loads(cp.stdout.strip().splitlines()[-1])
    res["speedup_cold"] = round(res["oda"]["cold_steps_per_s"] / res["always_full"]["cold_steps_per_s"], 3)
    res["speedup_warm"] = round(res["oda"]["warm_steps_per_s"] / res["always_full"]["warm_steps_per_s"], 3)
    return res


def first_request_cell(args, wl, stream, torch):
    """Child process of first_request(): mode oda:THETA or always-full:THETA."""
    import synth
    mode, theta = args.first_request_cell.split(":", 1)
    K = args.steps
    nsteps = max(K, args.warmup, 1)
    force_table = None
    if wl.bernoulli_odd is not None:
        force_table = np.stack([synth.bernoulli_force(wl, j) for j in range(nsteps)])
    S = Session(wl, nsteps, stream, theta=float(theta), force_table=force_table)
    af = mode == "always-full"
    S.reset()
    torch.cuda.synchronize()
    c0 = time.perf_counter()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        S.fixed_step(always_full=af)
    for _ in range(K):
        g.replay()
    torch.cuda.synchronize()
    cold_ms = (time.perf_counter() - c0) * 1e3
    warm_ms = S.time_graphs([g] * K, args.repeats)
    assert S.error_bits() == 0, "device error bits set"
    return {"mode": mode, "cold_ms_per_step": round(cold_ms / K, 4), "cold_steps_per_s": round(1e3 * K / cold_ms, 2),
            "warm_ms_per_step": round(warm_ms / K, 4), "warm_steps_per_s": round(1e3 * K / warm_ms, 2)}


TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "hbm_traffic.json")
KERNEL_SOURCES = ("conditional_sparse_attention_amd/csrc/attn.hip", "conditional_sparse_attention_amd/csrc/oda_internal.h")


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for p in KERNEL_SOURCES:
        with open(os.path.join(root, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def device_copy_gbs(torch, stream, n_bytes=1 << 30, reps=5):
    """The box's achievable streaming rate for a plain read + write kernel:
    a device-to-device copy of an n_bytes buffer (n_bytes read and n_bytes
    written per copy), timed with HIP events on the bench's stream after
    every timed region."""
    src = torch.empty(n_bytes // 2, dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)
    with torch.cuda.stream(stream):
        dst.copy_(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            dst.copy_(src)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return {"gbs": round(2 * n_bytes / (ms * 1e-3) / 1e9, 1), "bytes_per_copy": 2 * n_bytes,
            "note": "device-to-device copy of 1 GiB (read + write): the measured ceiling of a plain streaming kernel "
                    "on this box, for reading roofline.frac"}


def measured_traffic(workload, bytes_per_launch, kernel="k_attn_full"):
    """HBM bytes per launch of `kernel` on this workload from the committed
    rocprofv3 PMC measurement (FETCH_SIZE + WRITE_SIZE, each normalised on a
    1 GiB copy), as its ratio to the algorithmic bytes of the measured
    launches times this run's algorithmic bytes per launch; None when this
    kernel and workload were not counted, or the kernel source changed
    since."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None, "no counter measurement"
    ent = rec.get(kernel, {}).get(workload)
    if ent is None:
        return None, f"{kernel} not counted on {workload}"
    if ent.get("kernel_source_sha256") != kernel_source_hash():
        return None, "kernel changed since the counters were taken"
    ratio = ent["hbm_bytes_per_launch"] / ent["algorithmic_bytes_per_launch"]
    return int(ratio * bytes_per_launch), f"PMC ratio {ratio:.5f} of algorithmic bytes ({os.path.basename(TRAFFIC_FILE)})"


def rate_sweep(args, S, graphs):
    """Step time at forced full-branch rates: exact counts round(rate * K * B)
    placed by seeded uniforms (the pages' hand-scheduled calls), replaying
    the run's per-step graphs with the force table rewritten; then the run's
    own table is restored."""
    import synth
    torch = S.torch
    wl = S.wl
    res = []
    saved = S.force_dev.clone()
    for r in [float(x) for x in args.rate_sweep.split(",") if x]:
        flags = synth.forced_rate_flags(wl.seed, args.steps, wl.batch, r)
        S.force_dev[:args.steps].copy_(torch.from_numpy(flags).to("cuda"))
        ms = S.time_graphs(graphs, args.repeats) / args.steps
        res.append({"rate": r, "ms_per_step": round(ms, 4), "steps_per_s": round(1000.0 / ms, 2)})
    S.force_dev.copy_(saved)
    torch.cuda.synchronize()
    x = np.array([q["rate"] for q in res])
    y = np.array([q["ms_per_step"] for q in res])
    if len(res) >= 2:
        slope, icpt = np.polyfit(x, y, 1)
        pred = slope * x + icpt
        r2 = 1 - np.sum((y - pred) ** 2) / max(np.sum((y - y.mean()) ** 2), 1e-30)
        # one unit of rate flags every sequence: the slope over B is the
        # marginal cost of one flagged sequence-step, whose full-branch KV
        # bytes are L * 4096 B per key of its mean length over the steps
        t_mean = float(np.mean(wl.t0)) + (args.steps + 1) / 2.0
        seq_bytes = wl.layers * t_mean * wl.hkv * wl.head_dim * 2 * 2
        per_seq_ms = float(slope) / wl.batch
        return {"points": res, "timing": "per-step hip-graph replay, median of repeats",
                "fit_ms_per_step": {"slope_per_unit_rate": round(float(slope), 4),
                                    "intercept": round(float(icpt), 4), "r2": round(float(r2), 5)},
                "marginal_flagged_sequence": {"ms": round(per_seq_ms, 4), "kv_bytes": int(seq_bytes),
                                              "gbs": round(seq_bytes / (per_seq_ms * 1e-3) / 1e9, 1)}}
    return {"points": res}


def _short_kernel_name(name: str) -> str:
    """'void ns::(anonymous namespace)::k_x<2, false>(ns::P)' -> 'k_x<2, false>'."""
    n = name.strip().strip('"')
    depth, cut = 0, len(n)
    for i in range(len(n) - 1, -1, -1):  # drop the trailing parameter list
        c = n[i]
        if c == ")":
            depth += 1
        elif c == "(":
            depth -= 1
            if depth == 0:
                cut = i
                break
    n = n[:cut]
    depth, start = 0, 0
    for i, c in enumerate(n):  # last '::' outside template brackets
        if c == "<":
            depth += 1
        elif c == ">":
            depth -= 1
        elif c == ":" and depth == 0 and i + 1 < len(n) and n[i + 1] == ":":
            start = i + 2
    n = n[start:]
    return n[5:] if n.startswith("void ") else n


def trace_summary(trace_dir: str, bench_json: str) -> None:
    """Markdown summary of a rocprofv3 kernel trace of one bench run.  The
    process with the most k_attn_full dispatches is the bench itself (its
    first-request children trace separately).  Its kernels are listed over
    the whole run and over the split-graph region: the time span from the
    first k_attn_local to the last k_attn_full dispatch of the windows the
    bench's JSON line gives (dispatch order within the process)."""
    import csv
    import glob
    with open(bench_json) as f:
        line = [l for l in f.read().splitlines() if l.strip().startswith("{")][-1]
    rec = json.loads(line)
    win = rec.get("roofline", {}).get("trace_window")
    per_file = {}
    for path in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(path, newline="") as f:
            rows = [(r["Kernel_Name"], int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in csv.DictReader(f)]
        per_file[path] = rows
    if not per_file:
        raise SystemExit(f"no *kernel_trace.csv under {trace_dir}")
    pid = (win or {}).get("pid")
    path = _bench_process_file(list(per_file), pid,
                               lambda p: (sum("k_attn_full" in r[0] for r in per_file[p]), len(per_file[p])))
    rows = sorted(per_file[path], key=lambda r: r[1])

    def stats(sel):
        agg = {}
        for name, t0, t1 in sel:
            a = agg.setdefault(_short_kernel_name(name), [0, 0.0, math.inf, 0.0])
            us = (t1 - t0) / 1e3
            a[0] += 1
            a[1] += us
            a[2] = min(a[2], us)
            a[3] = max(a[3], us)
        return sorted(agg.items(), key=lambda kv: -kv[1][1])

    def window(kernel):
        first, n = win[kernel]
        ds = [r for r in rows if kernel in r[0]]
        return ds[first:first + n]

    if win is None:
        # a line without attention windows (decoder, hybrid, training): the
        # whole process only
        total = sum((t1 - t0) for _, t0, t1 in rows) / 1e3
        out = [f"Trace file: `{os.path.relpath(path, trace_dir)}` ({len(rows)} dispatches, {total / 1e3:.1f} ms of "
               f"kernel time). JSON line of the profiled run: `{rec['metric']}`, value {rec['value']} {rec['unit']}, "
               f"{rec['steps']} steps, warm-up {rec['warmup']}.", "",
               "| kernel | calls | total (us) | avg (us) | min (us) | max (us) | % of kernel time |",
               "|---|---|---|---|---|---|---|"]
        for name, (n, tot, mn, mx) in stats(rows)[:25]:
            out.append(f"| `{name}` | {n} | {tot:.1f} | {tot / n:.2f} | {mn:.2f} | {mx:.2f} | {100 * tot / total:.1f} |")
        print("\n".join(out))
        return
    wl_full, wl_local = window("k_attn_full"), window("k_attn_local")
    t_lo, t_hi = wl_local[0][1], wl_full[-1][2]
    region = [r for r in rows if r[1] >= t_lo and r[2] <= t_hi]
    K = rec["steps"]
    full_avg = sum((t1 - t0) for _, t0, t1 in wl_full) / len(wl_full) / 1e3
    local_avg = sum((t1 - t0) for _, t0, t1 in wl_local) / len(wl_local) / 1e3
    bpl = rec["roofline"]["algorithmic_bytes_per_launch"]
    frac = bpl / (full_avg * 1e-6) / 1e9 / HBM_PEAK_GBS
    cfg = rec["config"]
    out = [f"# Kernel trace of one bench run: {cfg['workload']}", "",
           f"Trace file: `{os.path.relpath(path, trace_dir)}` (the bench process). JSON line: `{rec['metric']}`, "
           f"value {rec['value']} {rec['unit']}, {K} steps, warm-up {rec['warmup']}.", "",
           "## Split-graph region (the launches the line's roofline and attention_kernels time)", "",
           f"{len(region)} dispatches, {K} steps; `k_attn_full` dispatches {win['k_attn_full'][0]}.."
           f"{win['k_attn_full'][0] + win['k_attn_full'][1] - 1} of the process.", "",
           "| kernel | calls | total (us) | avg (us) | min (us) | max (us) | per step (us) |", "|---|---|---|---|---|---|---|"]
    for name, (n, tot, mn, mx) in stats(region):
        out.append(f"| `{name}` | {n} | {tot:.1f} | {tot / n:.2f} | {mn:.2f} | {mx:.2f} | {tot / K:.2f} |")
    out += ["", "| quantity | kernel trace | the line (HIP events) |", "|---|---|---|",
            f"| `k_attn_full` avg launch (us) | {full_avg:.2f} | {rec['roofline']['avg_launch_us']} |",
            f"| `k_attn_full` frac of 8 TB/s ({bpl} algorithmic B per launch) | {frac:.4f} | "
            f"{rec['roofline']['frac']} |",
            f"| `k_attn_local` avg launch (us) | {local_avg:.2f} | {rec['attention_kernels']['local_avg_launch_us']} |",
            "", "## Whole process", "",
            "| kernel | calls | total (us) | avg (us) | min (us) | max (us) |", "|---|---|---|---|---|---|"]
    for name, (n, tot, mn, mx) in stats(rows)[:25]:
        out.append(f"| `{name}` | {n} | {tot:.1f} | {tot / n:.2f} | {mn:.2f} | {mx:.2f} |")
    print("\n".join(out))


def _bench_process_file(paths, pid, count_full):
    """The trace file of the bench process: the one rocprofv3 named after the
    pid the JSON line gives (<pid>_...csv); without a pid, the file with the
    most k_attn_full dispatches."""
    if pid is not None:
        own = [p for p in paths if os.path.basename(p).startswith(f"{pid}_")]
        if own:
            return own[0]
        raise SystemExit(f"no trace file of process {pid} among {len(paths)} files")
    return max(paths, key=count_full)


def _pmc_rows(run_dir: str, counter: str, pid=None):
    """Per-dispatch (kernel, value) of one counter from a rocprofv3 --pmc
    csv run: the process with the most k_attn_full dispatches, in dispatch
    order."""
    import csv
    import glob
    per_file = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path, newline="") as f:
            rows = [(int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"]))
                    for r in csv.DictReader(f) if r["Counter_Name"] == counter]
        per_file[path] = rows
    if not per_file:
        raise SystemExit(f"no {counter} rows under {run_dir}")
    path = _bench_process_file(list(per_file), pid, lambda p: sum("k_attn_full" in r[1] for r in per_file[p]))
    rows = sorted(per_file[path])
    return path, [(k, v) for _, k, v in rows]


def pmc_summary(fetch_dir: str, write_dir: str, bench_json: str) -> None:
    """HBM traffic per launch of the attention kernels over the split-graph
    region of a bench run with --copy-calibration, from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled so that it reads the 1 GiB
    (read + write) device copies' known bytes."""
    with open(bench_json) as f:
        rec = json.loads([l for l in f.read().splitlines() if l.strip().startswith("{")][-1])
    win = rec["roofline"]["trace_window"]
    K, L = rec["steps"], rec["config"]["layers"]
    B, Hkv, d = rec["config"]["batch"], rec["config"]["kv_heads"], rec["config"]["head_dim"]
    copy_bytes = rec["copy_calibration_bytes"] // 2        # bytes read (= bytes written) per copy
    out = {"workload": rec["config"]["workload"], "kernel_source_sha256": kernel_source_hash()}
    for counter, run_dir in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        path, rows = _pmc_rows(run_dir, counter)
        copies = [v for k, v in rows if "copyBuffer" in k][-3:]
        factor = copy_bytes / 1024.0 / (sum(copies) / len(copies))
        out[counter] = {"copy_kib": round(sum(copies) / len(copies), 1), "factor": round(factor, 5)}
        for kern in ("k_attn_full", "k_attn_local"):
            first, n = win[kern]
            vals = [v for k, v in rows if kern in k][first:first + n]
            assert len(vals) == n, (kern, len(vals), n)
            out[counter][kern + "_kib_raw"] = round(sum(vals) / n, 2)
            out[counter][kern + "_bytes"] = sum(vals) / n * 1024.0 * factor
    full_alg = rec["roofline"]["algorithmic_bytes_per_launch"]
    local_alg = rec["attention_kernels"]["local_algorithmic_bytes_per_launch"]
    ent = {}
    for kern, alg in (("k_attn_full", full_alg), ("k_attn_local", local_alg)):
        hbm = out["FETCH_SIZE"][kern + "_bytes"] + out["WRITE_SIZE"][kern + "_bytes"]
        ent[kern] = {"kernel_source_sha256": out["kernel_source_sha256"], "hbm_bytes_per_launch": int(hbm),
                     "algorithmic_bytes_per_launch": int(alg), "ratio": round(hbm / alg, 5) if alg else None,
                     "launches": win[kern][1], "fetch_factor": out["FETCH_SIZE"]["factor"],
                     "write_factor": out["WRITE_SIZE"]["factor"]}
    print(json.dumps({"workload": out["workload"], "entries": ent}))
    md = [f"| kernel | FETCH_SIZE raw (KiB/launch) | WRITE_SIZE raw (KiB/launch) | HBM bytes/launch | algorithmic | ratio |",
          "|---|---|---|---|---|---|"]
    for kern in ("k_attn_full", "k_attn_local"):
        e = ent[kern]
        md.append(f"| `{kern}` | {out['FETCH_SIZE'][kern + '_kib_raw']} | {out['WRITE_SIZE'][kern + '_kib_raw']} | "
                  f"{e['hbm_bytes_per_launch']:,} | {e['algorithmic_bytes_per_launch']:,} | {e['ratio']} |")
    md.append(f"\nCopy calibration: FETCH_SIZE reads {out['FETCH_SIZE']['copy_kib']} KiB and WRITE_SIZE "
              f"{out['WRITE_SIZE']['copy_kib']} KiB per 1 GiB copy (factors {out['FETCH_SIZE']['factor']}, "
              f"{out['WRITE_SIZE']['factor']}).")
    print("\n".join(md))


def host_cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or "" when unknown."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def cpu_baseline(wl, blob, theta, rate):
    """The oracle, untuned, on a bounded sample of the same workload: local
    attention of every sequence at the last two layers, the recall head for
    every sequence, and full attention of sequence 0 at the last layer (timed
    three times); scaled to a whole step as
    1 / (L * B * mean t_local + t_head + rate * B * L * mean t_full)."""
    import synth
    import oracle
    from threadpoolctl import threadpool_info
    L, B = wl.layers, wl.batch
    j = 0
    layers = [L - 1, L - 2] if L > 1 else [L - 1]
    emb = synth.embedding(wl, j)
    h0 = synth.h_prev0(wl)
    P = oracle.unpack_head(blob, wl.hidden)

    def history(l, b, lo_rows):
        # committed rows of sequence b (input generation: not timed); the
        # local branch reads only the sink and window rows
        t = int(wl.t0[b])
        K = np.zeros((wl.hkv, t, wl.head_dim), np.uint16)
        V = np.zeros((wl.hkv, t, wl.head_dim), np.uint16)
        lo = max(0, t - wl.window) if lo_rows else 0
        for g in range(wl.hkv):
            for buf, tag in ((K, synth.TAG_K), (V, synth.TAG_V)):
                if lo_rows:
                    buf[g, :wl.sink] = synth.cache_rows(wl, tag, l, b, g, 0, min(wl.sink, t))
                buf[g, lo:] = synth.cache_rows(wl, tag, l, b, g, lo, t)
        return K, V

    t_locals, oL_last = [], {}
    for l in layers:
        inp = {k: synth.step_tensor(wl, k, j, l) for k in ("qL", "kL", "vL")}
        for b in range(B):
            Kh, Vh = history(l, b, True)
            t = int(wl.t0[b])
            c0 = time.perf_counter()
            o = oracle.decode_attention(inp["qL"][b], Kh, Vh, inp["kL"][b], inp["vL"][b],
                                        oracle.local_index_set(t + 1, wl.sink, wl.window))
            t_locals.append(time.perf_counter() - c0)
            if l == L - 1:
                oL_last[b] = o
    c0 = time.perf_counter()
    for b in range(B):
        q = oracle.recall_score(P, h0[b], emb[b], oracle.f64_to_bf16(oL_last[b].reshape(-1)))
        oracle.branch_rule(q, theta)
    t_head = time.perf_counter() - c0
    l = L - 1
    inp = {k: synth.step_tensor(wl, k, j, l) for k in ("qF", "kF", "vF")}
    Kf, Vf = history(l, 0, False)
    t0 = int(wl.t0[0])
    t_fulls = []
    for _ in range(3):
        c0 = time.perf_counter()
        oracle.decode_attention(inp["qF"][0], Kf, Vf, inp["kF"][0], inp["vF"][0], oracle.full_index_set(t0 + 1))
        t_fulls.append(time.perf_counter() - c0)
    t_local, t_full = float(np.mean(t_locals)), float(np.mean(t_fulls))
    step_s = L * B * t_local + t_head + rate * B * L * t_full
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    sample_s = float(np.sum(t_locals) + t_head + np.sum(t_fulls))
    return {"value": round(1.0 / step_s, 5), "unit": "steps/s", "cores": int(threads), "kind": "oracle",
            "host_cpus": os.cpu_count(), "cpu_model": host_cpu_model(),
            "sample": (f"step 0: local attention of all {B} sequences at layers {layers} ({len(t_locals)} runs, "
                       f"mean {t_local:.2f} s), recall head of all {B} ({t_head:.2f} s), full attention of "
                       f"sequence 0 over {t0 + 1} keys at layer {l} (3 runs, mean {t_full:.2f} s); scaled to "
                       f"{L} layers x {B} sequences and {rate:.3f}*{B} flagged sequences per step"),
            "sample_cpu_s": round(sample_s, 2)}


# ---------------------------------------------------------------------------
# context x recall-rate matrix (batch 1), warm and first-request timings
# ---------------------------------------------------------------------------
MATRIX_LAYERS, MATRIX_HQ, MATRIX_HKV = 28, 16, 8


def matrix_workload(ctx, steps, synth):
    return synth.Workload(f"matrix-{ctx}", MATRIX_LAYERS, MATRIX_HQ, MATRIX_HKV, 128, 1,
                          np.array([ctx], dtype=np.int64), steps, seed=3, head_seed=103, t_cap_slack=16)


def matrix_cell(ctx, rate, args, stream, torch, cold):
    """One cell: forced rate `rate` (negative: the always-full baseline) at
    context `ctx`.  The cache and every step's inputs are written into HBM
    before the clock starts (the cache fill stands in for prefill).  A single
    graph serves every step, as a serving engine's would: each step first
    copies its inputs from the resident table into fixed buffers (device
    side, ~0.3 MB at batch 1).  Warm: W warm-up steps, capture, then the median
    of REPEATS replays of K steps.  Cold (a fresh process): capture and the
    first K steps, timed together on the host clock."""
    import synth
    wl = matrix_workload(ctx, args.steps + args.warmup, synth)
    nsteps = max(args.steps, args.warmup, 1)
    # exact count round(rate * steps) of forced full calls
    table = synth.forced_rate_flags(wl.seed, nsteps, wl.batch, max(rate, 0.0))
    S = Session(wl, nsteps, stream, theta=0.0, force_table=table)
    # the plumbing ops of the input selection load their kernels outside the clock
    S.feed_fixed()
    step = lambda: S.fixed_step(always_full=rate < 0)
    out = {"context": ctx, "rate": rate if rate >= 0 else "always-full", "steps": args.steps}
    S.reset()
    torch.cuda.synchronize()
    if cold:
        c0 = time.perf_counter()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            step()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - c0) * 1e3
        out.update({"cold_ms_per_step": round(ms / args.steps, 4), "cold_steps_per_s": round(1e3 * args.steps / ms, 2)})
    else:
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            step()
        ms = S.time_graphs([g] * args.steps, args.repeats) / args.steps
        out.update({"warm_ms_per_step": round(ms, 4), "warm_steps_per_s": round(1e3 / ms, 2)})
    assert S.error_bits() == 0, "device error bits set"
    return out


def matrix(args):
    """Parent of the matrix: warm cells in this process, each cold cell in a
    fresh child process (started as a subprocess before this process touches
    the GPU for that cell's timing)."""
    import subprocess
    import torch
    ctxs = [int(x) for x in args.matrix_contexts.split(",") if x]
    rates = [float(x) for x in args.matrix_rates.split(",") if x] + [-1.0]
    cells = []
    stream = torch.cuda.Stream()
    for ctx in ctxs:
        for r in rates:
            with torch.cuda.stream(stream):
                w = matrix_cell(ctx, r, args, stream, torch, cold=False)
            torch.cuda.empty_cache()
            cmd = [sys.executable, os.path.abspath(__file__), "--matrix-cell", f"{ctx}:{r}", "--steps",
                   str(args.steps), "--warmup", str(args.warmup)]
            cp = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
            if cp.returncode != 0:
                raise SystemExit(f"cold cell {ctx}:{r} failed ({cp.returncode}): {cp.stderr[-2000:]}")
            c = json.loads(cp.stdout.strip().splitlines()[-1])
            w.update({k: v for k, v in c.items() if k.startswith("cold")})
            cells.append(w)
            print(json.dumps(w), flush=True)
    summary = {"matrix": "ODA decode steps/s at batch 1, 28 layers, 16/8 heads, d 128: context x forced rate",
               "steps": args.steps, "warmup": args.warmup, "repeats": args.repeats, "cells": cells}
    for ctx in ctxs:
        base = [c for c in cells if c["context"] == ctx and c["rate"] == "always-full"][0]
        for c in cells:
            if c["context"] == ctx and c["rate"] != "always-full":
                c["warm_speedup_vs_always_full"] = round(c["warm_steps_per_s"] / base["warm_steps_per_s"], 3)
                c["cold_speedup_vs_always_full"] = round(c["cold_steps_per_s"] / base["cold_steps_per_s"], 3)
    print(json.dumps(summary), flush=True)


# ---------------------------------------------------------------------------
# the step with the dense decoder backbone around the path
# ---------------------------------------------------------------------------
DECODER_SHAPE = "qwen3-1.7b"


class DecSession:
    """Device state of a decoder workload: cache, decoder and head weights
    (device-generated, random init), workspaces and the step plan.  Every
    input of a step is device resident: the token comes from the previous
    step's argmax, so one captured graph serves every step.  `force_table`
    (host [steps][B] int8) forces per-step flags, looked up on the device from
    pos - t0."""

    def __init__(self, t0, nsteps, stream, theta, force_table=None, seed=3):
        import torch
        import synth
        import synth.device as sd
        import conditional_sparse_attention_amd as C
        from conditional_sparse_attention_amd.decoder import DecoderBuffers, DecoderPlan, DecoderWeights
        self.torch, self.C, self.stream, self.nsteps = torch, C, stream, nsteps
        sh = synth.decoder_shapes()[DECODER_SHAPE]
        self.sh = sh
        t0 = np.asarray(t0, dtype=np.int64)
        B = len(t0)
        wl = synth.Workload(f"decoder-{sh.name}", sh.layers, sh.hq, sh.hkv, sh.head_dim, B, t0, nsteps, seed=seed,
                            head_seed=seed + 100, t_cap_slack=16)
        self.wl = wl
        dev = "cuda"
        L, Dm = sh.layers, sh.hidden
        self.attn = C.make_dims(L, B, sh.hq, sh.hkv, t_cap=wl.t_cap, sink=wl.sink, window=wl.window)
        self.dd = C.make_dec_dims(self.attn, sh.inter, sh.vocab, sh.rope_theta, sh.eps)
        self.t0 = torch.from_numpy(t0.astype(np.int32)).to(dev)
        self.K = torch.empty((L, B, sh.hkv, wl.t_cap, sh.head_dim), dtype=torch.int16, device=dev)
        self.V = torch.empty_like(self.K)
        sd.fill_cache(self.K, wl, synth.TAG_K, self.t0)
        sd.fill_cache(self.V, wl, synth.TAG_V, self.t0)
        self.kv = C.make_kv(self.K, self.V)
        layers = torch.empty((L, C.oda_dec_layer_numel(self.dd)), dtype=torch.int16, device=dev)
        for l in range(L):
            sd.fill_dec_layer(layers[l], seed, sh, l)
        embed = torch.empty((sh.vocab, Dm), dtype=torch.int16, device=dev)
        sd.fill_dec_embed(embed, seed)
        gamma_f = torch.from_numpy(synth.dec_gain_bits(seed, L, "gamma_final", Dm, False).view(np.int16)).to(dev)
        self.weights = DecoderWeights(layers, embed, gamma_f)
        self.blob = synth.head_blob(Dm, wl.head_seed)
        self.tok0 = torch.from_numpy(synth.dec_first_tokens(seed, B, sh.vocab)).to(dev)
        self.h0 = torch.from_numpy(synth.h_prev0(wl).view(np.int16)).to(dev)
        self.bufs = DecoderBuffers.allocate(self.dd, torch.from_numpy(self.blob).to(dev), self.tok0.clone(),
                                            self.t0.clone(), self.h0.clone())
        self.ws = torch.zeros(C.oda_workspace_bytes(self.attn), dtype=torch.uint8, device=dev)
        C.oda_workspace_init(self.attn, self.ws)
        self.dws = torch.zeros(C.oda_dec_workspace_bytes(self.dd), dtype=torch.uint8, device=dev)
        C.oda_dec_workspace_init(self.dd, self.dws)
        self.plan = DecoderPlan(self.dd, self.kv, self.weights, self.bufs, self.ws, self.dws, theta=theta,
                                stream=stream)
        self.force_dev = None if force_table is None else torch.from_numpy(np.asarray(force_table, np.int8)).to(dev)
        self.flag_all = torch.ones(B, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    def reset(self):
        self.bufs.pos.copy_(self.t0)
        self.bufs.h_prev.copy_(self.h0)
        self.bufs.tokens.copy_(self.tok0)

    def step(self, always_full=False):
        torch = self.torch
        if always_full:
            self.plan.run_always_full(self.flag_all)
            return
        if self.force_dev is not None:
            j = (self.bufs.pos[:1] - self.t0[:1]).clamp(0, self.nsteps - 1).long()
            torch.index_select(self.force_dev, 0, j, out=self.bufs.force.unsqueeze(0))
        self.plan.run()

    def warm_ms(self, steps, warmup, repeats, always_full=False):
        """Median ms per step over repeats of `steps` graph replays."""
        torch = self.torch
        self.reset()
        for _ in range(warmup):
            self.step(always_full)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=self.stream):
            self.step(always_full)
        runs = []
        for _ in range(repeats):
            self.reset()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(self.stream)
            for _ in range(steps):
                g.replay()
            e1.record(self.stream)
            torch.cuda.synchronize()
            runs.append(e0.elapsed_time(e1))
        assert int(self.ws[:4].view(torch.int32).item()) == 0, "device error bits set"
        return statistics.median(runs) / steps


def decoder_bench(args, wl, stream, torch):
    """The workload's batch and contexts with the decoder backbone: theta
    tuned on an all-local pass to the workload's rate, then warm graph
    replay, against the always-full baseline."""
    from conditional_sparse_attention_amd.step import match_rate, tune_theta
    K = args.steps
    S = DecSession(wl.t0, max(K, args.warmup, 1), stream, theta=math.inf)
    scores = torch.zeros((K, wl.batch), dtype=torch.float32, device="cuda")
    flags = torch.zeros((K, wl.batch), dtype=torch.uint8, device="cuda")

    def run_pass(theta):
        S.plan.set_theta(theta)
        S.reset()
        for j in range(K):
            S.step()
            scores[j].copy_(S.bufs.score)
            flags[j].copy_(S.bufs.flag)
        torch.cuda.synchronize()
        return scores.cpu().numpy(), flags.cpu().numpy()

    # theta from an all-local pass, then re-tuned on the ODA step's own trajectory
    rate = wl.rate if wl.rate is not None else 0.0
    theta, n_full, _, passes = match_rate(run_pass, tune_theta(run_pass(math.inf)[0], rate), rate)
    S.plan.set_theta(theta)
    realised = n_full / flags.numel()
    ms = S.warm_ms(K, args.warmup, args.repeats)
    ms_af = S.warm_ms(K, args.warmup, args.repeats, always_full=True)
    sh = S.sh
    print(json.dumps({
        "metric": "ODA decode steps/s with the dense decoder backbone around the path",
        "value": round(1e3 / ms, 2), "unit": "steps/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "dtype": "bf16",
        "data": "synthetic (seeded generator; random-init bf16 decoder weights and fp32 recall head)",
        "config": {"workload": f"{wl.name} + {sh.name} decoder", "layers": sh.layers, "batch": wl.batch,
                   "context": int(wl.t0[0]), "hidden": sh.hidden, "mlp": sh.inter, "vocab": sh.vocab,
                   "recall_rate_target": rate, "recall_rate_realised": realised, "theta": theta,
                   "theta_tuning_passes": 1 + passes,
                   "tokens_per_s": round(1e3 / ms * wl.batch, 1), "timing": "hip-graph replay, median of repeats"},
        "always_full": {"steps_per_s": round(1e3 / ms_af, 2), "ms_per_step": round(ms_af, 4),
                        "oda_speedup": round(ms_af / ms, 3)},
    }), flush=True)


def decoder_cell(ctx, rate, args, stream, torch, cold):
    """Batch 1, context `ctx`, forced rate `rate` (negative: always-full)."""
    import synth
    nsteps = max(args.steps, args.warmup, 1)
    table = synth.forced_rate_flags(3, nsteps, 1, max(rate, 0.0))
    S = DecSession([ctx], nsteps, stream, theta=0.0, force_table=table)
    af = rate < 0
    out = {"context": ctx, "rate": rate if rate >= 0 else "always-full", "steps": args.steps}
    if cold:
        torch.index_select(S.force_dev, 0, (S.bufs.pos[:1] - S.t0[:1]).long(), out=S.bufs.force.unsqueeze(0))
        S.reset()
        torch.cuda.synchronize()
        c0 = time.perf_counter()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            S.step(af)
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - c0) * 1e3 / args.steps
        out.update({"cold_ms_per_step": round(ms, 4), "cold_tokens_per_s": round(1e3 / ms, 2)})
    else:
        ms = S.warm_ms(args.steps, args.warmup, args.repeats, always_full=af)
        out.update({"warm_ms_per_step": round(ms, 4), "warm_tokens_per_s": round(1e3 / ms, 2)})
    return out


def decoder_matrix(args):
    """Batch-1 decoder steps over contexts x forced rates plus always-full,
    warm in this process, first-request in a fresh child per cell."""
    import subprocess
    import torch
    ctxs = [int(x) for x in args.matrix_contexts.split(",") if x]
    rates = [float(x) for x in args.matrix_rates.split(",") if x] + [-1.0]
    cells = []
    stream = torch.cuda.Stream()
    for ctx in ctxs:
        for r in rates:
            with torch.cuda.stream(stream):
                w = decoder_cell(ctx, r, args, stream, torch, cold=False)
            torch.cuda.empty_cache()
            cmd = [sys.executable, os.path.abspath(__file__), "--decoder-cell", f"{ctx}:{r}", "--steps",
                   str(args.steps), "--warmup", str(args.warmup)]
            cp = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
            if cp.returncode != 0:
                raise SystemExit(f"cold decoder cell {ctx}:{r} failed ({cp.returncode}): {cp.stderr[-2000:]}")
            c = json.loads(cp.stdout.strip().splitlines()[-1])
            w.update({k: v for k, v in c.items() if k.startswith("cold")})
            cells.append(w)
            print(json.dumps(w), flush=True)
    for ctx in ctxs:
        base = [c for c in cells if c["context"] == ctx and c["rate"] == "always-full"][0]
        for c in cells:
            if c["context"] == ctx and c["rate"] != "always-full":
                c["warm_speedup_vs_always_full"] = round(c["warm_tokens_per_s"] / base["warm_tokens_per_s"], 3)
                c["cold_speedup_vs_always_full"] = round(c["cold_tokens_per_s"] / base["cold_tokens_per_s"], 3)
    print(json.dumps({"matrix": "ODA decode tokens/s at batch 1 with the Qwen3-1.7B-shaped decoder backbone: "
                                "context x forced rate", "steps": args.steps, "warmup": args.warmup,
                      "repeats": args.repeats, "cells": cells}), flush=True)


HYBRID_PATTERN = "GGGA" * 6


class HybridSession:
    """The attention Session of the hybrid workload (6 attention layers)
    plus the recurrent layers: the state pool with a seeded pre-step state in
    slot 0, its pristine copy for resets, every step's recurrent inputs
    resident in HBM, and one HybridPlan per step."""

    def __init__(self, nsteps, stream, theta):
        import torch
        import synth
        import conditional_sparse_attention_amd as C
        from conditional_sparse_attention_amd.hybrid import GdnBuffers, HybridPlan
        self.torch, self.C = torch, C
        wl = synth.workloads()["hybrid"]
        if nsteps > wl.steps:
            wl = wl.replace(steps=nsteps)
        self.wl = wl
        self.S = Session(wl, nsteps, stream, theta)
        self.sh = synth.GdnShape(layers=18, batch=wl.batch, heads=16, seed=67)
        sh = self.sh
        self.gd = C.make_gdn_dims(sh.layers, sh.batch, sh.heads, sh.d, sh.conv_width)
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
        g0 = GdnBuffers.allocate(self.gd)
        rec, conv = g0.views(self.gd)
        for l in range(sh.layers):
            for b in range(sh.batch):
                S0, c0 = synth.gdn_initial_state(sh, l, b)
                rec[l, b, 0] = dev(S0)
                conv[l, b, 0] = dev(c0.view(np.int16))
            g0.conv_w[l] = dev(synth.gdn_conv_weights(sh, l).view(np.int16))
        self.pool0 = g0.state.clone()
        Lg, B, H, Cc = sh.layers, sh.batch, sh.heads, sh.channels
        z = lambda *s, dt=torch.int16: torch.zeros(s, dtype=dt, device="cuda")
        self.xin = {k: z(nsteps, Lg, B, Cc) for k in ("xL", "xF")}
        self.gin = {k: z(nsteps, Lg, B, H, dt=torch.float32) for k in ("aL", "bL", "aF", "bF")}
        for j in range(nsteps):
            for l in range(Lg):
                for br, (xk, ak, bk) in enumerate((("xL", "aL", "bL"), ("xF", "aF", "bF"))):
                    self.xin[xk][j, l] = dev(synth.gdn_x(sh, l, br, j).view(np.int16))
                    a, bb = synth.gdn_gates(sh, l, br, j)
                    self.gin[ak][j, l] = dev(a)
                    self.gin[bk][j, l] = dev(bb)
        self.g0 = g0
        self.plans = []
        for j in range(nsteps):
            gj = dataclasses.replace(g0, xL=self.xin["xL"][j], xF=self.xin["xF"][j], aL=self.gin["aL"][j],
                                     bL=self.gin["bL"][j], aF=self.gin["aF"][j], bF=self.gin["bF"][j])
            self.plans.append(HybridPlan(self.S.plans[j], self.gd, gj, HYBRID_PATTERN, stream))
        self.flag_all = self.S.flag_all
        torch.cuda.synchronize()

    def reset(self):
        self.S.reset()
        self.g0.state.copy_(self.pool0)
        self.g0.slot.zero_()

    def set_theta(self, theta):
        self.S.set_theta(theta)

    def always_full_step(self, j):
        """Every sequence full: attention over S^F and the recurrent layers'
        full pass for all, no local trial and no recall head."""
        C, p, S = self.C, self.plans[j], self.S
        dp = ctypes.byref(S.dims)
        C.check(p.plan._lib.oda_worklist(dp, self.flag_all.data_ptr(), S.state.pos.data_ptr(), S.ws.data_ptr(),
                                         S.ws.numel(), S.stream.cuda_stream), "oda_worklist")
        fa = self.flag_all.data_ptr()
        for f, args, name in p.full_calls:
            if name == "oda_gdn_step":
                args = tuple(list(args[:5]) + [fa] + list(args[6:]))
            C.check(f(*args), name)
        a = list(p.plan.commit_args)
        a[3] = fa
        C.check(p.plan._lib.oda_commit(*a), "oda_commit")
        C.check(p._lib.oda_gdn_commit(p.gdn_commit_args[0], p.gdn_commit_args[1], fa, p.gdn_commit_args[3]),
                "oda_gdn_commit")

    def warm_ms(self, K, repeats, always_full=False):
        graphs = self.S.capture((lambda j: self.always_full_step(j)) if always_full else
                                (lambda j: self.plans[j].run()), K)
        torch = self.torch
        runs = []
        for _ in range(repeats):
            self.reset()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(self.S.stream)
            for g in graphs:
                g.replay()
            e1.record(self.S.stream)
            torch.cuda.synchronize()
            runs.append(e0.elapsed_time(e1))
        del graphs
        return statistics.median(runs) / K


def hybrid_bench(args, stream, torch):
    """Hybrid backbone (6 attention + 18 recurrent layers, 8 sequences at
    32K): theta tuned on an all-local pass to the pages' hybrid call rate,
    then one graph per step, against always-full."""
    from conditional_sparse_attention_amd.step import match_rate, tune_theta
    K = args.steps
    H = HybridSession(max(K, args.warmup, 1), stream, theta=math.inf)
    S = H.S
    scores = torch.zeros((K, H.wl.batch), dtype=torch.float32, device="cuda")
    flags = torch.zeros((K, H.wl.batch), dtype=torch.uint8, device="cuda")

    def run_pass(theta):
        H.set_theta(theta)
        H.reset()
        for j in range(K):
            H.plans[j].run()
            scores[j].copy_(S.state.score)
            flags[j].copy_(S.state.flag)
        torch.cuda.synchronize()
        return scores.cpu().numpy(), flags.cpu().numpy()

    # theta from an all-local pass, then re-tuned on the ODA step's own trajectory
    theta, n_full, _, passes = match_rate(run_pass, tune_theta(run_pass(math.inf)[0], H.wl.rate), H.wl.rate)
    H.set_theta(theta)
    H.reset()
    realised = n_full / flags.numel()
    assert S.error_bits() == 0, "device error bits set"
    ms = H.warm_ms(K, args.repeats)
    ms_af = H.warm_ms(K, args.repeats, always_full=True)
    sh, wl = H.sh, H.wl
    print(json.dumps({
        "metric": "hybrid-backbone ODA decode steps/s (attention layers on the ODA path, recurrent-state "
                  "transaction)",
        "value": round(1e3 / ms, 2), "unit": "steps/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "dtype": "bf16 attention, fp32 recurrent state",
        "data": "synthetic (seeded generator: KV cache, q/k/v and recurrent-layer inputs, random-init recall head)",
        "config": {"workload": wl.name, "pattern": HYBRID_PATTERN, "attention_layers": wl.layers,
                   "recurrent_layers": sh.layers, "batch": wl.batch, "context": int(wl.t0[0]),
                   "gdn_heads": sh.heads, "head_dim": sh.d, "conv_width": sh.conv_width,
                   "recall_rate_target": wl.rate, "recall_rate_realised": realised, "theta": theta,
                   "theta_tuning_passes": 1 + passes,
                   "tokens_per_s": round(1e3 / ms * wl.batch, 1), "timing": "hip-graph per step, median of repeats"},
        "always_full": {"steps_per_s": round(1e3 / ms_af, 2), "ms_per_step": round(ms_af, 4),
                        "oda_speedup": round(ms_af / ms, 3)},
    }), flush=True)


BF16_MFMA_PEAK_TFS = 2500.0   # MI355X dense bf16 matrix peak
FP32_MFMA_PEAK_TFS = 157.3    # MI355X fp32 matrix peak


def train_head_flops(N, D, T=1024, F=2048):
    """fp32 multiply-add flops of the head step's GEMMs: every forward product
    once more for its weight gradient and once more for its input gradient."""
    fwd = 2 * N * (3 * T * D + 9 * T * T + 2 * (2 * F * T + F * T))
    return 3 * fwd


def train_bench(args, stream, torch):
    """Recall-head training step on the 4 x 2048-position micro-batch:
    oda_train_labels (the LM head's log-sum-exp for both candidates of every
    row) then oda_train_head_step, inputs resident in HBM, HIP events on the
    stream around each call of every timed step."""
    import synth
    import synth.device as sd
    import conditional_sparse_attention_amd as C
    sh = synth.train_shapes()["qwen3-1.7b-8k"]
    N, D, V = sh.rows, sh.hidden, sh.vocab
    t_setup = time.perf_counter()
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    pos, prev, tok, nxt = synth.train_rows(sh)
    hl, hf = synth.train_hidden(sh)
    blob = synth.head_blob(D, sh.head_seed, perturb=True)
    td = C.make_train_dims(N, D, V, lam=sh.lam)
    E = torch.empty((V, D), dtype=torch.int16, device="cuda")
    sd.fill_dec_embed(E, sh.embed_seed)
    head_w = dev(blob)
    d_hl, d_hf = dev(hl.view(np.int16)), dev(hf.view(np.int16))
    d_pos, d_prev, d_tok, d_nxt = dev(pos), dev(prev), dev(tok), dev(nxt)
    gain = torch.zeros(N, dtype=torch.float32, device="cuda")
    label, score = torch.zeros_like(gain), torch.zeros_like(gain)
    valid = torch.zeros(N, dtype=torch.uint8, device="cuda")
    loss = torch.zeros(1, dtype=torch.float32, device="cuda")
    grad = torch.zeros(blob.size, dtype=torch.float32, device="cuda")
    ws = torch.zeros(C.oda_train_workspace_bytes(td), dtype=torch.uint8, device="cuda")
    C.oda_train_workspace_init(td, ws, stream)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    def labels():
        C.oda_train_labels(td, E, d_hl, d_hf, d_nxt, d_pos, gain, label, valid, ws, stream)

    def head():
        C.oda_train_head_step(td, head_w, E, d_hl, d_hf, d_tok, d_prev, gain, label, valid, score, loss, grad, ws,
                              stream)

    for _ in range(args.warmup):
        labels()
        head()
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for j in range(K):
        ev[j][0].record(stream)
        labels()
        ev[j][1].record(stream)
        head()
        ev[j][2].record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - w0) * 1e3 / K
    lab_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    head_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    ms = max(wall_ms, lab_ms + head_ms)
    assert int(ws[:4].view(torch.int32).item()) == 0, "device error bits set"
    nvalid = int(valid.sum().item())
    lse_flops = 2.0 * (2 * N) * V * D
    head_flops = float(train_head_flops(N, D))
    lse_tfs = lse_flops / (lab_ms * 1e-3) / 1e12
    head_tfs = head_flops / (head_ms * 1e-3) / 1e12
    out = {
        "metric": "recall-head training positions/s (labels through the tied LM head + fp32 head forward/backward)",
        "value": round(N / (ms * 1e-3), 1), "unit": "positions/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 LM head, fp32 head", "data": "synthetic (seeded generator: bf16 hidden states, random-init "
        "tied LM head and fp32 recall head)",
        "config": {"workload": sh.name, "rows": N, "sequences": sh.runs, "positions_per_sequence": sh.rows_per_run,
                   "first_position": sh.first_pos, "hidden": D, "vocab": V, "lambda": sh.lam,
                   "valid_rows": nvalid, "loss": round(float(loss.item()), 6)},
        "roofline": {"bound": "mfma", "kernel": "k_lse (oda_train_labels)", "achieved": round(lse_tfs, 1),
                     "peak": BF16_MFMA_PEAK_TFS, "unit": "TFLOP/s", "frac": round(lse_tfs / BF16_MFMA_PEAK_TFS, 4),
                     "traffic": None, "avg_launch_us": round(lab_ms * 1e3, 1),
                     "algorithmic_flops_per_launch": lse_flops,
                     "note": "event pair around oda_train_labels: k_lse plus three row kernels of a few us"},
        "head_step": {"ms": round(head_ms, 4), "flops": head_flops, "achieved_tflops": round(head_tfs, 1),
                      "peak": FP32_MFMA_PEAK_TFS, "frac": round(head_tfs / FP32_MFMA_PEAK_TFS, 4)},
        "labels_ms": round(lab_ms, 4), "wall_ms_per_step": round(wall_ms, 4), "setup_s": round(setup_s, 1),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = train_cpu_baseline(sh, E, blob, hl, hf, pos, prev, tok, nxt)
    print(json.dumps(out), flush=True)


def train_cpu_baseline(sh, E, blob, hl, hf, pos, prev, tok, nxt):
    """The training oracle, untuned, on a bounded sample: the labels of 640
    rows over the whole vocabulary and the head's forward and backward on 4096
    rows, each scaled to the micro-batch's N rows."""
    from oracle import train as T
    from oracle.oda_oracle import bf16_to_f64
    from threadpoolctl import threadpool_info
    N = sh.rows
    Eb = E.cpu().numpy().view(np.uint16)
    nl = 640
    rows = np.arange(N - nl, N)
    c0 = time.perf_counter()
    g, y, v = T.labels(Eb, hl[rows], hf[rows], nxt[rows], pos[rows], sh.lam)
    t_lab = (time.perf_counter() - c0) / len(rows)
    n = 4096
    rows = np.arange(N - n, N)
    P = T.unpack(blob, sh.hidden, 1024, 2048)
    hL = bf16_to_f64(hl[rows])
    Hp = bf16_to_f64(hl[rows - 1])
    Em = bf16_to_f64(Eb[tok[rows]])
    yy = np.resize(y, n)
    c0 = time.perf_counter()
    q, cache = T.head_forward(P, Hp, Em, hL)
    _, dq = T.loss_and_dq(q, yy, np.ones(n, dtype=bool))
    T.head_backward(P, cache, dq)
    t_head = (time.perf_counter() - c0) / n
    step_s = N * (t_lab + t_head)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(N / step_s, 2), "unit": "positions/s", "cores": int(threads), "kind": "oracle",
            "host_cpus": os.cpu_count(), "cpu_model": host_cpu_model(),
            "sample": (f"labels of {nl} rows over {sh.vocab} vocabulary rows ({t_lab * nl:.2f} s), head forward "
                       f"and backward on {n} rows ({t_head * n:.2f} s); scaled to {N} rows"),
            "sample_cpu_s": round(t_lab * nl + t_head * n, 2)}


if __name__ == "__main__":
    main()
