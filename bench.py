#!/usr/bin/env python
"""Throughput of one OasisKV look-ahead sparse-attention decode step of one layer on one MI355X.

A step is the whole path on one batch: score every candidate block against the
min/max key summaries, select the top-K blocks per KV head, build the capped
transfer plan against the resident set, and run sparse attention of the target
queries over the head-wise working set.  By default the step is the pipeline
the OasisKV pages describe (oasis_decode_step_overlapped): the foreground
attention over the blocks resident now runs beside the background look-ahead
(scoring, top-K, plan for the next step), as workgroups of the same two
launches on one stream.  With
--order serial it is oasis_decode_step: plan first, then attention over the
updated table, all on one stream; the JSON line reports that time as well.
Inputs are seeded synthetic tensors already resident in HBM.  Several
independent input sets are rotated step to step so that the 256 MB last-level
cache cannot serve a step from the previous one; each step reads its set's
resident table and writes the update to a scratch table, so every step does
the same work.

Prints one JSON line.  Default workload: the Qwen3-8B attention-layer shape at
32K context (batch 8, 8 KV heads x group 4, K = 128, 128-token window, fetch
ratio 0.05, 1 target + 4 drafts per query head).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse decode steps/s per layer + achieved HBM GB/s (% peak), Qwen3-8B 32K"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published peak
BLOCK_KV_BYTES = 16 * 128 * 2 * 2   # K and V of one 16-token block of one KV head, bf16


def block_kv_bytes(block: int) -> int:
    """K and V of one block of ``block`` tokens of one KV head, bf16."""
    return block * 128 * 2 * 2
SUMMARY_BYTES = 2 * 128 * 2         # min and max of one block, bf16
CALIBRATION_BYTES = 512 << 20       # the --calibrate copy: bytes read and bytes written per copy


def kv_cache_bytes(batch: int, ctx: int, layers: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """KV capacity M_KV(B, L) = B * L * N_layer * 2 * N_kv * d_h * s (xllm-io review, Eq. (1))."""
    return batch * ctx * layers * 2 * kv_heads * head_dim * elem_bytes


def working_set_blocks(w, lens, resident) -> int:
    """Blocks the overlapped step's attention reads: per (sequence, KV head) the
    resident blocks before the first window block plus the window blocks."""
    total = 0
    bs = w.block
    for b in range(w.batch):
        L = int(lens[b])
        w0 = max(0, (L - w.window) // bs)
        nblk = (L + bs - 1) // bs
        r = resident[b]
        total += int(((r >= 0) & (r < w0)).sum()) + w.num_kv_heads * (nblk - w0)
    return total


def algorithmic_bytes(w, lens, table_count) -> dict:
    """Bytes one step must move: candidate summaries, the K/V blocks of every table entry,
    the queries and the output.  Per kernel as well (inputs plus outputs)."""
    import synth
    H, G, Q = w.num_kv_heads, w.group, w.queries
    cand = sum(synth.first_window_block(int(x), w.window, w.block) for x in lens) * H
    blocks = int(table_count) if isinstance(table_count, int) else int(table_count.sum())
    kvb = block_kv_bytes(w.block)
    q_all = w.batch * H * G * Q * 128 * 2
    q_target = w.batch * H * G * 128 * 2
    out = w.batch * H * G * (128 + 1) * 4
    step = cand * SUMMARY_BYTES + blocks * kvb + q_all + out
    # Algorithmic bytes only: the scores, the split partials and the plan's tables are
    # intermediates of the implementation, not of the method, and count as overhead.
    return {
        "step": step,
        "score": cand * SUMMARY_BYTES + q_all,
        "attn_split": blocks * kvb + q_target,
        "launch1": cand * SUMMARY_BYTES + q_all + blocks * kvb,
        "launch2": out,
        "summaries": cand * SUMMARY_BYTES,
        "kv": blocks * kvb,
        "units": {"candidate_block_heads": cand, "table_blocks": blocks},
    }


def percentiles(xs) -> dict:
    """p10, median and p90 of a sample (nearest-rank on the sorted values)."""
    v = sorted(xs)
    pick = lambda p: v[min(len(v) - 1, max(0, math.ceil(p * len(v)) - 1))]
    return {"p10": pick(0.10), "p50": statistics.median(v), "p90": pick(0.90), "n": len(v)}


def copy_bandwidth(torch, dev, nbytes: int = 1 << 30, reps: int = 20) -> float:
    """Achievable HBM GB/s of a plain device-to-device copy: two buffers of nbytes
    each (four times the 256 MB last-level cache), bytes read plus bytes written
    per copy, over reps back-to-back copies timed with events."""
    src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbps = 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbps


# HBM traffic of the overlapped step, measured offline with rocprofv3 byte counters
# (FETCH_SIZE and WRITE_SIZE, one run each, scaled by what they read for the
# --calibrate copy) and kept under profiles/ with a hash of the kernel sources.
# bench.py reports it only while those sources are unchanged.


def step_kernels(oa, d, w) -> tuple:
    """The kernels of the overlapped step's two launches for dims d (launch 1, launch 2)."""
    if oa.overlapped_selects_in_launch1(d):
        return ("step_kernel", "attn_merge_kernel")
    if w.group * w.queries <= 96:
        return ("score_attn_kernel", "select_merge_kernel")
    return ("score_kernel+attn_split_kernel", "select_merge_kernel")


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"overlapped_step_{workload}_traffic.txt")


KERNEL_SOURCES = ("fused.hip", "attention.hip", "score_impl.h", "attention_impl.h", "select_impl.h", "common.h",
                  "launch.h")


def kernel_sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "oasis_score_summaries_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernels: tuple):
    """HBM bytes per launch of each of the step's kernels and per step, from the
    traffic file; None if it is absent, for another workload or other kernels, or
    taken on other kernel sources."""
    try:
        with open(traffic_file(workload)) as f:
            kv = dict(line.split("=", 1) for line in f.read().splitlines()
                      if "=" in line and not line.startswith("#"))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if (kv.get("workload") != workload or kv.get("sources_sha256") != kernel_sources_sha256()
            or kv.get("kernels") != ",".join(kernels)):
        return None
    out = {k: int(kv[f"{k}.traffic_bytes_per_launch"]) for k in kernels}
    out["per_step"] = int(kv["traffic_bytes_per_step"])
    return out


def kernel_matches(full_name: str, kernel: str) -> bool:
    """Whether a demangled dispatch name is liboasis's kernel ``kernel``."""
    import re
    return re.search(rf"(^|\s)oasis::{re.escape(kernel)}[<(]", full_name) is not None


def summarize_counters(fetch_dir: str, write_dir: str, workload: str, command: str, kernels: tuple) -> str:
    """Traffic file text from the counter-collection CSVs of a FETCH_SIZE run and a
    WRITE_SIZE run of ``bench.py --calibrate``: bytes per launch of each of the
    overlapped step's kernels, read plus written, and their sum per step."""
    import csv

    def per_kernel(d, counter):
        vals = {}
        for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
            if r["Counter_Name"] == counter:
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    notes, body = [], []
    per_launch = {k: 0.0 for k in kernels}
    for counter, d, direction in (("FETCH_SIZE", fetch_dir, "read"), ("WRITE_SIZE", write_dir, "written")):
        vals = per_kernel(d, counter)
        copy = [v for v in vals.get("__amd_rocclr_copyBuffer", []) if v > CALIBRATION_BYTES / 1024 / 8]
        if not copy:
            raise SystemExit(f"no calibration copy found in {d}")
        scale = (CALIBRATION_BYTES / 1024) / statistics.mean(copy[:3])
        notes.append(f"# {counter}: {statistics.mean(copy[:3]):.1f} KiB for the calibration copy "
                     f"({CALIBRATION_BYTES >> 20} MiB {direction}) -> scale {scale:.4f}")
        for kernel in kernels:
            xs = [v for name, v_list in vals.items() if kernel_matches(name, kernel) for v in v_list]
            if not xs:
                raise SystemExit(f"no dispatch of {kernel} in {d}")
            per_launch[kernel] += statistics.mean(xs) * 1024 * scale
            notes.append(f"#   {kernel}: {statistics.mean(xs):.1f} KiB per launch over {len(xs)} launches")
            body.append(f"{kernel}.{counter.split('_')[0].lower()}_bytes_per_launch = "
                        f"{int(round(statistics.mean(xs) * 1024 * scale))}")
    head = [f"# HBM traffic of the overlapped step's kernels ({', '.join(kernels)}), per launch and per step",
            f"# command (one run per counter): {command}"]
    body = ([f"kernels = {','.join(kernels)}", f"workload = {workload}",
             f"sources_sha256 = {kernel_sources_sha256()}"] + body +
            [f"{k}.traffic_bytes_per_launch = {int(round(v))}" for k, v in per_launch.items()] +
            [f"traffic_bytes_per_step = {int(round(sum(per_launch.values())))}"])
    return "\n".join(head + notes + body) + "\n"


OCCUPANCY_COUNTERS = ("OccupancyPercent", "MeanOccupancyPerCU", "MfmaUtil", "LDSBankConflict", "SQ_WAVES")


def summarize_occupancy(dirs, workload: str, command: str) -> str:
    """Per-kernel means of rocprofv3's occupancy counters (derived: OccupancyPercent,
    waves resident per CU over the kernel's busy time (MeanOccupancyPerCU), MfmaUtil,
    LDSBankConflict; raw: SQ_WAVES) from the counter-collection CSVs of one or more
    ``--pmc`` runs, as a markdown table for the library's kernels."""
    import csv
    import re

    vals = {}
    for d in dirs:
        for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
            name = r["Kernel_Name"]
            if "oasis::" not in name or r["Counter_Name"] not in OCCUPANCY_COUNTERS:
                continue
            name = re.sub(r"\(.*$", "", re.sub(r"^void ", "", name))
            vals.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    lines = [f"# Occupancy counters per kernel, {workload}",
             "",
             f"Command (one run per counter group): `{command}`",
             "",
             "OccupancyPercent = 400 * SQ_WAVE_CYCLES / GRBM_GUI_ACTIVE / CU_NUM / 32 (waves resident as a "
             "share of 32 per CU); MeanOccupancyPerCU = waves resident per CU, averaged over the kernel's "
             "busy cycles; MfmaUtil = % of SIMD cycles with the MFMA unit busy; LDSBankConflict = % of CU "
             "cycles stalled on LDS bank conflicts; SQ_WAVES = waves launched per dispatch. Means over "
             "the dispatches of each kernel.",
             "",
             "| kernel | dispatches | " + " | ".join(OCCUPANCY_COUNTERS) + " |",
             "|---|---|" + "---|" * len(OCCUPANCY_COUNTERS)]
    for name in sorted(vals):
        c = vals[name]
        n = max(len(v) for v in c.values())
        cells = [f"{statistics.mean(c[k]):.1f}" if k in c else "" for k in OCCUPANCY_COUNTERS]
        lines.append(f"| `{name}` | {n} | " + " | ".join(cells) + " |")
    return "\n".join(lines) + "\n"


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo where there is one)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(w, sets, budget_s: float, overlapped: bool) -> dict:
    """The fp64 oracle on the host: the same step (score, top-K, plan, attention) for
    (sequence, KV head) units, taken from the input sets in turn and round again,
    until ``budget_s`` seconds of oracle work have run, in two modes: as written,
    one unit after another on one core; then the same oracle mapped over the units
    by a pool of worker threads, one per core up to 16 (numpy leaves the
    interpreter lock while it works on arrays), for ``budget_s`` seconds more.
    Rates are scaled to whole steps (all units of one set)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    from oracle import ref

    per_set = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    units = [(i, b, h) for i in range(len(sets)) for (b, h) in per_set]
    scale = 1.0 / math.sqrt(128)
    step = ref.decode_step_overlapped if overlapped else ref.decode_step
    host = [{"lens": st["seq_lens"].cpu(), "res": st["resident"].cpu()} for st in sets]
    workers = max(1, min(16, os.cpu_count() or 1))
    # A unit's device inputs reach the oracle through host buffers allocated once per
    # worker (the copy, then its fp64 form): fresh host arrays for every unit made the
    # process's resident memory grow by about their size per unit with device inputs.
    names = ("q", "summ", "k", "v")
    slots = [[(torch.empty(tuple(sets[0][n][0:1, 0:1].shape), dtype=sets[0][n].dtype),
               torch.empty(tuple(sets[0][n][0:1, 0:1].shape), dtype=torch.float64)) for n in names]
             for _ in range(workers)]

    def unit_inputs(u, slot=0):
        i, b, h = units[u % len(units)]
        st = sets[i]
        xs = []
        for n, (copy, wide) in zip(names, slots[slot]):
            copy.copy_(st[n][b:b + 1, h:h + 1])
            wide.copy_(copy)
            xs.append(wide.numpy())
        return (*xs, host[i]["lens"][b:b + 1].numpy(),
                host[i]["res"][b:b + 1, h:h + 1].numpy().astype(np.int64))

    def run(x):
        step(*x, w.top_k, w.window, w.cap, scale)

    done, elapsed = 0, 0.0
    with threadpool_limits(1):
        while elapsed < budget_s:
            x = unit_inputs(done)              # conversion to fp64 is not timed
            t = time.perf_counter()
            run(x)
            elapsed += time.perf_counter() - t
            done += 1
    per_step = elapsed / done * len(per_set)
    out = {"value": 1.0 / per_step, "unit": "steps/s", "cores": 1, "kind": "oracle",
           "sample": f"{done} (sequence, KV head) units ({done / len(per_set):.2f} steps of "
                     f"{len(per_set)} units, from {len(sets)} input sets in turn), fp64 numpy, "
                     f"{elapsed:.1f} s of oracle time on one core, scaled to steps",
           "cpu": cpu_model(), "host_cpus": os.cpu_count()}

    done_p, elapsed_p = 0, 0.0
    with threadpool_limits(1), ThreadPoolExecutor(workers) as pool:
        while elapsed_p < budget_s:
            chunk = [unit_inputs(done_p + j, j) for j in range(workers)]
            t = time.perf_counter()
            list(pool.map(run, chunk))
            elapsed_p += time.perf_counter() - t
            done_p += len(chunk)
            del chunk
    out["pool"] = {"value": done_p / elapsed_p / len(per_set), "unit": "steps/s", "cores": workers,
                   "kind": "oracle",
                   "sample": f"{done_p} units ({done_p / len(per_set):.2f} steps) over a pool of {workers} "
                             f"threads, {workers} units at a time, {elapsed_p:.1f} s of wall time"}
    return out


def layer_pipelined(d, sets, ms_step: float, torch, oa, reps: int = 100, step_bytes: int = 0,
                    sweeps: int = 1) -> dict:
    """The input sets as the layers of a decode step, each layer's selection and plan
    riding in the next layer's first launch (oasis_decode_layer_pipelined): the
    steady-state time per layer of a whole sweep (graph replay; the first layer of a
    replay selects the previous replay's last layer; a graph holds ``sweeps`` sweeps, and
    about ``reps`` sweeps are timed, in whole graphs).  Every layer still does its whole
    step; only where its selection runs changes.  With ``step_bytes`` (one layer's
    algorithmic bytes) also the per-layer rate against the HBM peak."""
    replays = max(1, reps // sweeps)
    sweep = oa.PipelinedLayers(d, [(s["q"], s["summ"], s["k"], s["v"], s["seq_lens"], s["resident"])
                                   for s in sets])
    for _ in range(3):
        sweep()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sweep()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(sweeps):
            sweep()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (replays * len(sets) * sweeps)
    sweep.drain()
    torch.cuda.synchronize()
    out = {"us_per_layer": round(us, 3), "layers": len(sets), "sweeps_per_graph": sweeps, "layers_per_s": round(1e6 / us, 1),
           "overlapped_step_us": round(ms_step * 1e3, 3)}
    if step_bytes:
        gbps = step_bytes / (us * 1e-6) / 1e9
        out["hbm"] = {"achieved": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4),
                      "bytes_per_layer": step_bytes}
    return out


def transfer_pipeline(d, sets, wsets, hosts, torch, oa, steps: int = 20, streams=None) -> dict:
    """The input sets as the layers of one decode step, the full cache in pinned host
    memory: every layer's step over its working set with the plan's copies on the
    same stream, against the copies on a transfer stream that each layer's next step
    waits for (the pages' per-layer background transfer), and the foreground alone
    (no copies).  Eager launches; per-layer buffers; layer i copies from host buffer
    i mod 2 (the same bytes).  ``streams`` = (foreground, transfer) to reuse across calls
    (new ones otherwise)."""
    dev = torch.device("cuda:0")
    L = len(sets)
    per = []
    for i, (st, ws) in enumerate(zip(sets, wsets)):
        bufs = oa.StepBuffers(d, dev)
        rn = torch.empty_like(st["resident"])
        hk, hv = hosts[i % len(hosts)]
        per.append((oa.PreparedPoolStep(d, st["q"], st["summ"], hk, hv, ws, st["seq_lens"],
                                        st["resident"], bufs, rn),
                    oa.PreparedStep(d, st["q"], st["summ"], st["k"], st["v"], st["seq_lens"],
                                    st["resident"], bufs, resident_next=rn, overlapped=True)))
    fg, tr = streams if streams is not None else (torch.cuda.Stream(), torch.cuda.Stream())
    done = [torch.cuda.Event() for _ in range(L)]

    def run(mode):
        for t in range(steps + 2):                     # two warm-up steps
            if t == 2:
                fg.wait_stream(tr)
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(fg)
            for i, (pool_step, fg_step) in enumerate(per):
                if mode == "serial":
                    pool_step(stream=fg)
                elif mode == "pipelined":
                    fg.wait_event(done[i])
                    pool_step(stream=fg, transfer_stream=tr)
                    done[i].record(tr)
                else:
                    fg_step(stream=fg)
        fg.wait_stream(tr)
        e1.record(fg)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (steps * L)

    for ev in done:
        ev.record(tr)
    res = {"layers": L, "decode_steps": steps}
    for mode in ("foreground_only", "serial", "pipelined"):
        res[f"{mode}_us_per_layer"] = round(run(mode), 3)
    return res


def plan_execution(w, d, sets, buffers, res_next, ms_step: float, stage_us: dict, torch, oa,
                   host_sets: int = 2, reps: int = 40) -> dict:
    """The step over the working set in HBM (attention from the pool and the window
    ring, then the plan's block copies into the pool), with the full cache in HBM
    and in pinned host memory; the copy launch alone; the bulk host-to-device rate;
    and the per-step transfer budget of the pages' Eq. (3) and stage bound of
    Eq. (4).  Repeated steps re-run the same plan, so every step moves the same
    blocks (correctness is the parity tests' business)."""
    dev = torch.device("cuda:0")

    def graph_ms(step_list):
        for i in range(3 * len(step_list)):
            step_list[i % len(step_list)]()
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step_list[0]()
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for st in step_list:
                st()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * len(step_list))

    def launch_us(fn, n=60):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
        for i in range(n):
            evs[2 * i].record()
            fn()
            evs[2 * i + 1].record()
        torch.cuda.synchronize()
        return 1e3 * statistics.mean(evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(n))

    wsets = [oa.fill_working_set(d, s["resident"], s["seq_lens"], s["k"], s["v"]) for s in sets]
    dev_steps = [oa.PreparedPoolStep(d, s["q"], s["summ"], s["k"], s["v"], ws, s["seq_lens"],
                                     s["resident"], buffers, res_next) for s, ws in zip(sets, wsets)]
    out = {"device_tier_ms_per_step": round(graph_ms(dev_steps), 6)}
    # One step of set 0 leaves its plan in the buffers: the copies alone, from HBM.
    dev_steps[0]()
    torch.cuda.synchronize()
    moved = int(buffers.plan_count.sum()) * block_kv_bytes(w.block)
    plan = buffers.plan.clone()
    count = buffers.plan_count.clone()
    copy_dev = oa.PreparedPlanCopy(d, plan, count, sets[0]["k"], sets[0]["v"], wsets[0])
    us_dev = launch_us(copy_dev)
    out["plan_bytes_per_step"] = moved
    out["plan_bytes_cap"] = w.batch * w.num_kv_heads * w.cap * block_kv_bytes(w.block)
    out["copy_device_tier_us"] = round(us_dev, 3)
    out["copy_device_tier_gbps"] = round(moved / (us_dev * 1e-6) / 1e9, 1)
    # The full cache in pinned host memory (first host_sets input sets).
    hosts = [(s["k"].cpu().pin_memory(), s["v"].cpu().pin_memory()) for s in sets[:host_sets]]
    host_steps = [oa.PreparedPoolStep(d, s["q"], s["summ"], hk, hv, ws, s["seq_lens"], s["resident"],
                                      buffers, res_next)
                  for s, ws, (hk, hv) in zip(sets, wsets, hosts)]
    out["host_tier_ms_per_step"] = round(graph_ms(host_steps), 6)
    out["host_tier_input_sets"] = host_sets
    copy_host = oa.PreparedPlanCopy(d, plan, count, hosts[0][0], hosts[0][1], wsets[0])
    us_host = launch_us(copy_host)
    link_gbps = moved / (us_host * 1e-6) / 1e9
    out["copy_host_tier_us"] = round(us_host, 3)
    out["copy_host_tier_gbps"] = round(link_gbps, 2)
    # The same blocks moved by the DMA engine instead of the copy kernel: one
    # host-to-device copy per admitted block, K and V each (here into a staging buffer;
    # the destination does not change what the engine moves).  Every copy is a command
    # of its own (two per admitted block), so the host's submission sets the pace.
    rows, cnt = plan.cpu().reshape(-1, plan.shape[-2], 3), count.cpu().reshape(-1)
    admitted = [(bh // w.num_kv_heads, bh % w.num_kv_heads, int(rows[bh, r, 1]))
                for bh in range(rows.shape[0]) for r in range(int(cnt[bh]))]
    if admitted:
        hk, hv = hosts[0]
        stage = torch.empty((len(admitted), 2) + tuple(hk.shape[3:]), dtype=hk.dtype, device=dev)
        side = torch.cuda.Stream()
        with torch.cuda.stream(side):
            def dma_copies():
                for i, (b, h, j) in enumerate(admitted):
                    stage[i, 0].copy_(hk[b, h, j], non_blocking=True)
                    stage[i, 1].copy_(hv[b, h, j], non_blocking=True)
            dma_copies()
            side.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            e0.record()
            for _ in range(5):
                dma_copies()
            e1.record()
            submit_s = (time.perf_counter() - t0) / 5
            side.synchronize()
        out["dma_per_block"] = {
            "copies_per_step": 2 * len(admitted),
            "us_per_step": round(1e3 * e0.elapsed_time(e1) / 5, 3),
            "host_submit_us_per_step": round(1e6 * submit_s, 1),
            "note": "one torch copy (host-to-device, pinned) per admitted block's K and V; "
                    "the time includes the host's submission of every copy"}
        del stage
    # Bulk host-to-device copy of 1 GiB of pinned memory (the link's streaming rate).
    src = torch.empty(1 << 29, dtype=torch.bfloat16).pin_memory()
    dst = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev)
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(4):
        dst.copy_(src, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    bulk = 4 * (1 << 30) / (e0.elapsed_time(e1) * 1e-3) / 1e9
    out["bulk_h2d_gbps"] = round(bulk, 2)
    out["transfer_pipeline"] = transfer_pipeline(d, sets, wsets, hosts, torch, oa)
    del src, dst, hosts, host_steps
    # Eq. (3): bytes the link can move while one layer's step computes, at the rate the
    # plan's copies reach; Eq. (4): the slowest background stage against that step.
    # Reading of the two equations: the pages' T_decode is the compute time of a whole
    # decode step (every layer) and their per-layer stage budget is T_step / N_layer.
    # This path is one layer, so the layer's own measured step stands for both: the
    # plan's copies for a layer must cross the link within that layer's step.
    t_step = ms_step * 1e-3
    heads = w.batch * w.num_kv_heads
    per_cap_bytes = heads * block_kv_bytes(w.block)          # one more admitted block per head
    budget = link_gbps * 1e9 * t_step
    reading = ("T_decode and the per-layer budget T_step / N_layer are both taken as this one "
               "layer's measured step; the plan's copies of a layer must cross the host link "
               "within it")
    out["eq3"] = {"reading": reading, "link_gbps": round(link_gbps, 2), "t_step_us": round(ms_step * 1e3, 3),
                  "c_token_bytes": int(budget),
                  "plan_bytes_per_step": moved,
                  "fits": bool(moved <= budget),
                  "break_even_layer_us": round(moved / (link_gbps * 1e9) * 1e6, 3),
                  "largest_cap_fitting": int(min(w.top_k, budget // per_cap_bytes)),
                  "cap": w.cap}
    t_pipe = max(stage_us["score"], stage_us["select_plan"], us_host)
    out["eq4"] = {"reading": reading, "t_pred_us": round(stage_us["score"], 3),
                  "t_select_us": round(stage_us["select_plan"], 3),
                  "t_transfer_us": round(us_host, 3), "t_pipe_us": round(t_pipe, 3),
                  "delta_prefetch_us": round(ms_step * 1e3, 3)}
    return out


# (top_k, fetch_ratio, block size): the pages' K and fetch-ratio ablations at 16-token
# blocks, then other block sizes at the same 2048-token budget (K = 2048 / block).
SWEEP = [(64, 0.05, 16), (128, 0.05, 16), (192, 0.05, 16),
         (128, 0.01, 16), (128, 0.02, 16), (128, 0.10, 16), (128, 0.20, 16), (128, 1.0, 16),
         (256, 0.05, 8), (64, 0.05, 32), (32, 0.05, 64)]


def run_sweep(args) -> dict:
    """The pages' ablations at kernel level (K and the fetch ratio) on one workload's
    inputs, and block sizes other than 16 over the same K/V bytes (the tokens are
    contiguous, so a cache of 16-token blocks is one of 8-, 32- or 64-token blocks;
    only the summaries are rebuilt): per variant the overlapped step from the full
    cache in HBM, the step over the working set with the full cache in HBM and in
    pinned host memory (where the fetch ratio sets the bytes crossing the host
    link), and the plan's bytes."""
    import torch

    import oasis_score_summaries_amd as oa
    import synth

    dev = torch.device("cuda:0")
    base = synth.WORKLOADS[args.workload]
    n_sets = args.sets
    sets = []
    for i in range(n_sets):
        inp = synth.generate(base, dev, layer=i)
        d0 = oa.dims_for(base)
        sets.append({"q": inp["q"], "q_sel": inp["q_prev"] if base.resident == "prev" else inp["q"],
                     "k": inp["k"], "v": inp["v"], "seq_lens": inp["seq_lens"],
                     "summ": oa.build_summaries(d0, inp["k"], inp["seq_lens"])})
        del inp
    hosts = [(s["k"].cpu().pin_memory(), s["v"].cpu().pin_memory()) for s in sets[:2]]

    def graph_ms(step_list, reps=30):
        for i in range(3 * len(step_list)):
            step_list[i % len(step_list)]()
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step_list[0]()
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for st in step_list:
                st()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * len(step_list))

    def as_blocks(t, bs):
        return t.view(t.shape[0], t.shape[1], -1, bs, t.shape[-1])

    rows = []
    pipe_streams = (torch.cuda.Stream(), torch.cuda.Stream())   # one pair for every variant
    for top_k, ratio, bs in SWEEP:
        w = base.with_(top_k=top_k, fetch_ratio=ratio, block=bs)
        d = oa.dims_for(w)
        if bs == base.block:
            vsets, vhosts = sets, hosts
        else:
            vsets = [{**st, "k": as_blocks(st["k"], bs), "v": as_blocks(st["v"], bs)} for st in sets]
            for st in vsets:
                st["summ"] = oa.build_summaries(d, st["k"], st["seq_lens"])
            vhosts = [(as_blocks(hk, bs), as_blocks(hv, bs)) for hk, hv in hosts]
        residents = []
        for i, st in enumerate(vsets):
            sel = oa.topk_blocks(d, oa.score_summaries(d, st["q_sel"], st["summ"], st["seq_lens"]),
                                 st["seq_lens"])
            residents.append(synth.resident_from_selection(w, sel, st["seq_lens"].cpu(), layer=i).to(dev))
        bufs = oa.StepBuffers(d, dev)
        rn = torch.empty_like(residents[0])
        over = [oa.PreparedStep(d, st["q"], st["summ"], st["k"], st["v"], st["seq_lens"], r, bufs,
                                resident_next=rn, overlapped=True) for st, r in zip(vsets, residents)]
        ms_over = graph_ms(over)
        wsets = [oa.fill_working_set(d, r, st["seq_lens"], st["k"], st["v"]) for st, r in zip(vsets, residents)]
        pool_dev = [oa.PreparedPoolStep(d, st["q"], st["summ"], st["k"], st["v"], ws, st["seq_lens"], r,
                                        bufs, rn) for st, r, ws in zip(vsets, residents, wsets)]
        ms_pool_dev = graph_ms(pool_dev)
        pool_host = [oa.PreparedPoolStep(d, st["q"], st["summ"], hk, hv, ws, st["seq_lens"], r, bufs, rn)
                     for st, r, ws, (hk, hv) in zip(vsets, residents, wsets, vhosts)]
        ms_pool_host = graph_ms(pool_host, reps=max(3, int(30 * 0.1 / max(ratio, 0.01))))
        moved = 0
        table_blocks = 0
        for st, r in zip(vsets, residents):   # the plan bytes of every set's step
            oa.decode_step_overlapped(d, st["q"], st["summ"], st["k"], st["v"], st["seq_lens"], r, rn,
                                      buffers=bufs)
            moved += int(bufs.plan_count.sum()) * block_kv_bytes(bs)
            table_blocks += working_set_blocks(w, st["seq_lens"].cpu(), r.cpu())
        torch.cuda.synchronize()
        step_bytes = algorithmic_bytes(w, vsets[0]["seq_lens"].cpu(), table_blocks // n_sets)["step"]
        pipe = transfer_pipeline(d, [{**st, "resident": r} for st, r in zip(vsets, residents)], wsets, vhosts,
                                 torch, oa, steps=10, streams=pipe_streams)
        rows.append({"top_k": top_k, "fetch_ratio": ratio, "block_size": bs, "cap": w.cap,
                     "transfer_pipeline_us_per_layer": {k.replace("_us_per_layer", ""): v
                                                     for k, v in pipe.items() if k.endswith("_us_per_layer")},
                     "overlapped_ms_per_step": round(ms_over, 6),
                     "overlapped_steps_per_s": round(1e3 / ms_over, 1),
                     "pool_device_tier_ms_per_step": round(ms_pool_dev, 6),
                     "pool_host_tier_ms_per_step": round(ms_pool_host, 6),
                     "plan_bytes_per_step": moved // n_sets,
                     "overlapped_step_bytes": step_bytes,
                     "overlapped_step_gbps": round(step_bytes / (ms_over * 1e-3) / 1e9, 1),
                     "table_blocks_per_head": top_k + -(-w.window // bs)})
        del over, pool_dev, pool_host, wsets, bufs, residents, vsets
        torch.cuda.empty_cache()
    return {"metric": "variant sweep: step time against top-K, fetch ratio and block size",
            "workload": base.name, "input_sets": n_sets, "host_tier_input_sets": len(hosts),
            "rows": rows, "data": "synthetic"}


def block_shares_gpu(q_true, k, seq_lens, window: int, scale: float, torch):
    """Analysis, not the decode path: each candidate block's share of the true
    query's softmax over all valid tokens, per query head ([B, H, G, NB] fp32, 0
    outside the candidates), in fp32 torch on the device; k is [B, H, NB, bs, 128]."""
    B, H, NB, bs = k.shape[:4]
    G = q_true.shape[2]
    T = NB * bs
    lens = seq_lens.to(torch.int64)
    tok = torch.arange(T, device=k.device)
    blk = torch.arange(NB, device=k.device)
    out = torch.empty((B, H, G, NB), dtype=torch.float32, device=k.device)
    for b in range(B):
        kf = k[b].reshape(H, T, 128).float()                                # [H, T, d]
        qt = q_true[b].float().transpose(-1, -2).contiguous()               # [H, d, G]
        z = torch.matmul(kf, qt).transpose(-1, -2) * scale                  # [H, G, T]
        z = z.masked_fill(tok >= lens[b], float("-inf"))
        p = torch.softmax(z, dim=-1)
        share = p.reshape(H, G, NB, bs).sum(-1)                             # [H, G, NB]
        n_cand = max(0, (int(lens[b]) - window) // bs)
        out[b] = share.masked_fill(blk >= n_cand, 0.0)
    return out


def block_mass_gpu(q_true, k, seq_lens, window: int, scale: float, torch):
    """Each candidate block's share, largest over the group ([B, H, NB] fp32, -inf
    outside the candidates): the definition of the oracle's block_attention_mass."""
    bs = k.shape[3]
    shares = block_shares_gpu(q_true, k, seq_lens, window, scale, torch).amax(2)
    n_cand = ((seq_lens.to(torch.int64) - window).clamp(min=0) // bs)[:, None, None]
    blk = torch.arange(k.shape[2], device=k.device)
    return shares.masked_fill(blk >= n_cand, float("-inf"))


def captured_gpu(shares, selection, seq_lens, window: int, torch):
    """Share of each query head's candidate attention held by the selected blocks,
    averaged over the group ([B, H]): the definition of the oracle's
    captured_attention on shares from block_shares_gpu (block size from the shares'
    candidates: ids past them carry 0)."""
    NB = shares.shape[-1]
    sel = selection.to(torch.int64)
    ok = (sel >= 0) & (sel < NB)
    idx = sel.clamp(0, NB - 1)[:, :, None, :].expand(-1, -1, shares.shape[2], -1)
    got = (torch.gather(shares, -1, idx) * ok[:, :, None, :]).sum(-1)     # [B, H, G]
    tot = shares.sum(-1)
    frac = torch.where(tot > 0, got / torch.where(tot > 0, tot, torch.ones_like(tot)), torch.ones_like(tot))
    return frac.mean(2)


QUALITY_NOISE = (0.1, 0.3, 0.6, 1.0)
QUALITY_BLOCKS = (8, 16, 32, 64)


def prediction_quality(args) -> dict:
    """Synthetic analogue of the pages' Figures 4 and 6: how well the look-ahead
    selection finds the blocks the true next query attends to most.  The true next
    query is the workload's target row; a predictor is a set of query rows scored
    and selected by the library (min/max summaries, max over rows and the group,
    top-K): four drafts bf16(q + s*N(0,1)) ("lookahead"), one such row ("proxy",
    standing in for the previous token's query), both together (the rows the step
    scores), and the true query itself (s = 0: what the summary bound alone loses).
    Reported per noise level s: top-20 accuracy against the 20 largest attention
    shares, top-K agreement with the K largest, and top-K agreement with the set the
    true query itself selects (the same selection fed the true query), averaged over
    heads and layers (the input sets).  Then, per block size at the workload's token
    budget (K = K_16 * 16 / bs, the same K/V bytes viewed as blocks of bs tokens, the
    same noisy rows at s = 0.3): the share of each query head's attention over the
    candidates that the selected blocks hold (captured attention), for the same
    predictors and for the best selection the true shares allow (the K blocks of
    largest share, largest over the group)."""
    import torch

    import oasis_score_summaries_amd as oa
    import synth

    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[args.workload]
    boost = getattr(args, "boost", None)
    if boost is not None:   # sensitivity: a stronger planted shift concentrates the attention
        w = w.with_(boost=float(boost))
    scale = 1.0 / math.sqrt(128)
    K, D = w.top_k, 4
    budget = K * w.block
    gen = torch.Generator(device=dev).manual_seed(20260)
    gen_b = torch.Generator(device=dev).manual_seed(20261)   # the block-size rows' own draws
    acc = {}
    by_block = {}

    def predict(rows, inp, summ):
        Q = rows.shape[3]
        dq = oa.make_dims(w.batch, w.num_kv_heads, w.group, w.max_blocks, Q, K, w.window, w.fetch_ratio)
        sc = oa.score_summaries(dq, rows.contiguous(), summ, inp["seq_lens"])
        return oa.topk_blocks(dq, sc, inp["seq_lens"])

    layers = min(args.sets, w.layers if w.layers > 1 else args.sets)
    for layer in range(layers):
        inp = synth.generate(w, dev, layer=layer)
        d = oa.dims_for(w)
        summ = oa.build_summaries(d, inp["k"], inp["seq_lens"])
        q_true = inp["q"][:, :, :, 0, :]                                    # [B, H, G, d]
        mass = block_mass_gpu(q_true, inp["k"], inp["seq_lens"], w.window, scale, torch)
        true_rank = torch.topk(mass, K, dim=-1).indices.to(torch.int32)
        valid = torch.isfinite(torch.gather(mass, -1, true_rank.long()))
        true_rank = torch.where(valid, true_rank, torch.full_like(true_rank, -1)).cpu().numpy()

        def noisy(n, s, g=gen):
            x = q_true.float().unsqueeze(3).expand(-1, -1, -1, n, -1)
            return (x + s * torch.randn(x.shape, generator=g, device=dev)).to(torch.bfloat16)

        preds = {"exact": predict(q_true.unsqueeze(3), inp, summ)}
        for s in QUALITY_NOISE:
            drafts, proxy = noisy(D, s), noisy(1, s)
            preds[f"lookahead@{s}"] = predict(drafts, inp, summ)
            preds[f"proxy@{s}"] = predict(proxy, inp, summ)
            preds[f"proxy+lookahead@{s}"] = predict(torch.cat([proxy, drafts], dim=3), inp, summ)
        # Block sizes at one token budget, one set of noisy rows.
        s_b = 0.3
        drafts_b, proxy_b = noisy(D, s_b, gen_b), noisy(1, s_b, gen_b)
        rows_b = {"exact": q_true.unsqueeze(3), f"lookahead@{s_b}": drafts_b, f"proxy@{s_b}": proxy_b,
                  f"proxy+lookahead@{s_b}": torch.cat([proxy_b, drafts_b], dim=3)}
        for bs in QUALITY_BLOCKS:
            Kb = budget // bs
            kb = inp["k"].view(w.batch, w.num_kv_heads, -1, bs, 128)
            db = oa.make_dims(w.batch, w.num_kv_heads, w.group, kb.shape[2], 1, Kb, w.window,
                              w.fetch_ratio, block_size=bs)
            summ_b = oa.build_summaries(db, kb, inp["seq_lens"])
            shares = block_shares_gpu(q_true, kb, inp["seq_lens"], w.window, scale, torch)
            best = block_mass_gpu(q_true, kb, inp["seq_lens"], w.window, scale, torch)
            top = torch.topk(best, Kb, dim=-1)
            sels = {"best possible": torch.where(torch.isfinite(top.values), top.indices,
                                                 torch.full_like(top.indices, -1))}
            for name, rows in rows_b.items():
                dq = oa.make_dims(w.batch, w.num_kv_heads, w.group, kb.shape[2], rows.shape[3], Kb,
                                  w.window, w.fetch_ratio, block_size=bs)
                sc = oa.score_summaries(dq, rows.contiguous(), summ_b, inp["seq_lens"])
                sels[name] = oa.topk_blocks(dq, sc, inp["seq_lens"])
            for name, sel in sels.items():
                frac = captured_gpu(shares, sel, inp["seq_lens"], w.window, torch)
                by_block.setdefault(bs, {}).setdefault(name, []).append(float(frac.mean()))
            del summ_b, shares, best
        exact_sel = preds["exact"].cpu().numpy()
        for name, sel in preds.items():
            sel = sel.cpu().numpy()
            heads = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
            t20 = [top_overlap_rows(sel[b, h], true_rank[b, h], 20) for b, h in heads]
            tk = [top_overlap_rows(sel[b, h], true_rank[b, h], K) for b, h in heads]
            ts = [top_overlap_rows(sel[b, h], exact_sel[b, h], K) for b, h in heads]
            a = acc.setdefault(name, {"top20": [], "topk": [], "sel": []})
            a["top20"].append(statistics.mean(t20))
            a["topk"].append(statistics.mean(tk))
            a["sel"].append(statistics.mean(ts))
        del inp, summ, mass
        torch.cuda.empty_cache()
    rows = {name: {"top20_accuracy": round(statistics.mean(v["top20"]), 4),
                   "top20_min_layer": round(min(v["top20"]), 4),
                   "topk_agreement": round(statistics.mean(v["topk"]), 4),
                   "topk_min_layer": round(min(v["topk"]), 4),
                   "agreement_with_true_query_selection": round(statistics.mean(v["sel"]), 4),
                   "selection_min_layer": round(min(v["sel"]), 4)} for name, v in acc.items()}
    captured = {str(bs): {"top_k": budget // bs,
                          "captured_attention": {name: round(statistics.mean(v), 4) for name, v in c.items()},
                          "captured_min_layer": {name: round(min(v), 4) for name, v in c.items()}}
                for bs, c in by_block.items()}
    return {"metric": "look-ahead prediction quality (synthetic analogue)", "workload": w.name,
            "planted_boost": w.boost, "layers": layers, "top_k": K, "drafts": D, "noise_levels": list(QUALITY_NOISE),
            "predictors": rows, "token_budget": budget, "captured_attention_by_block_size": captured,
            "data": "synthetic"}


def top_overlap_rows(pred, true, n: int) -> float:
    """|first n of pred & first n of true| / (the larger of the two counts); rankings
    are block ids, best first, -1 padded."""
    a = {int(x) for x in pred[:n] if x >= 0}
    b = {int(x) for x in true[:n] if x >= 0}
    m = max(len(a), len(b))
    return 1.0 if m == 0 else len(a & b) / m


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="qwen3_8b_32k")
    ap.add_argument("--sets", type=int, default=6, help="independent input sets rotated per step")
    ap.add_argument("--graph-steps", type=int, default=36,
                    help="steps per captured graph, in whole rotations through the input sets (at least "
                         "one): 36, the layers of one decode token of Qwen3-8B")
    ap.add_argument("--mode", choices=("graph", "eager"), default="graph")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time (0: skip)")
    ap.add_argument("--stage-steps", type=int, default=300, help="evented steps for per-kernel times")
    ap.add_argument("--calibrate", action="store_true",
                    help="first copy a 512 MiB device buffer three times (a kernel of known traffic, "
                         "for scaling HBM byte counters)")
    ap.add_argument("--order", choices=("overlapped", "serial"), default="overlapped",
                    help="overlapped: attention over the resident set on one stream while the "
                         "look-ahead plans the next step on another; serial: plan, then attention "
                         "over the updated table on one stream")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the traffic file from two rocprofv3 --pmc runs of "
                         "'bench.py --calibrate' (FETCH_SIZE, then WRITE_SIZE) and exit")
    ap.add_argument("--summarize-occupancy", nargs="+", metavar="PMC_DIR",
                    help="write profiles/occupancy_<workload>.md from rocprofv3 --pmc runs of the "
                         "occupancy counters")
    ap.add_argument("--counter-command", default="", help="the command recorded in the traffic file")
    ap.add_argument("--boost", type=float, default=None,
                    help="with --quality: the planted blocks' key shift in place of the workload's")
    ap.add_argument("--quality", action="store_true",
                    help="print one JSON line with the prediction-quality analogue instead of the benchmark")
    ap.add_argument("--sweep", action="store_true",
                    help="print one JSON line with the K and fetch-ratio sweep instead of the benchmark")
    ap.add_argument("--pipeline-reps", type=int, default=100,
                    help="layer-pipelined sweeps timed (each runs every input set), in whole graphs")
    ap.add_argument("--no-plan-exec", action="store_true",
                    help="skip the working-set measurements (step over the pool, plan copies, host tier)")
    args = ap.parse_args(argv)
    if args.summarize_occupancy:
        text = summarize_occupancy(args.summarize_occupancy, args.workload, args.counter_command)
        path = os.path.join(ROOT, "profiles", f"occupancy_{args.workload}.md")
        with open(path, "w") as f:
            f.write(text)
        print(text)
        return 0
    if args.summarize_counters:
        import oasis_score_summaries_amd as oa
        import synth
        w = synth.WORKLOADS[args.workload]
        text = summarize_counters(*args.summarize_counters, args.workload, args.counter_command,
                                  step_kernels(oa, oa.dims_for(w), w))
        with open(traffic_file(args.workload), "w") as f:
            f.write(text)
        print(text, end="")
        return 0

    if args.steps < 1 or args.warmup < 0 or args.graph_steps < 1:
        print("bench.py needs --steps >= 1, --warmup >= 0 and --graph-steps >= 1", file=sys.stderr)
        return 2
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the decode step of one layer is measured on a single "
              "MI355X and no multi-GPU path is built", file=sys.stderr)
        return 2

    import torch

    import oasis_score_summaries_amd as oa
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.sweep:
        print(json.dumps(run_sweep(args)), flush=True)
        return 0
    if args.quality:
        print(json.dumps(prediction_quality(args)), flush=True)
        return 0
    w = synth.WORKLOADS[args.workload]
    d = oa.dims_for(w)
    n_sets = w.layers if w.layers > 1 else args.sets
    graph_rotations = max(1, args.graph_steps // n_sets)
    if args.calibrate:
        src = torch.ones(CALIBRATION_BYTES // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)          # reads and writes CALIBRATION_BYTES each
        torch.cuda.synchronize()
        del src, dst

    # ---- set-up (untimed): inputs, summaries, resident sets ------------------------
    t_setup = time.perf_counter()
    sets = []
    for i in range(n_sets):
        if n_sets > 1:
            # Progress on stderr (stdout carries only the JSON line): under a counter
            # profiler the set-up of many layers takes minutes.
            print(f"bench: set-up of input set {i + 1}/{n_sets}", file=sys.stderr, flush=True)
        inp = synth.generate(w, dev, layer=i)
        summ = oa.build_summaries(d, inp["k"], inp["seq_lens"])
        q_sel = inp["q_prev"] if w.resident == "prev" else inp["q"]
        sel = oa.topk_blocks(d, oa.score_summaries(d, q_sel, summ, inp["seq_lens"]), inp["seq_lens"])
        resident = synth.resident_from_selection(w, sel, inp["seq_lens"].cpu(), layer=i).to(dev)
        sets.append({"q": inp["q"], "k": inp["k"], "v": inp["v"], "seq_lens": inp["seq_lens"],
                     "summ": summ, "resident": resident})
        del inp, q_sel, sel
    buffers = oa.StepBuffers(d, dev)
    res_next = torch.empty_like(sets[0]["resident"])
    serial_steps = [oa.PreparedStep(d, s["q"], s["summ"], s["k"], s["v"], s["seq_lens"], s["resident"],
                                    buffers, resident_next=res_next) for s in sets]
    over_steps = [oa.PreparedStep(d, s["q"], s["summ"], s["k"], s["v"], s["seq_lens"], s["resident"],
                                  buffers, resident_next=res_next, overlapped=True) for s in sets]
    steps = over_steps if args.order == "overlapped" else serial_steps
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    def timed(step_list):
        """Warm-up, then exactly args.steps timed steps; returns (ms per step, steps,
        wall s, graph or None, per-step spread)."""
        for i in range(args.warmup):
            step_list[i % n_sets]()
        torch.cuda.synchronize()
        graph = rest = None
        n_graph = n_sets * graph_rotations
        reps, n_rest = divmod(args.steps, n_graph)

        def capture(n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(n):
                    step_list[i % n_sets]()
            return g

        if args.mode == "graph":
            # One graph holds graph_rotations rotations through the input sets (one step
            # per set each); replaying it walks the rotation.  A second graph holds the
            # first n_rest steps, so that exactly args.steps steps are timed whatever
            # their number.
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                step_list[0]()
            torch.cuda.current_stream().wait_stream(side)
            graph = capture(n_graph)
            rest = capture(n_rest) if n_rest else None
            torch.cuda.synchronize()
            for _ in range(max(1, args.warmup // n_graph)):
                graph.replay()
            if rest is not None:
                rest.replay()
            torch.cuda.synchronize()
        n = args.steps
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record()
        if graph is not None:
            for _ in range(reps):
                graph.replay()
            if rest is not None:
                rest.replay()
        else:
            for i in range(n):
                step_list[i % n_sets]()
        ev1.record()
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / n
        wall = time.perf_counter() - t0
        # Spread: 300 more replays (graph_rotations rotations through the input sets
        # each) or eager steps, whatever args.steps is, with an event after each; per-step
        # ms of each.
        n_samples = 300
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_samples + 1)]
        evs[0].record()
        for i in range(n_samples):
            if graph is not None:
                graph.replay()
            else:
                step_list[i % n_sets]()
            evs[i + 1].record()
        torch.cuda.synchronize()
        per = n_graph if graph is not None else 1
        spread = [evs[i].elapsed_time(evs[i + 1]) / per for i in range(n_samples)]
        return ms, n, wall, graph, spread

    # ---- the timed region (the chosen order), then the other order for reference ------
    print(f"bench: set-up done in {setup_s:.1f} s; timing", file=sys.stderr, flush=True)
    ms_per_step, n_timed, wall_s, graph, spread = timed(steps)
    check = {}
    if graph is not None:
        # The graph's last step ran set n_sets-1; an eager run of it must give the same bits.
        out_graph, res_graph = buffers.out.clone(), res_next.clone()
        steps[-1]()
        torch.cuda.synchronize()
        check["graph_matches_eager"] = bool(torch.equal(out_graph, buffers.out) and
                                            torch.equal(res_graph, res_next))
    other = "serial" if args.order == "overlapped" else "overlapped"
    ms_other, _, _, _, _ = timed(serial_steps if other == "serial" else over_steps)
    graph_mode = graph is not None
    del graph

    # ---- per-launch times: HIP events around each launch, on the launch stream --------
    def evented(step_list, overlapped):
        """Mean ms between the events around each launch.  Steps are queued in
        batches, each with its own events, and read after one synchronization, so
        that the GPU runs them back to back as in the timed region."""
        batch = 30
        evs = [oa.StageEvents(overlapped=overlapped) for _ in range(batch)]
        acc = {k: [] for k in evs[0].STAGES}
        done = 0
        while done < args.stage_steps:
            n = min(batch, args.stage_steps - done)
            for i in range(n):
                step_list[(done + i) % n_sets](events=evs[i])
            torch.cuda.synchronize()
            for i in range(n):
                for k, v in evs[i].elapsed_ms().items():
                    acc[k].append(v)
            done += n
        return {k: [1e3 * x for x in v] for k, v in acc.items()}

    print("bench: per-launch events", file=sys.stderr, flush=True)
    stage_samples = evented(serial_steps, False)
    stage_samples.update(evented(over_steps, True))
    stage_us = {k: statistics.mean(v) for k, v in stage_samples.items()}
    stage_method = "eager, queued in batches of 30"
    copy_gbps = copy_bandwidth(torch, dev)

    # ---- bytes and roofline ------------------------------------------------------------------
    torch.cuda.synchronize()
    s0 = sets[0]
    if args.order == "overlapped":
        blocks = working_set_blocks(w, s0["seq_lens"].cpu(), s0["resident"].cpu())
    else:
        serial_steps[0]()
        torch.cuda.synchronize()
        blocks = int(buffers.table_count.sum())
    nb = algorithmic_bytes(w, s0["seq_lens"].cpu(), blocks)
    step_gbps = nb["step"] / (ms_per_step * 1e-3) / 1e9
    kernels = step_kernels(oa, d, w)
    if args.order == "overlapped":
        launches = {"launch1": kernels[0], "launch2": kernels[1]}
        traffic = measured_traffic(w.name, kernels)
    else:
        launches = {"score": "score_kernel", "select_plan": "topk_plan_kernel",
                    "attn_split": "attn_split_kernel", "attn_merge": "attn_merge_kernel"}
        traffic = None
    per_launch = {}
    for stage, kernel in launches.items():
        us = stage_us[stage]
        e = {"kernel": kernel, "avg_launch_us": round(us, 3),
             "launch_us": {k: round(v, 3) if isinstance(v, float) else v
                           for k, v in percentiles(stage_samples[stage]).items()}}
        if nb.get(stage):
            gbps = nb[stage] / (us * 1e-6) / 1e9
            e.update({"bytes_per_launch": nb[stage], "achieved_gbps": round(gbps, 1),
                      "frac": round(gbps / HBM_PEAK_GBPS, 4)})
        if traffic is not None and kernel in traffic:
            e["traffic"] = traffic[kernel]
        per_launch[stage] = e
    dominant = max(per_launch, key=lambda k: per_launch[k]["avg_launch_us"])
    check["handoff_status_zero"] = oa.workspace_status(d, buffers.ws) == 0

    result = {
        "metric": METRIC if w.name == "qwen3_8b_32k" else METRIC.replace("Qwen3-8B 32K", w.name),
        "value": round(1e3 / ms_per_step, 2),   # one step = one layer
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": n_timed,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "kv_heads": w.num_kv_heads, "group": w.group,
                   "context": w.ctx, "queries_per_head": w.queries, "top_k": w.top_k,
                   "window_tokens": w.window, "fetch_ratio": w.fetch_ratio, "cap": w.cap,
                   "input_sets": n_sets, "mode": args.mode, "order": args.order,
                   "graph_steps": n_sets * graph_rotations if args.mode == "graph" else None},
        # The whole timed step against HBM: the method's bytes (candidate summaries,
        # the K/V blocks of every table entry, queries, outputs) over the step time.
        "roofline": {"bound": "hbm", "scope": "whole step",
                     "kernels": list(launches.values()),
                     "achieved": round(step_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(step_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic["per_step"] if traffic is not None else None,
                     "bytes_per_step": nb["step"], "units": nb["units"],
                     "copy_gbps": round(copy_gbps, 1),
                     "frac_of_copy": round(step_gbps / copy_gbps, 4)},
        "dominant_kernel": dict(per_launch[dominant], stage=dominant),
        "launches": per_launch,
        "step_ms": {k: round(v, 6) if isinstance(v, float) else v for k, v in percentiles(spread).items()},
        "step_ms_sample": (f"per graph replay ({graph_rotations} rotation(s) through the input sets), divided by its steps"
                           if graph_mode else "per eager step"),
        "stage_us": {k: round(v, 3) for k, v in stage_us.items()},
        "stage_timing": stage_method,
        f"{other}_ms_per_step": round(ms_other, 6),
        "serial_form": ("overlapped launch 1, touched splits redone, merge"
                        if oa.decode_step_redoes_touched_splits(d) else "four kernels"),
        "wall_s": round(wall_s, 3),
        "setup_s": round(setup_s, 1),
        "checks": check,
    }
    print("bench: layer-pipelined sweep", file=sys.stderr, flush=True)
    result["layer_pipelined"] = layer_pipelined(d, sets, ms_per_step, torch, oa, reps=max(1, args.pipeline_reps),
                                                step_bytes=nb["step"], sweeps=graph_rotations)
    if not args.no_plan_exec:
        print("bench: plan execution", file=sys.stderr, flush=True)
        result["plan_execution"] = plan_execution(w, d, sets, buffers, res_next, ms_per_step, stage_us,
                                                  torch, oa)
    if args.cpu_budget > 0:
        print("bench: oracle on the host cores", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, sets, args.cpu_budget, args.order == "overlapped")
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
