#!/usr/bin/env python3
"""Benchmark: effective masked-attention TFLOP/s, forward + backward, on one
MI355X.

A step is one pass of the hot path (forward, backward preprocess, dK/dV
pass, dQ pass) over every (sequence length, mask) pair of the workload.
Plans (mask compilation) are built before the timed region: one mask serves
every layer of a model, so it is compiled once; its build time is reported.

Effective FLOPs count only allowed (i, j) pairs: 4*d per pair per head for
the forward (Q K^T and P V), 10*d for the backward (five products), whatever
the kernels recompute.  Inputs are seeded synthetic N(0, 1) tensors rounded
to bf16, resident in HBM before timing starts.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA, 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
METRIC = "effective masked-attention TFLOP/s fwd+bwd (fraction of bf16 MFMA peak)"

# HBM traffic of the dominant kernel comes from two rocprofv3 counter runs of
# this script (FETCH_SIZE, then WRITE_SIZE) with --copy-calibration-mib: the
# counters of a plain device copy of known size in the same process give the
# scale from counter units to bytes.  --summarize-traffic turns the two
# counter files into TRAFFIC_FILE, tagged with a hash of the kernel's sources;
# the figure is reported only while the sources still hash the same.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_dkdv_dense.json")
TRAFFIC_SOURCES = ["long_context_masked_amd/csrc/bwd.hip", "long_context_masked_amd/csrc/kernels.hpp"]
TRAFFIC_KERNEL = "attn_dkdv_kernel"
COPY_KERNEL_HINT = "copy"

# Algorithmic work per allowed (i, j) pair per query head, in units of d
# flops, of each kernel: forward = Q K^T + P V; dK/dV pass = Q K^T, dO V^T,
# P^T dO, dS^T Q; dQ pass = Q K^T, dO V^T, dS K.  With dQ accumulated in the
# dK/dV pass (attn_bwd_atomic_dq) the whole backward is timed as one
# interval of five products (the "dkdv" entry).
KERNEL_FLOPS_PER_PAIR = {"fwd": 4, "dkdv": 8, "dq": 6}
KERNEL_FLOPS_PER_PAIR_FUSED = {"fwd": 4, "dkdv": 10, "dq": 0}
# MFMA-busy fraction and shader clock of the three main kernels, from one
# rocprofv3 --pmc pass (SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE) over a bench
# step, stored in MFMA_FILE with a hash of the kernels' sources, as for traffic.
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_dense.json")
MFMA_SOURCES = ["long_context_masked_amd/csrc/fwd.hip", "long_context_masked_amd/csrc/bwd.hip",
                "long_context_masked_amd/csrc/kernels.hpp"]
MFMA_KERNELS = {"fwd": "attn_fwd_kernel", "dkdv": "attn_dkdv_kernel", "dq": "attn_dq_kernel"}
N_CU, N_SIMD, BF16_FLOP_PER_CLK_CU, N_XCD = 256, 1024, 4096, 8


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def workload(name, seqs):
    import synthetic as syn
    out = []
    if name == "dense":
        seqs = seqs or [1024, 8192, 16384, 49152]
        for S in seqs:
            for label, spec in syn.config_mask_specs("dense", S):
                out.append((f"S{S // 1024}K_{label}", S, 64, 8, spec))
        desc = ("dense regular masks: B=1, GQA Hq=64/Hkv=8, d=128, bf16, S in {"
                + ", ".join(f"{s // 1024}K" for s in seqs)
                + "} x {FULL, CAUSAL, causal sliding window w=1024}, fwd+bwd")
    elif name == "document":
        for label, spec in syn.config_mask_specs("document"):
            out.append((label, spec["S"], 64, 8, spec))
        desc = "document masks: B=1, S=64K, GQA 64:8, d=128, log-uniform lengths in [256, 16K] (seed 0), FULL and CAUSAL DOCUMENT, fwd+bwd"
    elif name == "hetero":
        for label, spec in syn.config_mask_specs("hetero"):
            out.append((label, spec["S"], 64, 8, spec))
        desc = "heterogeneous masks: B=1, S=32K, GQA 64:8, d=128: PREFIX LM CAUSAL, SHARED QUESTION, GLOBAL SLIDING, CAUSAL BLOCKWISE, fwd+bwd"
    elif name == "tasks":
        for label, spec in syn.config_mask_specs("tasks"):
            out.append((label, spec["S"], 64, 8, spec))
        desc = ("token-level task batches: B=1, S=64K, GQA 64:8, d=128; query shards of 256, 1K "
                "and 4K tokens, each with a causal context uniform in [shard, 4 shard] tokens, fwd+bwd")
    elif name == "variants":
        for label, spec in syn.config_mask_specs("variants"):
            out.append((label, spec["S"], 64, 8, spec))
        desc = ("mask variants: B=1, S=32K, GQA 64:8, d=128: FULL SW w=1024, PREFIX LM DOCUMENT, "
                "BLOCK CAUSAL DOCUMENT (block 1K), bidirectional GLOBAL SLIDING, block-causal "
                "CAUSAL BLOCKWISE, fwd+bwd")
    elif name == "sparse":
        seqs = seqs or [32768, 131072]
        for S in seqs:
            for Hkv, heads in ((8, "gqa"), (64, "mha")):
                for label, spec in syn.config_mask_specs("sparse", S, Hq=64, Hkv=Hkv):
                    out.append((f"S{S // 1024}K_{heads}_{label}", S, 64, Hkv, spec))
        desc = ("block-sparse masks: B=1, d=128, S in {" + ", ".join(f"{s // 1024}K" for s in seqs)
                + "} x {GQA 64:8, MHA 64:64}, bitmap per KV head at 50% density, uniform 64/128 and "
                  "variable blocks")
        if seqs[0] <= 32768:
            # one bitmap per query head under GQA
            offs, bits = syn.uniform_block_bitmap(seqs[0], 128, 64, 0.5, 1)
            out.append((f"S{seqs[0] // 1024}K_gqa_perhead_block128_50", seqs[0], 64, 8,
                        syn.with_bitmap(syn.spec_full(seqs[0]), offs, offs, bits)))
            desc += f"; plus a bitmap per query head under GQA (128 blocks, {seqs[0] // 1024}K)"
        desc += ", fwd+bwd"
    else:
        raise SystemExit(f"unknown workload {name}")
    return out, desc


def cpu_baseline(seconds_min=10.0, seconds_cap=30.0, max_heads=16):
    """The fp64 oracle on the host: forward + backward of query heads at
    S = 8K (one head at a time, each over every dense mask: FULL, CAUSAL,
    causal SW w=1024) until at least seconds_min of work, at most
    seconds_cap."""
    import numpy as np
    import synthetic as syn
    from oracle import attention as ora
    from oracle import masks as om
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    S, d = 8192, 128
    flops, secs, heads, done = 0.0, 0.0, 0, []
    specs = syn.config_mask_specs("dense", S)
    while heads < max_heads and secs < seconds_min:
        x = syn.attention_inputs(1, S, 1, 1, d, seed=heads)
        f = {n: syn.bf16_bits_to_f32(x[n]).astype(np.float64) for n in x}
        for label, spec in specs:
            nnz = om.nnz(spec)
            t0 = time.perf_counter()
            ora.backward(f["q"], f["k"], f["v"], f["do"], spec)
            dt = time.perf_counter() - t0
            flops += 14.0 * d * nnz
            secs += dt
            if heads == 0:
                done.append(label)
            log(f"cpu oracle head {heads} {label}: {dt:.2f} s")
        heads += 1
        if secs > seconds_cap:
            break
    return {"value": round(flops / secs / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"fp64 numpy oracle, forward+backward of {heads} query head(s) at S=8K, d=128, "
                      f"each over masks {done}: {secs:.1f} s, effective flops as for the GPU"}


def merge_rate(lcm, torch, dev, S=16384, Hq=64, d=128, reps=20):
    """HBM rate of the merge of two fp32 partial results into the final bf16
    O and LSE at [1, S, Hq, d] (the partial-attention + merge primitive).
    Algorithmic bytes per (s, h) row: two fp32 O rows and two LSE read, one
    bf16 O row and one LSE written.  HIP events on the launch stream."""
    g = torch.Generator(device=dev).manual_seed(0)
    o1 = torch.randn((1, S, Hq, d), generator=g, device=dev)
    o2 = torch.randn((1, S, Hq, d), generator=g, device=dev)
    l1 = torch.randn((1, Hq, S), generator=g, device=dev)
    l2 = torch.randn((1, Hq, S), generator=g, device=dev)
    o = torch.empty((1, S, Hq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty_like(l1)
    lcm.merge(o1, l1, o2, l2, bf16_out=True, out=o, lse_out=lse)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        lcm.merge(o1, l1, o2, l2, bf16_out=True, out=o, lse_out=lse)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = S * Hq * (2 * d * 4 + 2 * 4 + d * 2 + 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"shape": [1, S, Hq, d], "ms_per_launch": round(ms, 4), "bytes_per_launch": nbytes,
            "achieved_GBps": round(gbs, 1), "peak_GBps": PEAK_HBM_GBS,
            "frac": round(gbs / PEAK_HBM_GBS, 4)}


def reference_gemm(torch, dev, sizes=(8192, 16384)):
    """Rate of the vendor GEMM on this machine, for context beside the kernels'
    rates: torch.matmul of two contiguous n x n bf16 matrices (hipBLASLt),
    HIP events on the current stream.  A plain GEMM has no softmax or mask
    and streams each operand once per output tile; on this chip its rate sits
    well below the nominal peak because the clock drops under full matrix
    load, and the attention kernels meet the same limit."""
    out = {"op": "torch.matmul, bf16 [n, n] x [n, n] (vendor BLAS), HIP events", "tflops": {}}
    stream = torch.cuda.current_stream(dev)
    g = torch.Generator(device=dev).manual_seed(0)
    for n in sizes:
        a = torch.randn((n, n), generator=g, device=dev).to(torch.bfloat16)
        b = torch.randn((n, n), generator=g, device=dev).to(torch.bfloat16)
        for _ in range(3):
            c = a @ b
        reps = max(3, int(4e13 / (2 * n ** 3)))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            c = a @ b
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out["tflops"][str(n)] = round(2 * n ** 3 / (ms * 1e-3) / 1e12, 1)
        del a, b, c
    best = max(out["tflops"].values())
    out["best_tflops"] = best
    out["fraction_of_peak"] = _frac(best)
    return out


def dynamic_rebuild(lcm, torch, dev, tensors_for, reps=20, steps=3):
    """Dynamic block-sparse plans: time of one attn_plan_set_bitmap (the
    device list rebuild, HIP events on the launch stream) against the host
    compile of an ordinary plan for the same bitmap, and the fwd+bwd time on
    the rebuilt lists against the ordinary plan's (the dynamic plan keeps
    its creation-time item order and does not split dK/dV items)."""
    import numpy as np
    import synthetic as syn
    d, out = 128, {}
    cases = [("S32K_gqa_block64_50", 32768, 8, 64, 8), ("S32K_gqa_perhead_block128_50", 32768, 8, 128, 64),
             ("S128K_gqa_block128_50", 131072, 8, 128, 8)]
    stream = torch.cuda.current_stream(dev)
    for label, S, Hkv, blk, heads in cases:
        offs, b1 = syn.uniform_block_bitmap(S, blk, heads, 0.5, seed=1)
        _, b2 = syn.uniform_block_bitmap(S, blk, heads, 0.5, seed=2)
        base = syn.spec_full(S)
        t0 = time.perf_counter()
        static = lcm.Plan(1, S, 64, Hkv, d, syn.with_bitmap(base, offs, offs, b2))
        host_s = time.perf_counter() - t0
        dyn = lcm.Plan(1, S, 64, Hkv, d, dict(syn.with_bitmap(base, offs, offs, b1), dynamic=True))
        dyn.bind(dev)
        static.bind(dev)
        g1 = torch.from_numpy(b1).to(dev)
        g2 = torch.from_numpy(b2).to(dev)
        dyn.set_bitmap(g2)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            dyn.set_bitmap(g1 if i % 2 == 0 else g2)   # ends on b2
        e1.record(stream)
        torch.cuda.synchronize()
        rebuild_ms = e0.elapsed_time(e1) / reps
        tt = tensors_for(S, Hkv)
        ms = {}
        for name, plan in (("dynamic", dyn), ("static", static)):
            o, lse = lcm.fwd(plan, tt["q"], tt["k"], tt["v"], out=tt["o"], lse=tt["lse"])
            lcm.bwd(plan, tt["q"], tt["k"], tt["v"], o, lse, tt["do"], grads=(tt["dq"], tt["dk"], tt["dv"]))
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(steps):
                o, lse = lcm.fwd(plan, tt["q"], tt["k"], tt["v"], out=tt["o"], lse=tt["lse"])
                lcm.bwd(plan, tt["q"], tt["k"], tt["v"], o, lse, tt["do"], grads=(tt["dq"], tt["dk"], tt["dv"]))
            e1.record(stream)
            torch.cuda.synchronize()
            ms[name] = e0.elapsed_time(e1) / steps
        nnz = static.stats["nnz_total"]
        out[label] = {"rebuild_us": round(rebuild_ms * 1e3, 1), "host_plan_ms": round(host_s * 1e3, 1),
                      "fwd_bwd_ms_dynamic": round(ms["dynamic"], 3), "fwd_bwd_ms_static": round(ms["static"], 3),
                      "tflops_dynamic": round(14.0 * d * nnz / (ms["dynamic"] * 1e-3) / 1e12, 1),
                      "tflops_static": round(14.0 * d * nnz / (ms["static"] * 1e-3) / 1e12, 1),
                      "plan_device_MB": round(dyn.device_bytes() / 1e6, 1)}
        log(f"dynamic {label}: {out[label]}")
        del dyn, static, g1, g2
    return out


def sources_sha256(sources=None):
    h = hashlib.sha256()
    for rel in (TRAFFIC_SOURCES if sources is None else sources):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _counter_rows(path, counter):
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                rows.append((r["Kernel_Name"], int(r.get("Dispatch_Id", 0) or 0),
                             float(r["Counter_Value"])))
    return rows


def summarize_traffic(fetch_csv, write_csv, copy_mib, workload_desc, commands):
    """Average HBM bytes per launch of the dominant kernel, from the two
    counter files (values in KiB per dispatch), each scaled by what the same
    counter reads for the calibration copy (copy_mib MiB read, copy_mib MiB
    written)."""
    out = {"kernel": TRAFFIC_KERNEL, "workload": workload_desc, "copy_mib": copy_mib,
           "commands": commands, "source_sha256": sources_sha256(), "sources": TRAFFIC_SOURCES}
    known = copy_mib * 1024.0  # KiB
    for name, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        rows = _counter_rows(path, counter)
        agg = {}
        for kname, did, val in rows:   # sum over counter instances of a dispatch
            agg.setdefault((kname, did), 0.0)
            agg[(kname, did)] += val
        copies = [v for (k, _), v in agg.items() if COPY_KERNEL_HINT in k.lower() and "attn" not in k]
        kern = [v for (k, _), v in agg.items() if TRAFFIC_KERNEL in k]
        if not copies or not kern:
            raise SystemExit(f"{path}: no calibration copy or no {TRAFFIC_KERNEL} dispatches")
        copy_kib = max(copies)
        factor = known / copy_kib
        mean_kib = sum(kern) / len(kern)
        out[name] = {"counter": counter, "copy_kib": round(copy_kib, 1), "factor": round(factor, 4),
                     "kernel_dispatches": len(kern), "kernel_mean_kib_raw": round(mean_kib, 1),
                     "bytes_per_launch": round(mean_kib * factor * 1024.0)}
        # the other main kernels of the same run, for comparison
        for short, kname in MFMA_KERNELS.items():
            vals = [v for (k, _), v in agg.items() if kname in k and "reduce" not in k]
            if vals:
                out.setdefault("per_kernel", {}).setdefault(short, {})[name + "_bytes_per_launch"] = \
                    round(sum(vals) / len(vals) * factor * 1024.0)
    out["bytes_per_launch"] = out["fetch"]["bytes_per_launch"] + out["write"]["bytes_per_launch"]
    return out


def traffic_for(desc):
    """Bytes per launch of the dominant kernel if the stored counters were
    taken on this workload with the current kernel sources, else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != sources_sha256() or t.get("workload") != desc:
        return None
    return t.get("bytes_per_launch")


def _workload_nnz(name, seqs):
    """nnz per case of a workload, from host-only plan creation (no GPU)."""
    import long_context_masked_amd as lcm
    cases, _ = workload(name, seqs)
    return [(label, lcm.Plan(1, S, Hq, Hkv, 128, spec).stats["nnz_total"]) for label, S, Hq, Hkv, spec in cases]


def summarize_mfma(csv_path, workload_name, seqs, workload_desc, commands):
    """Per main kernel, all from one counter run of one bench step: the
    MFMA-busy fraction (busy cycles over all SIMDs divided by the active
    clocks of one XCD times the SIMD count), the shader clock (active clocks
    of one XCD over the dispatch durations), the algorithmic rate of the same
    dispatches (their cases' nnz times the kernel's flops per pair, over the
    summed dispatch durations) and that rate as a fraction of the MFMA peak
    at the measured clock.  Dispatch k of a kernel belongs to case k mod n
    (the bench launches the cases in order, once per step)."""
    nnz = [n for _, n in _workload_nnz(workload_name, seqs)]
    disp = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            key = (r["Kernel_Name"], int(r["Dispatch_Id"]))
            e = disp.setdefault(key, {"t": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
            e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    out = {"workload": workload_desc, "commands": commands, "sources": MFMA_SOURCES,
           "source_sha256": sources_sha256(MFMA_SOURCES), "kernels": {}}
    # the separate dQ pass ran only if its kernel was dispatched
    fused = not any(MFMA_KERNELS["dq"] in k for (k, _) in disp)
    fpp = KERNEL_FLOPS_PER_PAIR_FUSED if fused else KERNEL_FLOPS_PER_PAIR
    out["backward"] = "fused" if fused else "separate"
    for short, name in MFMA_KERNELS.items():
        rows = [e for (k, did), e in sorted(disp.items(), key=lambda kv: kv[0][1])
                if name in k and "reduce" not in k]
        if not rows:
            if short == "dq" and fused:
                continue
            raise SystemExit(f"{csv_path}: no {name} dispatches")
        clk = sum(e["GRBM_GUI_ACTIVE"] for e in rows) / N_XCD   # cycles, per XCD
        busy = sum(e["SQ_VALU_MFMA_BUSY_CYCLES"] for e in rows)
        ns = sum(e["t"] for e in rows)
        flops = sum(fpp[short] * 128 * nnz[i % len(nnz)] for i in range(len(rows)))
        ghz = clk / ns
        rate = flops / ns / 1e3                                 # TFLOP/s
        out["kernels"][short] = {"dispatches": len(rows), "mfma_busy_frac": round(busy / (clk * N_SIMD), 4),
                                 "clock_GHz": round(ghz, 3), "alg_tflops": round(rate, 1),
                                 "frac_at_clock": round(rate / (N_CU * BF16_FLOP_PER_CLK_CU * ghz / 1e3), 4),
                                 "mfma_insts": sum(e.get("SQ_INSTS_MFMA", 0.0) for e in rows)}
    return out


def mfma_for(desc):
    """The stored MFMA counters if taken on this workload with the current
    kernel sources, else None."""
    try:
        with open(MFMA_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != sources_sha256(MFMA_SOURCES) or t.get("workload") != desc:
        return None
    return t["kernels"]


# Every configuration of the target under the same clock as the headline:
# (workload, sequence lengths, warmup steps, timed steps).
WORKLOADS = [
    ("document", None, 1, 3),
    ("hetero", None, 1, 3),
    ("sparse", [32768], 1, 3),
    ("sparse", [131072], 1, 2),
    ("dense", [131072], 1, 2),
]


class Runner:
    """Plans, device tensors and timed steps of one workload's cases."""

    def __init__(self, lcm, torch, dev, cases, device_inputs=False, fused=False):
        import ctypes
        self.lcm, self.torch, self.dev = lcm, torch, dev
        self.fused = fused
        self.fpp = KERNEL_FLOPS_PER_PAIR_FUSED if fused else KERNEL_FLOPS_PER_PAIR
        self.tensors, self.runs, self.plan_secs = {}, [], 0.0
        self.L = lcm._lib
        self.lib = self.L.lib()
        self.P = ctypes.c_void_p
        self.stream = torch.cuda.current_stream(dev)
        d = 128
        for label, S, Hq, Hkv, spec in cases:
            if (S, Hkv) not in self.tensors:
                log(f"inputs S={S} Hkv={Hkv}")
                self.tensors[(S, Hkv)] = self._inputs(S, Hq, Hkv, d, device_inputs)
            t0 = time.perf_counter()
            plan = lcm.Plan(1, S, Hq, Hkv, d, spec)
            self.plan_secs += time.perf_counter() - t0
            plan.bind(dev)
            nws = plan.atomic_workspace_bytes() if fused else plan.workspace_bytes()
            ws = torch.empty(nws + 256, dtype=torch.uint8, device=dev)
            self.runs.append(dict(label=label, S=S, Hq=Hq, Hkv=Hkv, plan=plan, ws=ws,
                                  nnz=plan.stats["nnz_total"], events=[]))
            log(f"plan {label}: nnz {plan.stats['nnz_total']:.4g}, fwd partial tiles "
                f"{plan.stats['fwd_tiles_partial']}, full {plan.stats['fwd_tiles_full']}, "
                f"dK/dV items of {plan.stats['bwd_tile_cols']} keys")

    def _inputs(self, S, Hq, Hkv, d, on_device):
        """Q, K, V, dO ~ N(0, 1) rounded to bf16: from the seeded numpy
        generator the tests use, or (large shapes) torch's seeded generator
        on the GPU, which gives the same distribution without the host's
        minutes of sampling."""
        torch, dev = self.torch, self.dev
        if on_device:
            g = torch.Generator(device=dev).manual_seed(0)
            mk = lambda h: torch.randn((1, S, h, d), generator=g, device=dev).to(torch.bfloat16)
            q, k, v, do = mk(Hq), mk(Hkv), mk(Hkv), mk(Hq)
        else:
            import numpy as np
            import synthetic as syn
            x = syn.attention_inputs(1, S, Hq, Hkv, d, seed=0)
            t = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)
            q, k, v, do = t(x["q"]), t(x["k"]), t(x["v"]), t(x["do"])
        return dict(q=q, k=k, v=v, do=do, o=torch.empty_like(q),
                    lse=torch.empty((1, Hq, S), dtype=torch.float32, device=dev),
                    dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v))

    def step(self, record):
        L, lib, P, torch, stream = self.L, self.lib, self.P, self.torch, self.stream
        sp = P(stream.cuda_stream)
        for r in self.runs:
            tt = self.tensors[(r["S"], r["Hkv"])]
            h = r["plan"].handle
            wptr = r["ws"].data_ptr()
            wptr += (-wptr) % 256
            nws = r["plan"].atomic_workspace_bytes() if self.fused else r["plan"].workspace_bytes()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)] if record else None
            if record:
                ev[0].record(stream)
            L.check(lib.attn_fwd(h, P(tt["q"].data_ptr()), P(tt["k"].data_ptr()), P(tt["v"].data_ptr()),
                                 P(tt["o"].data_ptr()), P(tt["lse"].data_ptr()), sp))
            if record:
                ev[1].record(stream)
            if self.fused:
                # the whole backward with dQ accumulated in the dK/dV pass, timed
                # as one interval (the "dkdv" split)
                if record:
                    ev[2].record(stream)
                L.check(lib.attn_bwd_atomic_dq(h, P(tt["q"].data_ptr()), P(tt["k"].data_ptr()),
                                               P(tt["v"].data_ptr()), P(tt["o"].data_ptr()),
                                               P(tt["lse"].data_ptr()), P(tt["do"].data_ptr()),
                                               P(tt["dq"].data_ptr()), P(tt["dk"].data_ptr()),
                                               P(tt["dv"].data_ptr()), P(wptr), nws, sp))
                if record:
                    ev[3].record(stream)
                    ev[4].record(stream)
                    r["events"].append(ev)
                continue
            L.check(lib.attn_bwd_preprocess(h, P(tt["o"].data_ptr()), P(tt["lse"].data_ptr()),
                                            P(tt["do"].data_ptr()), P(wptr), nws, sp))
            if record:
                ev[2].record(stream)
            L.check(lib.attn_bwd_dkdv(h, P(tt["q"].data_ptr()), P(tt["k"].data_ptr()), P(tt["v"].data_ptr()),
                                      P(tt["lse"].data_ptr()), P(tt["do"].data_ptr()), P(tt["dk"].data_ptr()),
                                      P(tt["dv"].data_ptr()), P(wptr), nws, sp))
            if record:
                ev[3].record(stream)
            L.check(lib.attn_bwd_dq(h, P(tt["q"].data_ptr()), P(tt["k"].data_ptr()), P(tt["v"].data_ptr()),
                                    P(tt["lse"].data_ptr()), P(tt["do"].data_ptr()), P(tt["dq"].data_ptr()),
                                    P(wptr), nws, sp))
            if record:
                ev[4].record(stream)
                r["events"].append(ev)

    def measure(self, steps, warmup):
        """Warmup steps, then `steps` timed steps between two device
        synchronisations; kernel splits from the HIP events on the launch
        stream."""
        import numpy as np
        torch = self.torch
        for _ in range(warmup):
            self.step(False)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step(True)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        d = 128
        kern = {"fwd": 0.0, "pre": 0.0, "dkdv": 0.0, "dq": 0.0}
        alg = {"fwd": 0.0, "dkdv": 0.0, "dq": 0.0}
        launches = {k: 0 for k in kern}
        pre_bytes = eff_fwd = eff_bwd = 0.0
        detail = {}
        for r in self.runs:
            ms = np.zeros(4)
            for ev in r["events"]:
                ms += [ev[j].elapsed_time(ev[j + 1]) for j in range(4)]
            n = len(r["events"])
            for j, key in enumerate(("fwd", "pre", "dkdv", "dq")):
                kern[key] += ms[j] / 1e3
                launches[key] += n
            for key in alg:
                alg[key] += self.fpp[key] * d * r["nnz"] * n
            pre_bytes += 2.0 * r["S"] * r["Hq"] * d * 2 * n + 3.0 * r["S"] * r["Hq"] * 4 * n
            ffl, bfl = 4.0 * d * r["nnz"], 10.0 * d * r["nnz"]
            eff_fwd += ffl * n
            eff_bwd += bfl * n
            detail[r["label"]] = {"fwd_tflops": round(ffl * n / (ms[0] / 1e3) / 1e12, 1),
                                  "bwd_tflops": round(bfl * n / (ms[1:].sum() / 1e3) / 1e12, 1),
                                  "fwd_ms": round(ms[0] / n, 3), "bwd_ms": round(ms[1:].sum() / n, 3)}
            r["events"] = []
        t_fwd, t_bwd = kern["fwd"], kern["pre"] + kern["dkdv"] + kern["dq"]
        value = (eff_fwd + eff_bwd) / wall / 1e12
        return {
            "value": value, "wall": wall, "kern": kern, "alg": alg, "launches": launches,
            "fwd_tflops": eff_fwd / t_fwd / 1e12, "bwd_tflops": eff_bwd / t_bwd / 1e12,
            "kernel_tflops": {k: alg[k] / kern[k] / 1e12 for k in alg if alg[k] > 0},
            "preprocess_GBps": None if self.fused else pre_bytes / kern["pre"] / 1e9, "detail": detail,
        }

    def free(self):
        self.tensors.clear()
        self.runs.clear()
        self.torch.cuda.synchronize()
        self.torch.cuda.empty_cache()


def _frac(x):
    return round(x / PEAK_BF16_TFLOPS, 4)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="dense", choices=["dense", "document", "hetero", "sparse", "variants", "tasks"])
    ap.add_argument("--seqs", default=None,
                    help="comma-separated sequence lengths (dense: default 1024,8192,16384,49152; "
                         "sparse: default 32768,131072; ignored by document and hetero)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--bwd", default="separate", choices=["separate", "atomic"],
                    help="backward: the separate dQ pass (attn_bwd), or dQ accumulated in the "
                         "dK/dV pass with fp32 atomics (attn_bwd_atomic_dq, timed as one interval)")
    ap.add_argument("--bwd-key-tile", type=int, default=0, choices=[0, 64, 128],
                    help="keys per dK/dV work item for every plan (0: each plan chooses)")
    ap.add_argument("--no-workloads", action="store_true",
                    help="default dense run: skip the timing of the other configurations")
    ap.add_argument("--no-dynamic", action="store_true",
                    help="sparse workload: skip the dynamic block-sparse (device list rebuild) figures")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this size before warmup (counter scale)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic file from two counter runs and exit (no GPU)")
    ap.add_argument("--traffic-commands", default="", help="commands recorded in the traffic file")
    ap.add_argument("--summarize-mfma", metavar="PMC_CSV",
                    help="write the MFMA counter file from one counter run of one step and exit (no GPU)")
    args = ap.parse_args()
    seqs = [int(x) for x in args.seqs.split(",") if x] if args.seqs else []
    if args.summarize_mfma:
        _, desc = workload(args.workload, seqs)
        t = summarize_mfma(args.summarize_mfma, args.workload, seqs, desc, args.traffic_commands)
        with open(MFMA_FILE, "w") as f:
            json.dump(t, f, indent=1)
        print(json.dumps(t))
        return
    if args.summarize_traffic:
        _, desc = workload(args.workload, seqs)
        t = summarize_traffic(args.summarize_traffic[0], args.summarize_traffic[1],
                              args.copy_calibration_mib, desc, args.traffic_commands)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(t, f, indent=1)
        print(json.dumps(t))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import long_context_masked_amd as lcm

    dev = torch.device("cuda:0")
    cases, desc = workload(args.workload, seqs)
    fused = args.bwd == "atomic"
    key_tile = 128 if fused else args.bwd_key_tile  # the fused dQ pass runs on 128-key items
    if key_tile:
        cases = [(label, S, Hq, Hkv, dict(spec, bwd_key_tile=key_tile)) for label, S, Hq, Hkv, spec in cases]
        desc += f"; dK/dV items of {key_tile} keys"
    run = Runner(lcm, torch, dev, cases, fused=fused)

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy of {args.copy_calibration_mib} MiB done")
        del src, dst

    log(f"warmup {args.warmup}, timing {args.steps} steps")
    m = run.measure(args.steps, args.warmup)
    kern, alg = m["kern"], m["alg"]
    dom = max(("fwd", "dkdv", "dq"), key=lambda k: kern[k])
    achieved = alg[dom] / kern[dom] / 1e12
    out = {
        "metric": METRIC,
        "value": round(m["value"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["wall"] / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": desc, "global_batch": 1, "seq_len": max(r["S"] for r in run.runs),
                   "cases": [r["label"] for r in run.runs]},
        "fraction_of_peak": _frac(m["value"]),
        "fwd": {"tflops": round(m["fwd_tflops"], 2), "fraction_of_peak": _frac(m["fwd_tflops"])},
        "bwd": {"tflops": round(m["bwd_tflops"], 2), "fraction_of_peak": _frac(m["bwd_tflops"]),
                "preprocess_GBps": m["preprocess_GBps"] and round(m["preprocess_GBps"], 1)},
        "backward": ("dQ accumulated in the dK/dV pass with fp32 atomics, then converted "
                     "(attn_bwd_atomic_dq)" if fused else "separate dQ pass (attn_bwd)"),
        "kernel_ms_per_launch": {k: round(kern[k] / m["launches"][k] * 1e3, 4) for k in kern},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": _frac(achieved),
                     "traffic": traffic_for(desc) if dom == "dkdv" else None},
        "kernel_tflops": {k: round(v, 2) for k, v in m["kernel_tflops"].items()},
        "plan_build_s": round(run.plan_secs, 3),
        "detail": m["detail"],
    }
    mf = mfma_for(desc)
    if mf:
        # from one rocprofv3 counter run of one step of this workload (another
        # process, same sources): MFMA-busy fraction, clock, and that run's
        # own algorithmic rate against the peak at its clock
        out["mfma_profile"] = {k: {n: v[n] for n in ("mfma_busy_frac", "clock_GHz", "alg_tflops", "frac_at_clock")
                                   if n in v} for k, v in mf.items()}
        out["roofline"]["mfma_busy_frac_profile"] = mf[dom]["mfma_busy_frac"]
    run.free()
    log("merge of partial results")
    out["merge"] = merge_rate(lcm, torch, dev)
    log("reference GEMM")
    out["reference_gemm"] = reference_gemm(torch, dev)
    out["roofline"]["frac_of_reference_gemm"] = round(achieved / out["reference_gemm"]["best_tflops"], 4)
    if args.workload == "sparse" and not args.no_dynamic:
        log("dynamic block-sparse: device list rebuild")
        dyn_run = Runner(lcm, torch, dev, [])

        def tensors_for(S, Hkv):
            if (S, Hkv) not in dyn_run.tensors:
                dyn_run.tensors[(S, Hkv)] = dyn_run._inputs(S, 64, Hkv, 128, True)
            return dyn_run.tensors[(S, Hkv)]
        out["dynamic"] = dynamic_rebuild(lcm, torch, dev, tensors_for)
        dyn_run.free()
    if args.workload == "dense" and not seqs and not args.no_workloads:
        out["workloads"] = {}
        for name, wseqs, wwarm, wsteps in WORKLOADS:
            wcases, wdesc = workload(name, wseqs)
            key = name + ("_" + "_".join(f"{s // 1024}K" for s in wseqs) if wseqs else "")
            log(f"workload {key}: {len(wcases)} cases, warmup {wwarm}, {wsteps} timed steps")
            wr = Runner(lcm, torch, dev, wcases, device_inputs=True, fused=fused)
            wm = wr.measure(wsteps, wwarm)
            out["workloads"][key] = {
                "config": wdesc, "steps": wsteps, "warmup": wwarm,
                "inputs": "N(0,1) rounded to bf16, torch CUDA generator seed 0",
                "plan_build_s": round(wr.plan_secs, 2),
                "tflops": round(wm["value"], 2), "fraction_of_peak": _frac(wm["value"]),
                "ms_per_step": round(wm["wall"] / wsteps * 1e3, 3),
                "fwd": {"tflops": round(wm["fwd_tflops"], 2), "fraction_of_peak": _frac(wm["fwd_tflops"])},
                "bwd": {"tflops": round(wm["bwd_tflops"], 2), "fraction_of_peak": _frac(wm["bwd_tflops"])},
                "kernel_tflops": {k: round(v, 2) for k, v in wm["kernel_tflops"].items()},
                "detail": wm["detail"],
            }
            log(f"workload {key}: {out['workloads'][key]['tflops']} TFLOP/s "
                f"(fwd {out['workloads'][key]['fwd']['tflops']}, bwd {out['workloads'][key]['bwd']['tflops']})")
            wr.free()
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
