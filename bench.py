"""Benchmark: attention TFLOP/s (forward + backward, SWA+sink and global layers) on the 32768-token THD batch.

One step = the whole hot path of one training pass over the synthetic batch: the sliding-window layer
(64 Q / 8 KV heads, window 128, sink, RoPE base 1e4) forward and backward, then the global layer (64 Q /
4 KV heads, causal, base 1e7) forward and backward, with dO ~ N(0,1).  Inputs are resident in HBM before
the timed region.  FLOPs are algorithmic: attended (query, key) pairs x 640 (forward) and x 1664 (backward).

The decode step (batch 64, SWA ring of 128 + sink; global cache lengths in [8192, 131072]) is timed in the
same run and reported as GB/s of cache traffic under "decode"; the prefill forward alone ("prefill") and a
prefill of 16 chunks over cached prefixes ("prefill_cached"), the step at the per-GPU shapes of a 4-way head
split ("tp4_shard_step"), a decode against one 1,048,576-row cache ("decode_1m") and decode plus 8-token verify
over a paged cache ("paged") likewise.  None of them is
part of the step's value.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-decode] [--step-only]

HBM traffic of the kernels (the roofline's "traffic") is taken with two rocprofv3 counter passes over
`--traffic-probe` (one warm step plus a plain 1 GiB copy that calibrates the counters), then summarised:

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d D1 -o p -- python3 bench.py --traffic-probe D1
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d D2 -o p -- python3 bench.py --traffic-probe D2
    python bench.py --traffic-summary D1 D2      # writes profiles/traffic.json
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

MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
HBM_PEAK_GBS = 8000.0              # MI355X HBM3E, published
FWD_FLOP_PER_PAIR = 2 * (192 + 128)
BWD_FLOP_PER_PAIR = 2 * (3 * 192 + 2 * 128)
# per-kernel algorithmic work: the dK/dV kernel does S, dP, dV, dK (2*(192+128+128+192) per pair); the dQ
# kernel's new work is dQ (2*192 per pair; its S and dP are recomputation)
KERNEL_FLOP_PER_PAIR = {"attn_fwd": FWD_FLOP_PER_PAIR, "bwd_dkdv": 2 * (192 + 128 + 128 + 192), "bwd_dq": 2 * 192,
                        "bwd_dq_ds": 2 * 192}


def pairs_per_head(lengths, window):
    tot = 0
    for L in lengths:
        if window < 0 or L <= window + 1:
            tot += L * (L + 1) // 2
        else:
            tot += (window + 1) * L - window * (window + 1) // 2
    return tot


def code_only(text):
    """C++ source with comments and whitespace removed (string literals kept as they are)."""
    import re

    pat = re.compile(r'"(?:\\.|[^"\\])*"|//[^\n]*|/\*.*?\*/', re.S)
    text = pat.sub(lambda m: m.group(0) if m.group(0).startswith('"') else " ", text)
    return re.sub(r"\s+", "", text)


def kernel_source_hash(csrc=None):
    """Hash of the kernel sources' code (comments and whitespace do not count): the traffic counters in
    profiles/traffic.json stand only for the code they were taken on."""
    h = hashlib.sha256()
    csrc = csrc or os.path.join(ROOT, "global_gqa_attention_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp")):
            h.update(f.encode() + b"\0" + code_only(open(os.path.join(csrc, f)).read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary, if it was taken on the
    current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None
    if data.get("source_hash") != kernel_source_hash():
        return None
    rec = data.get("kernels", {}).get(kernel)
    return None if rec is None else rec.get("bytes_per_launch")


def cpu_info():
    """Host CPUs as the OS reports them and the CPU model name (from /proc/cpuinfo)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"host_cpus": os.cpu_count(), "cpu_model": model}


def cpu_baseline(thd, dout, nthreads):
    """The fp64 oracle, as it stands, on bounded samples of the workloads (about 20-30 s on 16 host threads),
    each reported in GFLOP/s with the same algorithmic FLOP count as the GPU lines.  `value` is the sample of
    the benchmarked step (the first two sequences of the 32K batch, both layers, forward and backward, all 64
    heads); the other configurations are timed beside it:
      swa_512     one 512-token sliding-window layer, forward and backward, every row
      global_2x4096  the 2 x 4096 global forward on the last 256 tokens of each sequence (its costliest rows)
      decode_swa  the batch-64 ring-cache decode step, every (sequence, head) row
      decode_global  the global decode step on 2 sequences drawn by the same recipe (seed 3, batch 2)."""
    import numpy as np
    import torch

    import mimo_inputs as mi
    import oracle

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    configs = {}
    flops, secs, parts = 0.0, 0.0, []
    for name, d, n_tok, lens in (
        ("swa", thd["swa"], sum(thd["swa"]["lengths"][:2]), thd["swa"]["lengths"][:2]),
        ("glb", thd["glb"], sum(thd["glb"]["lengths"][:2]), thd["glb"]["lengths"][:2]),
    ):
        q, k, v = d["q"][:n_tok], d["k"][:n_tok], d["v"][:n_tok]
        cu = mi.cu_from_lengths(lens)
        dO = dout[:n_tok]

        def fb():
            o, _ = oracle.prefill(q, k, v, d["sink"], cu, d["window"], d["rope_base"], nthreads=nthreads)
            og = torch.from_numpy(o).to(torch.bfloat16)
            oracle.prefill_bwd(q, k, v, d["sink"], dO, cu, d["window"], d["rope_base"], out_given=og,
                               nthreads=nthreads)
        dt = timed(fb)
        f = pairs_per_head(lens, d["window"]) * q.shape[1] * (FWD_FLOP_PER_PAIR + BWD_FLOP_PER_PAIR)
        flops += f
        secs += dt
        parts.append(f"{name}: {n_tok} tokens x 64 heads fwd+bwd in {dt:.1f}s")
        configs[f"thd_32k_{name}_fwd_bwd_2seq"] = {"s": round(dt, 2), "GFLOP/s": round(f / dt / 1e9, 2)}

    d = mi.swa_512()
    dO = mi.dout_like(512, 4)
    holder = {}
    dt_f = timed(lambda: holder.setdefault("o", oracle.prefill(d["q"], d["k"], d["v"], d["sink"], d["cu_seqlens"],
                                                                128, 1e4, nthreads=nthreads)))
    og = torch.from_numpy(holder["o"][0]).to(torch.bfloat16)
    dt_b = timed(lambda: oracle.prefill_bwd(d["q"], d["k"], d["v"], d["sink"], dO, d["cu_seqlens"], 128, 1e4,
                                            out_given=og, nthreads=nthreads))
    p = pairs_per_head([512], 128) * 64
    configs["swa_512"] = {"fwd_s": round(dt_f, 3), "fwd_GFLOP/s": round(p * FWD_FLOP_PER_PAIR / dt_f / 1e9, 2),
                          "bwd_s": round(dt_b, 3), "bwd_GFLOP/s": round(p * BWD_FLOP_PER_PAIR / dt_b / 1e9, 2)}

    d = mi.global_2x4096()
    rows = np.concatenate([np.arange(t * 64, (t + 1) * 64) for s0 in (0, 4096) for t in range(s0 + 3840, s0 + 4096)])
    dt = timed(lambda: oracle.prefill_rows(d["q"], d["k"], d["v"], None, d["cu_seqlens"], -1, 1e7, rows=rows,
                                           nthreads=nthreads))
    p = 2 * sum(i + 1 for i in range(3840, 4096)) * 64
    configs["global_2x4096_fwd_last256"] = {"s": round(dt, 2), "GFLOP/s": round(p * FWD_FLOP_PER_PAIR / dt / 1e9, 2)}

    d = mi.decode_swa()
    dt = timed(lambda: oracle.decode_rows(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["cu_cache"],
                                          d["positions"], d["sink"], d["window"], d["rope_base"], nthreads=nthreads))
    p = 64 * 64 * 129
    configs["decode_swa"] = {"s": round(dt, 3), "GFLOP/s": round(p * FWD_FLOP_PER_PAIR / dt / 1e9, 2)}
    d = mi.decode_global(batch=2)
    cuc = d["cu_cache"]
    rows_c = int(cuc[-1])
    dt = timed(lambda: oracle.decode_rows(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], cuc,
                                          d["positions"], None, -1, 1e7, nthreads=nthreads))
    p = (rows_c + 2) * 64
    configs["decode_global_2seq"] = {"s": round(dt, 3), "cache_rows": rows_c,
                                     "GFLOP/s": round(p * FWD_FLOP_PER_PAIR / dt / 1e9, 2),
                                     "GB/s": round(rows_c * 4 * 640 / dt / 1e9, 2)}
    out = {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": nthreads, "kind": "oracle",
           "sample": "; ".join(parts) + " (fp64 C oracle, algorithmic FLOPs as the GPU line)", "configs": configs}
    out.update(cpu_info())
    return out


def run_decode(ga, torch, mi, reps=20):
    res = {}
    for name, gen in (("swa", mi.decode_swa), ("global", mi.decode_global)):
        d = gen(device="cuda")
        cu = d["cu_cache"].cpu()
        lens = (cu[1:] - cu[:-1]).tolist()
        max_len = max(lens)
        ws = torch.empty(ga.decode_workspace_size(64, max_len, 64, d["window"]), dtype=torch.uint8, device="cuda")
        out = torch.empty(64, 64, 128, dtype=torch.bfloat16, device="cuda")
        call = lambda: ga.decode(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["cu_cache"],  # noqa
                                 d["positions"], d["sink"], max_len, d["window"], d["rope_base"], out, ws)
        flush = torch.empty(1 << 29, dtype=torch.uint8, device="cuda")   # 512 MiB: evicts L2 and MALL
        for _ in range(3):
            call()
        times = []
        for _ in range(reps):
            flush.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            call()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        ms = sorted(times)[len(times) // 2]
        hkv = d["n_kv_heads"]
        rows = sum(min(n, d["window"]) if d["window"] >= 0 else n for n in lens)
        cache_bytes = rows * hkv * (192 + 128) * 2
        io_bytes = 64 * 64 * (192 + 128) * 2 + 64 * hkv * (192 + 128) * 2
        pairs = rows * 64 + 64 * 64      # every cached row is seen by all 64 query heads; plus the new token
        res[name] = {"ms": round(ms, 4), "GB/s": round((cache_bytes + io_bytes) / ms / 1e6, 1),
                     "hbm_frac": round((cache_bytes + io_bytes) / ms / 1e6 / HBM_PEAK_GBS, 4),
                     "TFLOP/s": round(pairs * FWD_FLOP_PER_PAIR / ms / 1e9, 2), "cache_rows": rows}
        del d, flush
        torch.cuda.empty_cache()
    return res


def setup_layers(ga, torch, mi, dev):
    """The 32768-token THD batch of both layers, resident on `dev`, with outputs, gradients and workspaces
    allocated; returns (thd on the host, dO on the host, layers, step)."""
    thd = mi.thd_32k()
    dout_cpu = mi.dout_like(32768, 4)
    layers = {}
    for name in ("swa", "glb"):
        d = thd[name]
        g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
        T, hq, hkv = g["q"].shape[0], g["q"].shape[1], g["k"].shape[1]
        g["max_seqlen"] = max(d["lengths"])
        g["out"] = torch.empty(T, hq, 128, dtype=torch.bfloat16, device=dev)
        g["lse"] = torch.empty(hq, T, dtype=torch.float32, device=dev)
        # the forward's rotated q and k, handed to the backward (a training step keeps them like out and lse)
        g["q_rot"] = torch.empty(T, hq, 192, dtype=torch.bfloat16, device=dev)
        g["k_rot"] = torch.empty(T, hkv, 192, dtype=torch.bfloat16, device=dev)
        g["grads"] = (torch.empty_like(g["q"]), torch.empty_like(g["k"]), torch.empty_like(g["v"]),
                      torch.empty(hq, dtype=torch.float32, device=dev) if g["sink"] is not None else None)
        # the workspace that keeps the dS blocks (the dQ kernel reads them back instead of recomputing)
        g["ws"] = torch.empty(ga.bwd_workspace_size(T, hq, hkv, g["window"], len(d["lengths"]), max(d["lengths"])),
                              dtype=torch.uint8, device=dev)
        g["pairs"] = pairs_per_head(d["lengths"], d["window"]) * hq
        layers[name] = g
    dout = dout_cpu.to(dev)
    for g in layers.values():
        g["dout"] = dout

    def step():
        for g in layers.values():
            ga.fwd(g["q"], g["k"], g["v"], g["sink"], g["cu_seqlens"], g["max_seqlen"], g["window"], g["rope_base"],
                   out=g["out"], lse=g["lse"], q_rot=g["q_rot"], k_rot=g["k_rot"])
            ga.bwd(g["q"], g["k"], g["v"], g["sink"], g["out"], g["lse"], dout, g["cu_seqlens"], g["max_seqlen"],
                   g["window"], g["rope_base"], workspace=g["ws"], grads=g["grads"], q_rot=g["q_rot"],
                   k_rot=g["k_rot"])

    return thd, dout_cpu, layers, step


# trace name prefix -> kernel function name (checks that traced launches and counted dispatches line up)
TRACE_TO_KERNEL = (("kv_prep", "kv_prep_kernel"), ("attn_fwd", "attn_fwd_kernel"), ("bwd_prep", "row_prep_kernel"),
                   ("bwd_pre", "bwd_pre_kernel"), ("bwd_dsink", "bwd_dsink_kernel"),
                   ("bwd_ds_index", "bwd_ds_index_kernel"), ("bwd_dq_ds", "bwd_dq_ds_kernel"),
                   ("bwd_dkdv", "bwd_dkdv_kernel"), ("bwd_dkv_reduce", "bwd_dkv_reduce_kernel"),
                   ("bwd_dq", "bwd_dq_kernel"), ("decode_split", "decode_split_kernel"),
                   ("decode_combine", "decode_combine_kernel"))
COPY_BYTES = 1 << 30    # the calibration copy: 1 GiB read, 1 GiB written


def traffic_probe(outdir):
    """One warm step of the hot path and a plain device copy of COPY_BYTES, for rocprofv3 counter passes; the
    library kernels' launch order of the step is written to <outdir>/traffic_order.json."""
    import torch

    import global_gqa_attention_amd as ga
    import mimo_inputs as mi

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    _, _, layers, step = setup_layers(ga, torch, mi, dev)
    step()
    torch.cuda.synchronize()
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    ga.trace_read(clear=True)
    ga.trace_enable(True)
    step()
    torch.cuda.synchronize()
    ga.trace_enable(False)
    names = [n for n, _ in ga.trace_read(clear=True)]
    os.makedirs(outdir, exist_ok=True)
    with open(os.path.join(outdir, "traffic_order.json"), "w") as f:
        json.dump({"launches": names}, f)
    print(f"traffic probe: {len(names)} library launches in the step", flush=True)


def _counter_rows(d, counter):
    """(kernel name, value) per dispatch, in dispatch order, from a rocprofv3 counter_collection.csv."""
    import csv

    path = None
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith("counter_collection.csv"):
                path = os.path.join(root, f)
    if path is None:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        key = int(r["Dispatch_Id"])
        name, val = rows.get(key, (r["Kernel_Name"], 0.0))
        rows[key] = (name, val + float(r["Counter_Value"]))
    return [rows[k] for k in sorted(rows)]


def traffic_summary(fetch_dir, write_dir):
    """Writes profiles/traffic.json: per library kernel of the step, HBM bytes per launch read and written,
    each counter (KiB per dispatch) scaled by what it reads for the COPY_BYTES copy."""
    order = json.load(open(os.path.join(fetch_dir, "traffic_order.json")))["launches"]
    out = {"source_hash": kernel_source_hash(), "copy_bytes": COPY_BYTES,
           "commands": [f"cd /tmp && rocprofv3 --pmc {c} --output-format csv -d $REPO/{d} -o p -- python3 "
                        f"$REPO/bench.py --traffic-probe $REPO/{d}"
                        for c, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir))]
           + [f"python bench.py --traffic-summary {fetch_dir} {write_dir}"],
           "note": "bytes = counter (KiB per dispatch) x 1024 x scale; scale = copy_bytes / the counter's reading "
                   "for a plain device copy of copy_bytes in the same run", "kernels": {}}
    per = {}
    for d, counter in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        rows = _counter_rows(d, counter)
        copies = [v for n, v in rows if "copy" in n.lower()]
        if not copies:
            raise SystemExit(f"{counter}: no copy dispatch found")
        scale = COPY_BYTES / (max(copies) * 1024.0)
        out[f"{counter.lower()}_scale"] = round(scale, 5)
        if not 0.25 < scale < 4.0:
            raise SystemExit(f"{counter}: implausible copy calibration {scale}")
        lib = [(n, v) for n, v in rows if "mimo::" in n]
        if len(lib) < len(order):
            raise SystemExit(f"{counter}: {len(lib)} library dispatches, expected at least {len(order)}")
        for name, (kname, v) in zip(order, lib[-len(order):]):
            want = next(k for p, k in TRACE_TO_KERNEL if name.startswith(p))
            if want not in kname:
                raise SystemExit(f"{counter}: launch {name} lines up with dispatch {kname}")
            per.setdefault(name, {}).setdefault(counter, []).append(v * 1024.0 * scale)
    for name, rec in per.items():
        fb = sum(rec["FETCH_SIZE"]) / len(rec["FETCH_SIZE"])
        wb = sum(rec["WRITE_SIZE"]) / len(rec["WRITE_SIZE"])
        out["kernels"][name] = {"fetch_bytes": round(fb), "write_bytes": round(wb), "bytes_per_launch": round(fb + wb)}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(f"wrote {path}")


def _short_kernel(n):
    import re

    m = re.search(r"mimo::\(anonymous namespace\)::(\w+)(<[^>(]*>)?", n)
    return m.group(1) + (m.group(2) or "") if m else n.split("(")[0][-70:]


def _find_csv(d, suffix):
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(root, f)
    raise SystemExit(f"no *{suffix} under {d}")


def stats_summary(trace_dir, title, command, timed):
    """Prints a rocprofv3 kernel trace (kernel_trace.csv under trace_dir) as a short text table: per kernel the
    launches, the average over all of them, the average over the last `timed` launches (the timed steps of a
    bench run; warm-up launches come first), and min / max, in microseconds."""
    import csv

    per = {}
    for r in csv.DictReader(open(_find_csv(trace_dir, "kernel_trace.csv"))):
        per.setdefault(r["Kernel_Name"], []).append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]) -
                                                     int(r["Start_Timestamp"])))
    timed = int(timed)
    total = sum(d for v in per.values() for _, d in v)
    print(f"# {title}\n# command: {command}\n# source: rocprofv3 --kernel-trace (kernel_trace.csv); avg_timed_us = "
          f"average of each kernel's last {timed} launches (the timed steps)\n")
    print(f"{'kernel':56s} {'calls':>6s} {'avg_us':>9s} {'avg_timed_us':>12s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s}")
    for name, v in sorted(per.items(), key=lambda kv: -sum(d for _, d in kv[1])):
        v.sort()
        ds = [d for _, d in v]
        last = ds[-timed:] if len(ds) >= timed else ds
        print(f"{_short_kernel(name)[:56]:56s} {len(ds):6d} {sum(ds) / len(ds) / 1e3:9.1f} "
              f"{sum(last) / len(last) / 1e3:12.1f} {min(ds) / 1e3:9.1f} {max(ds) / 1e3:9.1f} "
              f"{100.0 * sum(ds) / total:6.2f}")


def mfma_summary(pmc_dir, title, command):
    """Per library kernel of the traced step of --traffic-probe (rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16
    SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE --kernel-trace): bf16 MFMA flops executed (MOPS x 512), the
    MFMA-busy share of the SIMD cycles, the clock implied by GRBM_GUI_ACTIVE over the kernel's traced duration,
    and the executed MFMA rate.  rocprofv3 reports GRBM_GUI_ACTIVE summed over the XCDs (Num_Xcc in the agent
    file), so one XCD's busy cycles are that sum / Num_Xcc; busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x SIMDs).
    Prints a text table."""
    import csv

    nxcc, nsimd = 8, 1024
    try:
        for a in csv.DictReader(open(_find_csv(pmc_dir, "agent_info.csv"))):
            if a.get("Name", "").startswith("gfx"):
                nxcc, nsimd = int(a["Num_Xcc"]), int(a["Simd_Count"])
    except (SystemExit, KeyError, ValueError):
        pass

    order = json.load(open(os.path.join(pmc_dir, "traffic_order.json")))["launches"]
    vals = {}
    for r in csv.DictReader(open(_find_csv(pmc_dir, "counter_collection.csv"))):
        key = int(r["Dispatch_Id"])
        rec = vals.setdefault(key, {"name": r["Kernel_Name"]})
        c, v = r["Counter_Name"], float(r["Counter_Value"])
        rec[c] = max(rec.get(c, 0.0), v) if c == "GRBM_GUI_ACTIVE" else rec.get(c, 0.0) + v
    dur = {}
    for r in csv.DictReader(open(_find_csv(pmc_dir, "kernel_trace.csv"))):
        dur[int(r["Dispatch_Id"])] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    lib = [k for k in sorted(vals) if "mimo::" in vals[k]["name"]]
    if len(lib) < len(order):
        raise SystemExit(f"{len(lib)} library dispatches with counters, expected at least {len(order)}")
    print(f"# {title}\n# command: {command}\n# MFMA flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; cycles = "
          f"GRBM_GUI_ACTIVE / {nxcc} XCDs; busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x {nsimd} SIMDs); clock = cycles / "
          f"traced duration; durations and clocks are those of the counter run, which runs the kernels serialised "
          f"and slower than a plain run (compare the kernel-trace summary)\n")
    print(f"{'launch':24s} {'kernel':34s} {'us':>9s} {'MFMA_TFLOP':>11s} {'TFLOP/s':>9s} {'mfma_busy%':>10s} {'GHz':>6s}")
    for name, k in zip(order, lib[-len(order):]):
        rec = vals[k]
        want = next(kn for pfx, kn in TRACE_TO_KERNEL if name.startswith(pfx))
        if want not in rec["name"]:
            raise SystemExit(f"launch {name} lines up with dispatch {rec['name']}")
        us = dur.get(k, 0) / 1e3
        flop = rec.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512
        gui = rec.get("GRBM_GUI_ACTIVE", 0.0) / nxcc
        busy = 100.0 * rec.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (gui * nsimd) if gui else 0.0
        ghz = gui / (us * 1e3) if us else 0.0
        rate = flop / (us * 1e-6) / 1e12 if us else 0.0
        print(f"{name:24s} {_short_kernel(rec['name'])[:34]:34s} {us:9.1f} {flop / 1e12:11.4f} {rate:9.1f} "
              f"{busy:10.1f} {ghz:6.2f}")


def run_prefill(ga, torch, layers, reps=10):
    """Prefill (inference) forward of each layer alone, without the training-only rotated-q output: median
    per-launch times of its kernels over `reps` calls, algorithmic FLOPs and the forward kernel's algorithmic
    HBM bytes (q and K/V read once, out and LSE written once)."""
    res = {}
    for lname, g in layers.items():
        T, hq, hkv = g["q"].shape[0], g["q"].shape[1], g["k"].shape[1]
        ws = torch.empty(ga.fwd_workspace_size(T, hq, hkv, g["window"]), dtype=torch.uint8, device=g["q"].device)
        call = lambda: ga.fwd(g["q"], g["k"], g["v"], g["sink"], g["cu_seqlens"], g["max_seqlen"], g["window"],
                              g["rope_base"], out=g["out"], lse=g["lse"], workspace=ws)
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        ga.trace_read(clear=True)
        ga.trace_enable(True)
        for _ in range(reps):
            call()
        torch.cuda.synchronize()
        ga.trace_enable(False)
        per = {}
        for name, ms in ga.trace_read(clear=True):
            per.setdefault(name.rsplit("_", 1)[0], []).append(ms)
        med = {k: sorted(v)[len(v) // 2] for k, v in per.items()}
        attn = med.get("attn_fwd", 0.0)
        total = attn + med.get("kv_prep", 0.0)
        flop = g["pairs"] * FWD_FLOP_PER_PAIR
        hbm = T * hq * (2 * 192 + 2 * 128 + 4) + T * hkv * 2 * (192 + 128)
        res[lname] = {"ms": round(total, 4), "attn_fwd_ms": round(attn, 4),
                      "TFLOP/s": round(flop / (total * 1e-3) / 1e12, 1),
                      "frac_of_mfma_peak": round(flop / (total * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                      "attn_fwd_TFLOP/s": round(flop / (attn * 1e-3) / 1e12, 1),
                      "attn_fwd_GB/s": round(hbm / (attn * 1e-3) / 1e9, 1),
                      "attn_fwd_hbm_frac": round(hbm / (attn * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    return res


def run_bwd_paths(ga, torch, layers, reps=10):
    """Backward of each layer with the stored-dS workspace (the step's) and with the least workspace (the dQ
    kernel recomputes S and dP): median of `reps` traced calls, sum of the backward's kernels."""
    res = {}
    for lname, g in layers.items():
        T, hq, hkv = g["q"].shape[0], g["q"].shape[1], g["k"].shape[1]
        least = torch.empty(ga.bwd_workspace_size(T, hq, hkv, g["window"]), dtype=torch.uint8, device=g["q"].device)
        rec = {}
        for path, ws in (("stored_dS", g["ws"]), ("least", least)):
            call = lambda: ga.bwd(g["q"], g["k"], g["v"], g["sink"], g["out"], g["lse"], g["dout"], g["cu_seqlens"],  # noqa
                                  g["max_seqlen"], g["window"], g["rope_base"], workspace=ws, grads=g["grads"],
                                  q_rot=g["q_rot"], k_rot=g["k_rot"])
            for _ in range(2):
                call()
            torch.cuda.synchronize()
            ga.trace_read(clear=True)
            ga.trace_enable(True)
            totals = []
            for _ in range(reps):
                call()
                torch.cuda.synchronize()
                totals.append(sum(ms for _, ms in ga.trace_read(clear=True)))
            ga.trace_enable(False)
            rec[f"{path}_ms"] = round(sorted(totals)[len(totals) // 2], 4)
            rec[f"{path}_workspace_GB"] = round(ws.numel() / 1e9, 3)
        res[lname] = rec
        del least
    torch.cuda.empty_cache()
    return res


def cached_pairs(chunks, cache_rows, window):
    """Attended (query, key) pairs per head of a chunk over cached prefixes: new token i of a sequence with n
    cache rows (the keys just before it) sees n + i + 1 keys, at most window + 1."""
    tot = 0
    for L, n in zip(chunks, cache_rows):
        for i in range(L):
            keys = n + i + 1
            tot += keys if window < 0 else min(keys, window + 1)
    return tot


def run_prefill_cached(ga, torch, mi, reps=10):
    """Prefill of a chunk over cached prefixes (16 sequences, prefixes 2048..8192, chunks 1024..2048), each
    layer alone: median per-launch times of its kernels over `reps` calls and algorithmic FLOPs."""
    res = {}
    both = mi.chunked_16(device="cuda")
    for lname in ("swa", "glb"):
        d = both[lname]
        T, hq, hkv = d["q"].shape[0], d["q"].shape[1], d["k"].shape[1]
        Tc = d["k_cache"].shape[0]
        ws = torch.empty(ga.prefill_cached_workspace_size(T, Tc, hkv), dtype=torch.uint8, device="cuda")
        out = torch.empty(T, hq, 128, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(hq, T, dtype=torch.float32, device="cuda")
        call = lambda: ga.prefill_cached(d["q"], d["k"], d["v"], d["k_cache"], d["v_cache"], d["sink"],  # noqa
                                         d["cu_seqlens"], d["cu_cache"], d["positions"], max(d["lengths"]),
                                         d["max_position"], d["window"], d["rope_base"], out=out, lse=lse,
                                         workspace=ws)
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        ga.trace_read(clear=True)
        ga.trace_enable(True)
        for _ in range(reps):
            call()
        torch.cuda.synchronize()
        ga.trace_enable(False)
        per = {}
        for name, ms in ga.trace_read(clear=True):
            per.setdefault(name.rsplit("_", 1)[0], []).append(ms)
        med = {k: sorted(v)[len(v) // 2] for k, v in per.items()}
        attn = med.get("attn_fwd", 0.0)
        total = attn + med.get("kv_prep_cached", 0.0)
        pairs = cached_pairs(d["lengths"], d["cache_rows"], d["window"]) * hq
        flop = pairs * FWD_FLOP_PER_PAIR
        res[lname] = {"new_tokens": T, "cache_rows": Tc, "ms": round(total, 4), "attn_fwd_ms": round(attn, 4),
                      "TFLOP/s": round(flop / (total * 1e-3) / 1e12, 1),
                      "frac_of_mfma_peak": round(flop / (total * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                      "attn_fwd_TFLOP/s": round(flop / (attn * 1e-3) / 1e12, 1)}
        del d, ws, out, lse
    del both
    torch.cuda.empty_cache()
    return res


def run_shards(ga, torch, thd, dout_cpu, steps=5):
    """The training step at the per-GPU shapes of a 4-way head split of the same 32K THD batch: 16 query heads
    with 2 KV heads (sliding-window layer) and 1 KV head (global layer), forward and backward of both."""
    dev = torch.device("cuda", 0)
    layers = {}
    for name, hkv in (("swa", 2), ("glb", 1)):
        d = thd[name]
        g = {"q": d["q"][:, :16].contiguous().to(dev), "k": d["k"][:, :hkv].contiguous().to(dev),
             "v": d["v"][:, :hkv].contiguous().to(dev), "cu_seqlens": d["cu_seqlens"].to(dev),
             "sink": None if d["sink"] is None else d["sink"][:16].contiguous().to(dev),
             "window": d["window"], "rope_base": d["rope_base"], "max_seqlen": max(d["lengths"])}
        T = g["q"].shape[0]
        g["out"] = torch.empty(T, 16, 128, dtype=torch.bfloat16, device=dev)
        g["lse"] = torch.empty(16, T, dtype=torch.float32, device=dev)
        g["q_rot"] = torch.empty(T, 16, 192, dtype=torch.bfloat16, device=dev)
        g["k_rot"] = torch.empty(T, hkv, 192, dtype=torch.bfloat16, device=dev)
        g["grads"] = (torch.empty_like(g["q"]), torch.empty_like(g["k"]), torch.empty_like(g["v"]),
                      torch.empty(16, dtype=torch.float32, device=dev) if g["sink"] is not None else None)
        g["ws"] = torch.empty(ga.bwd_workspace_size(T, 16, hkv, g["window"], len(d["lengths"]), g["max_seqlen"]),
                              dtype=torch.uint8, device=dev)
        g["pairs"] = pairs_per_head(d["lengths"], d["window"]) * 16
        layers[name] = g
    dout = dout_cpu[:, :16].contiguous().to(dev)

    def step():
        for g in layers.values():
            ga.fwd(g["q"], g["k"], g["v"], g["sink"], g["cu_seqlens"], g["max_seqlen"], g["window"], g["rope_base"],
                   out=g["out"], lse=g["lse"], q_rot=g["q_rot"], k_rot=g["k_rot"])
            ga.bwd(g["q"], g["k"], g["v"], g["sink"], g["out"], g["lse"], dout, g["cu_seqlens"], g["max_seqlen"],
                   g["window"], g["rope_base"], workspace=g["ws"], grads=g["grads"], q_rot=g["q_rot"],
                   k_rot=g["k_rot"])
    for _ in range(2):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    flop = sum(g["pairs"] for g in layers.values()) * (FWD_FLOP_PER_PAIR + BWD_FLOP_PER_PAIR)
    res = {"shapes": "16 q heads; 2 kv heads (SWA), 1 kv head (global)", "ms_per_step": round(ms, 3),
           "TFLOP/s": round(flop / (ms * 1e-3) / 1e12, 1),
           "frac_of_mfma_peak": round(flop / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
    del layers, dout
    torch.cuda.empty_cache()
    return res


def run_decode_1m(ga, torch, mi, reps=10):
    """Decode of one sequence against 1,048,576 cached rows (global layer, 64 q / 4 kv heads)."""
    n = 1 << 20
    d = mi.decode_global(batch=1, len_lo=n, len_hi=n, device="cuda")
    ws = torch.empty(ga.decode_workspace_size(1, n, 64, -1), dtype=torch.uint8, device="cuda")
    out = torch.empty(1, 64, 128, dtype=torch.bfloat16, device="cuda")
    call = lambda: ga.decode(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["cu_cache"],  # noqa
                             d["positions"], None, n, -1, 1e7, out, ws)
    flush = torch.empty(1 << 29, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        call()
    times = []
    for _ in range(reps):
        flush.zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = sorted(times)[len(times) // 2]
    byts = n * 4 * (192 + 128) * 2 + 64 * (192 + 128) * 2 + 4 * (192 + 128) * 2
    del d, ws, out, flush
    torch.cuda.empty_cache()
    return {"cache_rows": n, "ms": round(ms, 4), "GB/s": round(byts / ms / 1e6, 1),
            "hbm_frac": round(byts / ms / 1e6 / HBM_PEAK_GBS, 4)}


def run_paged(ga, torch, mi, reps=10):
    """Batch-64 decode and an 8-token verify per sequence over the global-layer decode caches held in a paged
    pool whose table is a random permutation of the pool rows (every cache row in its own place)."""
    d = mi.decode_global(device="cuda")
    cu = d["cu_cache"]
    lens = (cu[1:] - cu[:-1]).tolist()
    N = int(d["k_cache"].shape[0])
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    table = torch.randperm(N, generator=g, device="cuda").to(torch.int32)
    ws = torch.empty(ga.decode_workspace_size(64, max(lens), 64, -1), dtype=torch.uint8, device="cuda")
    out = torch.empty(64, 64, 128, dtype=torch.bfloat16, device="cuda")
    flush = torch.empty(1 << 29, dtype=torch.uint8, device="cuda")

    def timed(call):
        for _ in range(3):
            call()
        times = []
        for _ in range(reps):
            flush.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            call()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        return sorted(times)[len(times) // 2]

    ms = timed(lambda: ga.decode_paged(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], table, cu,
                                       d["positions"], None, max(lens), -1, 1e7, out, ws))
    byts = N * 4 * 640 + 64 * (64 + 4) * 640
    res = {"decode_ms": round(ms, 4), "decode_GB/s": round(byts / ms / 1e6, 1),
           "decode_hbm_frac": round(byts / ms / 1e6 / HBM_PEAK_GBS, 4)}
    # verify: 8 draft tokens per sequence; the last 8 rows of each cache list play the drafts (already
    # appended), at positions len_b - 8 .. len_b - 1
    gq = torch.Generator(device="cuda")
    gq.manual_seed(8)
    q = torch.randn(64 * 8, 64, 192, generator=gq, device="cuda").to(torch.bfloat16)
    k = torch.randn(64 * 8, 4, 192, generator=gq, device="cuda").to(torch.bfloat16)
    v = torch.randn(64 * 8, 4, 128, generator=gq, device="cuda").to(torch.bfloat16)
    cuq = torch.arange(0, 64 * 8 + 1, 8, dtype=torch.int32, device="cuda")
    wsv = torch.empty(ga.prefill_cached_workspace_size(64 * 8, N, 4), dtype=torch.uint8, device="cuda")
    outv = torch.empty(64 * 8, 64, 128, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(64, 64 * 8, dtype=torch.float32, device="cuda")
    posv = (d["positions"] - 8).contiguous()
    wsq = torch.empty(ga.verify_workspace_size(64, 8, max(lens), 64, -1), dtype=torch.uint8, device="cuda")
    msv = timed(lambda: ga.verify_paged(q, d["k_cache"], d["v_cache"], table, cu, posv, None, 8, max(lens), -1, 1e7,
                                        out=outv, workspace=wsq))
    byv = N * 4 * 640 + 64 * 8 * 64 * 640
    # the same verify through the cached-prefill path: the drafts as a chunk over each list without its last
    # 8 entries (a table of exactly those entries, so cu_before[-1] equals its length)
    idx = torch.arange(N, device="cuda")
    seq = torch.bucketize(idx, cu[1:].long(), right=True)
    keep = idx < (cu[1:].long()[seq] - 8)
    table_before = table[keep].contiguous()
    cu_before = (cu - torch.arange(0, 65 * 8, 8, dtype=torch.int32, device="cuda")).contiguous()
    assert table_before.numel() == int(cu_before[-1])
    msp = timed(lambda: ga.prefill_paged(q, k, v, d["k_cache"], d["v_cache"], table_before, None, cuq, cu_before,
                                         posv, 8, max(lens) + 8, -1, 1e7, out=outv, lse=lse, workspace=wsv))
    res.update({"verify_tokens_per_sequence": 8, "verify_ms": round(msv, 4),
                "verify_ms_per_token": round(msv / 8, 4), "verify_GB/s": round(byv / msv / 1e6, 1),
                "verify_via_cached_prefill_ms": round(msp, 4)})
    del d, table, ws, out, flush, q, k, v, wsv, wsq, outv, lse
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=int(os.environ.get("WORLD_SIZE", "1")))
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--step-only", action="store_true",
                    help="only the training step (for profiles whose per-kernel averages are the step's)")
    ap.add_argument("--cpu-threads", type=int, default=min(16, os.cpu_count() or 1))
    ap.add_argument("--traffic-probe", metavar="DIR", help="run the counter-pass workload (see the module doc)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.json from two counter passes")
    ap.add_argument("--stats-summary", nargs=4, metavar=("TRACE_DIR", "TITLE", "COMMAND", "TIMED"),
                    help="print a rocprofv3 kernel trace as a text table (TIMED: launches per kernel in the timed "
                         "steps)")
    ap.add_argument("--mfma-summary", nargs=3, metavar=("PMC_DIR", "TITLE", "COMMAND"),
                    help="print the MFMA counters of a --traffic-probe counter run per kernel of the step")
    args = ap.parse_args()
    if args.stats_summary:
        stats_summary(*args.stats_summary)
        return
    if args.mfma_summary:
        mfma_summary(*args.mfma_summary)
        return
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.traffic_probe:
        traffic_probe(args.traffic_probe)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build runs the attention layer on a single MI355X and "
              f"has no multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch

    import global_gqa_attention_amd as ga
    import mimo_inputs as mi

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    thd, dout_cpu, layers, step = setup_layers(ga, torch, mi, dev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ga.trace_read(clear=True)

    ga.trace_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ga.trace_enable(False)
    trace = ga.trace_read(clear=True)

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    flops = sum(g["pairs"] * (FWD_FLOP_PER_PAIR + BWD_FLOP_PER_PAIR) for g in layers.values())
    value = flops / (ms_per_step * 1e-3) / 1e12

    # per-kernel averages over the timed region (HIP events on the launch stream)
    per = {}
    for name, ms in trace:
        per.setdefault(name, []).append(ms)
    kernels = {}
    for name, v in per.items():
        layer = "swa" if name.endswith("_swa") else ("glb" if name.endswith("_global") else None)
        base = name.rsplit("_", 1)[0] if layer else name
        avg = sum(v) / len(v)
        rec = {"avg_ms": round(avg, 4), "launches": len(v)}
        if layer and base in KERNEL_FLOP_PER_PAIR:
            rec["TFLOP/s"] = round(layers[layer]["pairs"] * KERNEL_FLOP_PER_PAIR[base] / (avg * 1e-3) / 1e12, 1)
        kernels[name] = rec
    dom = max(kernels, key=lambda k: kernels[k]["avg_ms"] * kernels[k]["launches"])
    drec = kernels[dom]
    layer = "swa" if dom.endswith("_swa") else "glb"
    base = dom.rsplit("_", 1)[0]
    ach = layers[layer]["pairs"] * KERNEL_FLOP_PER_PAIR.get(base, 0) / (drec["avg_ms"] * 1e-3) / 1e12
    traffic = measured_traffic(dom)
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic}

    layer_tflops = {}
    for lname, g in layers.items():
        suf = "_swa" if lname == "swa" else "_global"
        mine = {k[: -len(suf)]: v for k, v in kernels.items() if k.endswith(suf)}
        fwd_ms = sum(v["avg_ms"] for k, v in mine.items() if k in ("kv_prep", "attn_fwd"))
        bwd_ms = sum(v["avg_ms"] for k, v in mine.items() if k.startswith("bwd_"))
        layer_tflops[lname] = {
            "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
            "fwd_TFLOP/s": round(g["pairs"] * FWD_FLOP_PER_PAIR / (fwd_ms * 1e-3) / 1e12, 1) if fwd_ms else None,
            "bwd_TFLOP/s": round(g["pairs"] * BWD_FLOP_PER_PAIR / (bwd_ms * 1e-3) / 1e12, 1) if bwd_ms else None,
            "pairs": g["pairs"]}

    line = {
        "metric": "attention TFLOP/s fwd+bwd (SWA+sink, global) at 32K THD tokens; % bf16 MFMA peak",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "THD prefill fwd+bwd, 32768 tokens (16 x U[1024,2048] + pad), SWA layer "
                               "(64q/8kv, window 128, sink, base 1e4) + global layer (64q/4kv, causal, base 1e7)",
                   "global_batch": len(thd["swa"]["lengths"]), "seq_len": 32768, "parallelism": "none (1 GPU)"},
        "frac_of_mfma_peak": round(value / MFMA_BF16_PEAK_TFLOPS, 4),
        "layers": layer_tflops, "kernels": kernels, "roofline": roofline,
    }
    if not args.step_only:
        line["prefill"] = run_prefill(ga, torch, layers)
        line["bwd_paths"] = run_bwd_paths(ga, torch, layers)
        line["prefill_cached"] = run_prefill_cached(ga, torch, mi)
        line["tp4_shard_step"] = run_shards(ga, torch, thd, dout_cpu)
    if not args.no_decode and not args.step_only:
        line["decode"] = run_decode(ga, torch, mi)
        line["decode_1m"] = run_decode_1m(ga, torch, mi)
        line["paged"] = run_paged(ga, torch, mi)
    if not args.no_cpu_baseline and not args.step_only:
        line["cpu_baseline"] = cpu_baseline(thd, dout_cpu, args.cpu_threads)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
