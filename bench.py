#!/usr/bin/env python3
"""Benchmark of the blockwise causal varlen attention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--rows all|headline]

A step is one pass of the hot path over the headline workload: one zig-zag
virtual rank of a cp=8 ring at its real shape (rank 3 of 131072 packed tokens,
log-uniform documents in [1024, 32768], 16384 local rows, HQ=32, HKV=8,
D=128, bf16): the 8 forward blocks in ring order with their 7 online-softmax
merges (the last one fused with the bf16 cast), then the backward: delta once
and the 8 merged-lse block backwards accumulating dq and every owner's dk/dv.
The metric is causal-effective TFLOP/s of forward + backward: visible pairs x
(4 + 10) x D x HQ per step over the timed wall time (masked work never
counts). Inputs are resident in HBM before timing starts.

The JSON line also carries
  * roofline: the dominant kernel's algorithmic FLOPs (or bytes) per launch
    over its mean launch duration, from hipEvents the library records around
    its own launches on their stream during the timed steps, against the
    MI355X peak (bf16 dense MFMA 2.5 PFLOP/s, HBM 8 TB/s);
  * kernels: the same for every kernel of the step;
  * rows: the other workloads of the path measured the same way (packed
    varlen forward over 4 ranks, KV-parallel paged prefill for both windows,
    EAGLE-3 mixed attention on the headline rank with 3 TTT diagonal blocks,
    one-query decode GB/s) -- skipped with --rows headline;
  * cpu_baseline: the fp64 oracle timed on the host on a bounded sample of
    the same workload (sampled query rows, forward and backward).
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

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (AMD published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (AMD published)
BF16_FLOP_PER_CLK_CU = 4096  # dense bf16 MFMA flops per clock per CDNA4 compute unit
METRIC = "causal-effective TFLOP/s fwd(+bwd) & % bf16 MFMA peak; decode GB/s & % HBM peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def device_peaks():
    """The bf16 MFMA peak re-derived from the GPU agent rocminfo reports
    (compute units x max engine clock x 4096 flop/clk/CU), beside the
    published figures the roofline fractions use. rocminfo reports no memory
    bandwidth, so the HBM peak is the published 8 TB/s."""
    import re
    import subprocess
    info = {"bf16_tflops_published": PEAK_BF16_TFLOPS, "hbm_gbs_published": PEAK_HBM_GBS,
            "used_for_frac": "published"}
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError) as e:
        info["rocminfo"] = f"unavailable: {e}"
        return info
    for agent in txt.split("Agent ")[1:]:
        if not re.search(r"Name:\s+gfx9", agent):
            continue
        cu = re.search(r"Compute Unit:\s+(\d+)", agent)
        clk = re.search(r"Max Clock Freq\. \(MHz\):\s+(\d+)", agent)
        if cu and clk:
            cus, mhz = int(cu.group(1)), int(clk.group(1))
            info.update({"rocminfo_compute_units": cus, "rocminfo_max_clock_mhz": mhz,
                         "bf16_tflops_rocminfo": round(cus * mhz * 1e6 * BF16_FLOP_PER_CLK_CU / 1e12, 1)})
            return info
    info["rocminfo"] = "no gfx9 agent found"
    return info


def sources_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "blockwise_causal_varlen_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel):
    """HBM bytes per launch measured by rocprofv3 counters, if the committed
    record matches the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#") or "=" not in line:
            continue
        k, v = line.split("=", 1)
        rec[k.strip()] = v.strip()
    if rec.get("sources") != sources_digest():
        return None
    v = rec.get(f"{kernel}.bytes_per_launch")
    return float(v) if v else None


# rocprofv3 kernel names -> the library's timing names
TRAFFIC_KERNELS = {"fwd_bf16_kernel": "attn_fwd", "dkdv_bf16_kernel": "attn_dkdv", "dq_bf16_kernel": "attn_dq",
                   "diag_merge_kernel": "attn_merge_diag", "diag_bwd_kernel": "attn_diag_bwd",
                   "merge_kernel": "attn_merge", "delta_kernel": "attn_delta", "decode_kernel": "attn_decode"}
CALIB_BYTES = 1 << 30  # the plain device copy measured beside the kernels


def calib_copy(torch):
    """A plain device-to-device copy of CALIB_BYTES (3 times): what the HBM
    counters read for it calibrates FETCH_SIZE / WRITE_SIZE."""
    src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def traffic_summary(fetch_csv, write_csv, out_path, command):
    """Per-launch HBM bytes of each kernel from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each divided by what the
    same counter reads for the plain copy of CALIB_BYTES."""
    import csv
    import statistics

    def read(path, counter):
        per = {}
        calib = []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name, kib = r["Kernel_Name"], float(r["Counter_Value"])
            if "copyBuffer" in name or "copy_kernel" in name or "CopyKernel" in name:
                if kib * 1024 > CALIB_BYTES / 8:  # the big copy, not small runtime blits
                    calib.append(kib * 1024 / CALIB_BYTES)
                continue
            for key, tname in TRAFFIC_KERNELS.items():  # first match (diag_merge before merge)
                if key in name:
                    per.setdefault(tname, []).append(kib * 1024)
                    break
        if not calib:
            raise SystemExit(f"{path}: no copy of {CALIB_BYTES} bytes found for the calibration")
        return per, statistics.median(calib)

    fetch, ff = read(fetch_csv, "FETCH_SIZE")
    write, wf = read(write_csv, "WRITE_SIZE")
    lines = ["# HBM traffic per launch from rocprofv3 counters (bytes); counter readings are",
             "# divided by the reading for a plain device copy of %d bytes" % CALIB_BYTES,
             "# commands:"] + ["#   " + c for c in command] + [
             f"fetch_calibration = {ff:.4f}", f"write_calibration = {wf:.4f}", f"sources = {sources_digest()}"]
    for tname in sorted(set(fetch) | set(write)):
        fb = statistics.mean(fetch.get(tname, [0.0])) / ff
        wb = statistics.mean(write.get(tname, [0.0])) / wf
        lines += [f"{tname}.launches = {len(fetch.get(tname, []))}", f"{tname}.fetch_bytes_per_launch = {fb:.0f}",
                  f"{tname}.write_bytes_per_launch = {wb:.0f}", f"{tname}.bytes_per_launch = {fb + wb:.0f}"]
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


TRACE_FILE = os.path.join(ROOT, "profiles", "zigzag_cp8_rank3_fwd_bwd_kernel_trace.md")


def trace_summary(stats_csv, trace_csv, bench_json, out_path, command, timed_fraction):
    """Kernel-trace summary of a rocprofv3 --kernel-trace --stats run over the
    headline bench: the stats table (every dispatch), then each library
    kernel's mean over the timed steps only (the last timed_fraction of its
    dispatches), beside the mean launch duration the bench measured live with
    hipEvents (bench_json: the JSON line of a bench.py run of the same sources,
    normally the traced run itself, so both columns time the same launches)."""
    import csv
    import statistics
    rows = list(csv.DictReader(open(stats_csv)))
    lines = ["# Kernel trace: zig-zag cp=8 rank-3 step (131072 tokens, HQ=32, HKV=8, D=128, bf16), fwd + bwd", "",
             "Commands (from the repository root, on one MI355X):", "", "```"] + command + ["```", "",
             f"Sources digest {sources_digest()}. All dispatches of the profiled run (durations in microseconds):",
             "", "| kernel | calls | total us | mean us | % |", "|---|---:|---:|---:|---:|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"]))[:16]:
        name = r["Name"] if len(r["Name"]) <= 90 else r["Name"][:87] + "..."
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e3:.1f} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    per = {}
    for r in csv.DictReader(open(trace_csv)):
        for key, tname in TRAFFIC_KERNELS.items():
            if key in r["Kernel_Name"]:
                per.setdefault(tname, []).append((int(r["Start_Timestamp"]),
                                                  (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
                break
    bench = {}
    if bench_json:
        rec = json.loads(open(bench_json).read().strip().splitlines()[-1])
        bench = {k: v.get("mean_launch_us") for k, v in rec.get("kernels", {}).items() if v}
        lines += ["", f"bench.py line used for the hipEvent column: {rec.get('value')} {rec.get('unit')}, "
                      f"{rec.get('ms_per_step')} ms per step, sources {rec.get('sources')}."]
    lines += ["", f"Per kernel, the mean over the timed steps (the last {timed_fraction:.2f} of its dispatches) "
                  "beside the bench's hipEvent mean:", "",
              "| kernel | rocprofv3 timed-step mean us | bench.py hipEvent mean us |", "|---|---:|---:|"]
    for tname in ("attn_fwd", "attn_dkdv", "attn_dq", "attn_delta"):
        if tname not in per:
            continue
        d = [x[1] for x in sorted(per[tname])]
        timed = d[len(d) - max(1, round(len(d) * timed_fraction)):]
        b = bench.get(tname)
        lines.append(f"| {tname} | {statistics.mean(timed):.1f} | {b if b is not None else '-'} |")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


STATS_FILE = os.path.join(ROOT, "profiles", "all_rows_kernel_stats.md")


def stats_summary(stats_csv, bench_json, out_path, command):
    """Per-kernel statistics of a rocprofv3 --kernel-trace --stats run over the
    whole bench (every row): calls, total and mean duration of each kernel,
    beside the row figures the same run printed (bench_json: its JSON line)."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    lines = ["# Kernel statistics: every bench row (headline, packed varlen, KV-parallel, EAGLE-3, Ulysses, "
             "merge, decode)", "", "Commands (from the repository root, on one MI355X):", "", "```"] + command + \
            ["```", "", f"Sources digest {sources_digest()}. All dispatches of the profiled run, longest total first "
             "(durations in microseconds):", "", "| kernel | calls | total us | mean us | % |",
             "|---|---:|---:|---:|---:|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"] if len(r["Name"]) <= 90 else r["Name"][:87] + "..."
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e3:.1f} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    if bench_json:
        rec = json.loads(open(bench_json).read().strip().splitlines()[-1])
        lines += ["", f"The same run's bench line: headline {rec.get('value')} {rec.get('unit')}, "
                      f"{rec.get('ms_per_step')} ms per step, sources {rec.get('sources')}. Its rows, with the "
                      "mean launch duration of each row's measured kernel (hipEvents):", "",
                  "| row | ms per step | kernel | mean launch us | fraction of peak |", "|---|---:|---|---:|---:|"]
        for name, row in rec.get("rows", {}).items():
            for sub in row.values():
                if isinstance(sub, dict) and "mean_launch_us" in sub:
                    lines.append(f"| {name} | {row.get('ms', 0):.4f} | {sub['kernel']} | {sub['mean_launch_us']} | "
                                 f"{sub['frac']} |")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# Counters of one rocprofv3 --pmc pass each (at most 8 SQ and 2 GRBM counters a pass)
COUNTER_PASSES = [
    ["GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU",
     "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_LDS", "SQ_INSTS_SALU"],
    ["GRBM_GUI_ACTIVE", "SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_VALU",
     "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_ANY", "SQ_LDS_BANK_CONFLICT"],
]
SIMDS = 256 * 4
XCDS = 8  # GRBM_GUI_ACTIVE comes summed over the 8 XCDs (each counts its active cycles)
COUNTERS_FILE = os.path.join(ROOT, "profiles", "zigzag_cp8_rank3_fwd_bwd_counters.txt")


def load_counters(kernel):
    """MFMA-busy fraction and instruction mix of a kernel from the committed
    rocprofv3 counter summary, if it matches the current kernel sources."""
    path = COUNTERS_FILE
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#") or "=" not in line:
            continue
        k, v = line.split("=", 1)
        rec[k.strip()] = v.strip()
    if rec.get("sources") != sources_digest():
        return None
    keys = ("mfma_busy", "valu_per_mfma", "trans_per_mfma", "lds_per_mfma", "coexec_of_mfma_busy", "wait_lds_of_wave",
            "wait_any_of_wave", "lds_bank_conflict_of_lds_active")
    out = {k: float(rec[f"{kernel}.{k}"]) for k in keys if f"{kernel}.{k}" in rec}
    return out or None


def counter_summary(csvs, out_path, command):
    """Per-kernel means of the rocprofv3 --pmc passes (COUNTER_PASSES), and the
    derived MFMA-busy fraction (SQ_VALU_MFMA_BUSY_CYCLES over the active cycles
    of one XCD, GRBM_GUI_ACTIVE / 8, times 1024 SIMDs: the share of the SIMDs'
    cycles at the clock the kernel ran at), VALU / transcendental / LDS
    instructions per MFMA, co-execution and wait fractions."""
    import csv
    import statistics
    vals = {}
    for path in csvs:
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"]
            for key, tname in TRAFFIC_KERNELS.items():
                if key in name:
                    vals.setdefault(tname, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                    break
    lines = ["# rocprofv3 counters per launch (mean over the profiled launches) and derived ratios",
             "# commands:"] + ["#   " + c for c in command] + [f"sources = {sources_digest()}"]
    for tname in sorted(vals):
        c = {k: statistics.mean(v) for k, v in vals[tname].items()}
        for k in sorted(c):
            lines.append(f"{tname}.{k} = {c[k]:.6g}")
        gui = c.get("GRBM_GUI_ACTIVE")
        mf = c.get("SQ_INSTS_MFMA")
        if gui and "SQ_VALU_MFMA_BUSY_CYCLES" in c:
            lines.append(f"{tname}.mfma_busy = {c['SQ_VALU_MFMA_BUSY_CYCLES'] / (gui / XCDS * SIMDS):.4f}")
        if mf:
            for src, dst in (("SQ_INSTS_VALU", "valu_per_mfma"), ("SQ_INSTS_VALU_TRANS_F32", "trans_per_mfma"),
                             ("SQ_INSTS_LDS", "lds_per_mfma")):
                if src in c:
                    lines.append(f"{tname}.{dst} = {c[src] / mf:.3f}")
        if c.get("SQ_VALU_MFMA_BUSY_CYCLES") and "SQ_VALU_MFMA_COEXEC_CYCLES" in c:
            lines.append(f"{tname}.coexec_of_mfma_busy = "
                         f"{c['SQ_VALU_MFMA_COEXEC_CYCLES'] / c['SQ_VALU_MFMA_BUSY_CYCLES']:.4f}")
        if c.get("SQ_WAVE_CYCLES"):
            for src, dst in (("SQ_WAIT_INST_LDS", "wait_lds_of_wave"), ("SQ_WAIT_INST_ANY", "wait_any_of_wave")):
                if src in c:
                    lines.append(f"{tname}.{dst} = {c[src] / c['SQ_WAVE_CYCLES']:.4f}")
        if c.get("SQ_ACTIVE_INST_LDS") and "SQ_LDS_BANK_CONFLICT" in c:
            lines.append(f"{tname}.lds_bank_conflict_of_lds_active = "
                         f"{c['SQ_LDS_BANK_CONFLICT'] / c['SQ_ACTIVE_INST_LDS']:.4f}")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def timed_steps(step, steps, warmup, torch, lib, timing=True):
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    if timing:
        lib.attn_timing_enable(True)
        lib.attn_timing_report()  # clear
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kt = {}
    if timing:
        kt = lib.attn_timing_report()
        lib.attn_timing_enable(False)
    return (t1 - t0) / steps, kt


def roofline(name, work_per_step, kt, steps, bound, traffic=None):
    """achieved = algorithmic work of all launches / their summed durations."""
    cnt, ms = kt.get(name, (0, 0.0))
    if cnt == 0 or ms <= 0:
        return None
    per_launch = work_per_step * steps / cnt
    mean_s = ms / 1e3 / cnt
    if bound == "mfma":
        achieved = per_launch / mean_s / 1e12
        peak, unit = PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved = per_launch / mean_s / 1e9
        peak, unit = PEAK_HBM_GBS, "GB/s"
    return {"kernel": name, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic, "launches_per_step": cnt / steps,
            "mean_launch_us": round(mean_s * 1e6, 2), "work_per_launch": per_launch}


def headline(args, torch, lib, I, W):
    case = I.cfg3(rank=3)
    cp, r = case.cp, 3
    nloc, hq, d = case.q.shape
    wl = W.ZigzagWorkload(case, ranks=[r], with_bwd=True)

    def step():
        wl.forward()
        wl.backward()

    sec, kt = timed_steps(step, args.steps, args.warmup, torch, lib)
    pairs = wl.pairs_per_rank()
    fwd_f, bwd_f = 4 * d * hq * pairs, 10 * d * hq * pairs
    tflops = (fwd_f + bwd_f) / sec / 1e12
    doc_lens = wl.doc_lens
    rows_all = sum(L_ // cp for L_ in doc_lens)
    # the delta pass reads dout and out (bf16) and writes delta; with bf16
    # inputs it also reads q and writes the f16 copies of q and dout
    delta_bytes = rows_all * hq * (2 * d * 2 + 4 + (d * 2 + 2 * d * 2 if case.q.dtype == torch.bfloat16 else 0))
    kernels = {
        "attn_fwd": roofline("attn_fwd", fwd_f, kt, args.steps, "mfma", load_traffic("attn_fwd")),
        "attn_dkdv": roofline("attn_dkdv", 8 * d * hq * pairs, kt, args.steps, "mfma", load_traffic("attn_dkdv")),
        "attn_dq": roofline("attn_dq", 2 * d * hq * pairs, kt, args.steps, "mfma", load_traffic("attn_dq")),
        "attn_delta": roofline("attn_delta", delta_bytes, kt, args.steps, "hbm", load_traffic("attn_delta")),
    }
    for name, rec in kernels.items():
        if rec is not None:
            rec["counters"] = load_counters(name)
    times = {k: v[1] for k, v in kt.items()}
    dominant = max((k for k in kernels if kernels[k]), key=lambda k: times.get(k, 0.0))
    cfg = {"workload": "zigzag cp=8, virtual rank 3 of 131072 packed tokens (16384 local rows), fwd 8 blocks "
                       "(7 merges in the forward epilogue) + bwd (delta + 8 merged-lse blocks)",
           "tokens_global": 131072, "local_rows": nloc, "docs": len(doc_lens), "hq": hq, "hkv": 8, "head_dim": d,
           "cp": cp, "rank": r, "visible_pairs_per_head": pairs,
           "flops_fwd": fwd_f, "flops_bwd": bwd_f, "parallelism": "one virtual rank on one GPU"}
    return {"ms_per_step": sec * 1e3, "value": tflops, "fwd_flops": fwd_f, "bwd_flops": bwd_f, "pairs": pairs,
            "kernels": kernels, "dominant": dominant, "kernel_ms": kt, "config": cfg, "wl": wl, "case": case}


def other_rows(args, torch, lib, I, W):
    rows = {}
    steps = max(3, args.steps // 2)
    # packed varlen forward, 4 zig-zag ranks (all of them)
    c2 = I.cfg2()
    w2 = W.ZigzagWorkload(c2)
    f = w2.fwd_flops()
    # the 4 virtual ranks on 4 streams (each rank's 4 blocks its own launches) ...
    sec, kt = timed_steps(w2.forward, steps, args.warmup, torch, lib)
    rows["packed_varlen_fwd_cp4"] = {"ms": sec * 1e3, "TFLOP/s": f / sec / 1e12, "frac": f / sec / 1e12 / PEAK_BF16_TFLOPS,
                                     "ranks": "4 streams, 16 forward launches",
                                     "fwd_kernel": roofline("attn_fwd", f, kt, steps, "mfma")}
    # ... and batched: each ring step's 4 blocks in one launch
    sec, kt = timed_steps(w2.forward_batched, steps, args.warmup, torch, lib)
    rows["packed_varlen_fwd_cp4_batched"] = {"ms": sec * 1e3, "TFLOP/s": f / sec / 1e12,
                                             "frac": f / sec / 1e12 / PEAK_BF16_TFLOPS,
                                             "ranks": "one stream, 4 forward launches (one per ring step)",
                                             "fwd_kernel": roofline("attn_fwd", f, kt, steps, "mfma")}
    del w2, c2
    for window in (0, 4096):
        c4 = I.cfg4(window=window)
        w4 = W.KvpWorkload(c4)
        sec, kt = timed_steps(w4.forward, steps, args.warmup, torch, lib)
        f = w4.fwd_flops()
        R, n, hq, d = c4.R, w4.s_q, w4.hq, w4.d
        merge_bytes = n * hq * (R * (d * 4 + 4) + d * 2 + 4)
        rows[f"kvp_prefill_W{window}"] = {"ms": sec * 1e3, "TFLOP/s": f / sec / 1e12,
                                          "frac": f / sec / 1e12 / PEAK_BF16_TFLOPS,
                                          "fwd_kernel": roofline("attn_fwd", f, kt, steps, "mfma"),
                                          "rank_merge": roofline("attn_merge_n", merge_bytes, kt, steps, "hbm"),
                                          "kernel_ms": kt}
        del w4, c4
    # EAGLE-3 mixed attention on the headline rank: zig-zag block 0 + 3 TTT diagonals
    n_ttt = 3
    ce = I.eagle_case(I.cfg3(), n_ttt)
    we = W.EagleWorkload(ce, ranks=[3], with_bwd=True)

    def eagle_step():
        we.forward()
        we.backward()

    sec, kt = timed_steps(eagle_step, steps, args.warmup, torch, lib)
    nq, hq, d = we.zz.q_loc[3].shape
    pairs = we.zz.pairs_per_rank() + nq * n_ttt
    f = (4 + 10) * d * hq * pairs
    mb, mbl, bb = we.diag_bytes()
    rows[f"eagle_ttt{n_ttt}_fwd_bwd"] = {
        "ms": sec * 1e3, "TFLOP/s": f / sec / 1e12, "frac": f / sec / 1e12 / PEAK_BF16_TFLOPS,
        "merge_diag": roofline("attn_merge_diag", (n_ttt - 1) * mb + mbl, kt, steps, "hbm",
                               load_traffic("attn_merge_diag")),
        "diag_bwd": roofline("attn_diag_bwd", n_ttt * bb, kt, steps, "hbm", load_traffic("attn_diag_bwd")),
        "kernel_ms": kt}
    del we, ce
    torch.cuda.empty_cache()
    # Ulysses EAGLE-3 over the whole 131072-token sequence, uly = 8 virtual ranks
    c3 = I.cfg3()
    cu = c3.cu
    full = I.zigzag_case("ulysses base", (cu[1:] - cu[:-1]).tolist(), c3.q.shape[1], c3.k.shape[1], c3.q.shape[2],
                         c3.q.dtype, c3.cp)
    del c3
    cu_case = I.eagle_case(full, n_ttt)
    wu = W.UlyssesWorkload(cu_case, 8, with_bwd=True)

    def uly_step():
        wu.forward()
        wu.backward()

    sec, kt = timed_steps(uly_step, max(2, steps // 2), 1, torch, lib)
    nu = max(2, steps // 2)
    f = (4 + 10) * wu.d * wu.hq * (wu.block0_pairs() + wu.S * n_ttt)
    rows[f"ulysses_uly8_ttt{n_ttt}_fwd_bwd"] = {
        "ms": sec * 1e3, "TFLOP/s": f / sec / 1e12, "frac": f / sec / 1e12 / PEAK_BF16_TFLOPS,
        "workload": "131072 tokens (the headline documents), HQ=32, HKV=8, D=128, all 8 virtual ranks",
        "reshard": roofline("attn_reshard", wu.reshard_bytes(), kt, nu, "hbm"),
        "fwd_kernel": roofline("attn_fwd", 4 * wu.d * wu.hq * wu.block0_pairs(), kt, nu, "mfma"),
        "kernel_ms": kt}
    del wu, cu_case, full
    torch.cuda.empty_cache()
    # the standalone merge kernel (one block into the running state) at the
    # headline rank's shape: f32 state read + written, bf16 block out, lse
    gm = torch.Generator(device="cuda")
    gm.manual_seed(7)
    n, hq, d = 16384, 32, 128
    acc = torch.randn(n, hq, d, device="cuda", dtype=torch.float32, generator=gm)
    lse = torch.randn(hq, n, device="cuda", dtype=torch.float32, generator=gm)
    bo = torch.randn(n, hq, d, device="cuda", dtype=torch.float32, generator=gm).to(torch.bfloat16)
    bl = torch.randn(hq, n, device="cuda", dtype=torch.float32, generator=gm)
    sec, kt = timed_steps(lambda: lib.merge(acc, lse, bo, bl), steps, 1, torch, lib)
    b = n * hq * (d * 4 * 2 + d * 2 + 12)
    rows["merge_16384x32x128"] = {"ms": sec * 1e3, "GB/s": b / sec / 1e9, "frac": b / sec / 1e9 / PEAK_HBM_GBS,
                                  "bytes": b, "merge_kernel": roofline("attn_merge", b, kt, steps, "hbm",
                                                                       load_traffic("attn_merge"))}
    del acc, lse, bo, bl
    c5 = I.cfg5(device="cuda")
    w5 = W.DecodeWorkload(c5)
    sec, kt = timed_steps(w5.forward, steps, 1, torch, lib)
    b = w5.bytes()
    rows["decode_65536"] = {"ms": sec * 1e3, "GB/s": b / sec / 1e9, "frac": b / sec / 1e9 / PEAK_HBM_GBS,
                            "bytes": b, "decode_kernel": roofline("attn_decode", b, kt, steps, "hbm",
                                                                  load_traffic("attn_decode"))}
    del w5, c5
    # split-KV (flash-decoding): 16 sequences x 65536 keys, HQ=32, HKV=4
    c6 = I.long_decode([65536] * 16, device="cuda")
    w6 = W.DecodeWorkload(c6)
    sec, kt = timed_steps(w6.forward, steps, 1, torch, lib)
    b = w6.bytes()
    rows["decode_split_16x65536"] = {"ms": sec * 1e3, "GB/s": b / sec / 1e9, "frac": b / sec / 1e9 / PEAK_HBM_GBS,
                                     "bytes": b, "decode_kernel": roofline("attn_decode", b, kt, steps, "hbm"),
                                     "kernel_ms": kt}
    del w6, c6
    torch.cuda.empty_cache()
    return rows


def cpu_baseline(case, target_s, np):
    """fp64 oracle on sampled query rows of the headline workload: the 8
    forward blocks + merges and the 8 backward blocks for those rows."""
    import oracle as O
    from threadpoolctl import threadpool_info, threadpool_limits

    cp, r = case.cp, 3
    cu = case.cu
    cu_l = (cu // cp).numpy()
    ks = [O.zigzag_shard(case.k, cu, cp, s)[0] for s in range(cp)]
    vs = [O.zigzag_shard(case.v, cu, cp, s)[0] for s in range(cp)]
    q, do = O.as_f64(case.q), O.as_f64(case.dout)
    rng = np.random.default_rng(0)

    def run(nrows):
        rows = np.sort(rng.choice(q.shape[0], nrows, replace=False))
        t0 = time.perf_counter()
        out = lse = None
        for s in range(cp):
            src, kind = O.zigzag_step(r, s, cp)
            bo, bl = O.block_forward(q, ks[src], vs[src], cu_l, cu_l, case.scale, rows=rows,
                                     **O.zigzag_block_args(kind))
            out, lse = (bo, bl) if out is None else O.merge(out, lse, bo, bl)[:2]
        for s in range(cp):
            src, kind = O.zigzag_step(r, s, cp)
            O.block_backward(do, q, ks[src], vs[src], out, lse, cu_l, cu_l, case.scale, rows=rows,
                             **O.zigzag_block_args(kind))
        dt = time.perf_counter() - t0
        pairs = 0
        # visible pairs of the sampled rows per q head
        for s in range(cp):
            kind = O.zigzag_step(r, s, cp)[1]
            a = O.zigzag_block_args(kind)
            for d_, (qs, qe) in enumerate(O.doc_bounds(cu_l)):
                qa, qb = O.view_range(qs, qe, a.get("q_view", "all"))
                ka, kb = O.view_range(qs, qe, a.get("k_view", "all"))
                sel = rows[(rows >= qa) & (rows < qb)]
                if a.get("causal"):
                    pairs += int(np.sum(np.minimum(sel - qs + 1, kb - ka)))
                else:
                    pairs += len(sel) * (kb - ka)
        return dt, pairs

    # all the host cores this process may run on, capped by the thread count
    # the environment grants (OMP_NUM_THREADS, when set)
    affinity = len(os.sched_getaffinity(0))
    cap = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    cores = min(affinity, cap) if cap > 0 else affinity
    with threadpool_limits(limits=cores, user_api="blas"):
        # grow the sample until it takes about target_s (the cost per row is not
        # linear at small samples: whole documents' keys are read per row chunk)
        n = 16
        dt, pairs = run(n)
        while dt < 0.6 * target_s and n < 8192:
            n = min(8192, int(n * min(8.0, max(1.5, 0.9 * target_s / max(dt, 1e-3)))))
            dt, pairs = run(n)
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    hq, d = q.shape[1], q.shape[2]
    flops = pairs * (4 + 10) * d * hq
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "affinity_cores": affinity,
            "sample": f"{n} sampled query rows of the headline rank (fwd 8 blocks + merges, bwd 8 blocks), "
                      f"{pairs} visible pairs x 32 heads, {dt:.1f} s on the host, fp64 numpy with {threads} "
                      f"BLAS threads ({affinity} cores in the affinity mask)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--rows", choices=["all", "headline"], default="all")
    ap.add_argument("--cpu-baseline", choices=["on", "off"], default="on")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration for --traffic-summary)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="host only: turn two rocprofv3 --pmc counter CSVs into profiles/traffic.txt")
    ap.add_argument("--traffic-command", action="append", default=[],
                    help="with --traffic-summary / --counter-summary / --trace-summary / --stats-summary: a command line "
                         "to record in the summary")
    ap.add_argument("--counter-summary", nargs="+", metavar="CSV",
                    help="host only: turn rocprofv3 --pmc counter CSVs (the passes of COUNTER_PASSES) into "
                         "the counter summary under profiles/")
    ap.add_argument("--trace-summary", nargs=3, metavar=("STATS_CSV", "TRACE_CSV", "BENCH_JSON"),
                    help="host only: turn a rocprofv3 --kernel-trace --stats run of the headline (its "
                         "kernel_stats and kernel_trace CSVs) and a bench.py JSON line into the kernel-trace "
                         "summary under profiles/ (BENCH_JSON may be '-')")
    ap.add_argument("--stats-summary", nargs=2, metavar=("STATS_CSV", "BENCH_JSON"),
                    help="host only: turn a rocprofv3 --kernel-trace --stats run of the whole bench (its "
                         "kernel_stats CSV) and that run's JSON line into the all-rows summary under profiles/")
    ap.add_argument("--trace-timed-fraction", type=float, default=0.75,
                    help="with --trace-summary: the share of each kernel's dispatches in the timed steps")
    ap.add_argument("--print-counter-passes", action="store_true",
                    help="print the counter list of each --pmc pass, one line each")
    args = ap.parse_args()
    if args.print_counter_passes:
        for p in COUNTER_PASSES:
            print(" ".join(p))
        return
    if args.counter_summary:
        counter_summary(args.counter_summary, COUNTERS_FILE, args.traffic_command)
        return
    if args.stats_summary:
        st, bj = args.stats_summary
        stats_summary(st, None if bj == "-" else bj, STATS_FILE, args.traffic_command)
        return
    if args.trace_summary:
        st, tr, bj = args.trace_summary
        trace_summary(st, tr, None if bj == "-" else bj, TRACE_FILE, args.traffic_command,
                      args.trace_timed_fraction)
        return
    if args.traffic_summary:
        traffic_summary(args.traffic_summary[0], args.traffic_summary[1],
                        os.path.join(ROOT, "profiles", "traffic.txt"), args.traffic_command)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the virtual-rank schedules run all ranks on a single device and "
              "the library has no multi-GPU path (--gpus 1).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from blockwise_causal_varlen_amd import inputs as I, lib, workloads as W
    lib.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    log(f"device: {torch.cuda.get_device_name(0)}")
    peaks = device_peaks()
    log(f"peaks: {json.dumps(peaks)}")
    h = headline(args, torch, lib, I, W)
    log(f"headline: {h['ms_per_step']:.3f} ms/step, {h['value']:.1f} TFLOP/s fwd+bwd")
    case = h.pop("case")
    del h["wl"]
    torch.cuda.empty_cache()
    rows = other_rows(args, torch, lib, I, W) if args.rows == "all" else {}
    for k, v in rows.items():
        log(f"row {k}: {json.dumps({kk: vv for kk, vv in v.items() if kk != 'kernel_ms'})}")
    if args.calib_copy:
        calib_copy(torch)
    cpu = cpu_baseline(case, args.cpu_seconds, np) if args.cpu_baseline == "on" else None
    dom = h["kernels"][h["dominant"]]
    line = {
        "metric": METRIC,
        "value": round(h["value"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(h["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": h["config"],
        "roofline": {k: dom[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic", "kernel")},
        "cpu_baseline": cpu,
        "fraction_of_bf16_peak": round(h["value"] / PEAK_BF16_TFLOPS, 4),
        "peaks": peaks,
        "kernels": h["kernels"],
        "kernel_ms_total": {k: {"launches": v[0], "ms": round(v[1], 4)} for k, v in h["kernel_ms"].items()},
        "rows": rows,
        "sources": sources_digest(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
