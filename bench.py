"""Benchmark of the attention forward hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  * prefill: Llama-3-8B-shaped causal GQA, B=1 H_q=32 H_kv=8 T=8192 D=128,
    bf16 (attn_fwd_prefill, one kernel);
  * decode:  B=64 H_q=32 H_kv=8, one query token against 4096 cached keys,
    D=128, bf16 (attn_fwd_decode; the 512 (batch, kv head) groups fill the
    GPU, so one split kernel writes O and no combine pass runs).
Inputs are seeded N(0,1) tensors, resident in HBM before timing starts.

Prints one JSON line.  ``value`` is the prefill throughput in TFLOP/s with
causal FLOPs counted once (4*D per visible (query, key) pair per q head);
the decode KV-read rate in GB/s is reported beside it.  Kernel durations come
from HIP events recorded on the stream the kernels run on.

Beside the step: lines for the paged decode, sliding window, packed batch,
QKV projection, the three small workloads (B1 H1 T128 fp32, B1 H4 T128,
B4 H12 T1024) and a long-context decode whose keys are split (B=4,
T_kv=32768); measured ceilings (register-fed MFMA loop, 1 GiB streaming
read, shader clock during the prefill) beside the published peaks; the
timed outputs of the prefill (the heads the CPU baseline computed) and of
the decode compared with the oracle (max|dO|, relative Frobenius error, bf16
floor).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "attention fwd TFLOP/s (causal GQA T=8K prefill); decode KV-read GB/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_F32_VALU_TFLOPS = 157.3  # MI355X fp32 vector (256 CUs, 2.4 GHz)
PROFILES = ROOT / "profiles"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def percentiles_us(ms, what):
    """p10 / median / p90 of per-launch times given in milliseconds, in us."""
    t = sorted(ms)
    pick = lambda q: round(t[min(len(t) - 1, int(q * (len(t) - 1) + 0.5))] * 1e3, 2)
    return {f"p10_{what}_us": pick(0.1), f"median_{what}_us": pick(0.5), f"p90_{what}_us": pick(0.9)}


def source_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        h.update(Path(p).read_bytes())
    return h.hexdigest()


def traffic_from_profile(name, digest):
    """Measured HBM bytes per launch from the committed counter summary, or
    None when it is missing or was taken on different kernel source."""
    f = PROFILES / f"{name}_traffic.json"
    if not f.exists():
        return None
    d = json.loads(f.read_text())
    if d.get("source_sha256") != digest:
        return None
    return d.get("hbm_bytes_per_launch")


def counters_from_profile(name, digest):
    """Matrix-core busy fraction and shader clock from the committed shader
    counters of a kernel (profiles/<name>_counters.json), or None when they
    are missing or were taken on different kernel source."""
    f = PROFILES / f"{name}_counters.json"
    if not f.exists():
        return None
    d = json.loads(f.read_text())
    if d.get("source_sha256") != digest:
        return None
    busy = d["counters_per_dispatch"].get("SQ_VALU_MFMA_BUSY_CYCLES")
    cyc = d.get("shader_cycles_per_launch")
    return {"mfma_busy": round(busy / (cyc * 1024), 3) if busy and cyc else None,
            "shader_clock_ghz": d.get("shader_clock_ghz"), "source": f"profiles/{name}_counters.md"}


def cpu_info():
    """Host facts for the CPU baseline: logical CPUs, CPUs this process may
    run on, the BLAS thread pool numpy uses, and the CPU model."""
    info = {"host_logical_cpus": os.cpu_count(), "affinity_cpus": None, "blas_threads": None,
            "cpu_model": None}
    try:
        info["affinity_cpus"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        pass
    try:
        from threadpoolctl import threadpool_info
        info["blas_threads"] = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        pass
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                info["cpu_model"] = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return info


def cpu_baseline(budget_s=15.0):
    """The CPU oracle, timed on this host on a bounded sample of the prefill
    workload: q heads in order, every query row of each, until the budget is
    spent (at least one head).  Returns (record, {head: oracle output})."""
    import numpy as np
    import oracle
    from transformer_scaled_dot_flash_amd import inputs
    from transformer_scaled_dot_flash_amd.workloads import PREFILL_HEADLINE as w
    q, k, v = w.make_inputs()
    Q, K, V = (inputs.as_f64(x, w.dtype) for x in (q, k, v))
    rows = np.arange(0, w.T_q)
    flop_per_head = sum(4 * w.D * (int(i) + 1) for i in rows)
    done = 0
    outs = {}
    t0 = time.perf_counter()
    for h in range(w.H_q):
        outs[h] = oracle.attention(Q, K, V, w.scale, w.causal, rows=rows, heads=[h])[0, 0]
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    ci = cpu_info()
    rec = {
        "value": round(done * flop_per_head / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": ci["affinity_cpus"] or ci["host_logical_cpus"],
        "kind": "oracle",
        "sample": f"{done} of {w.H_q} q heads x all {rows.size} query rows of the "
                  f"T=8192 causal GQA prefill, float64 three-stage oracle, {dt:.1f} s "
                  f"(the oracle forms each head's full 8192 x 8192 score block before masking, "
                  f"so it executes about twice the causal FLOPs it is credited with)",
        **ci,
    }
    return rec, outs


def parity_stats(got, want):
    """max|dO|, relative Frobenius error and the bf16 floor
    max|bf16_RNE(O_ref) - O_ref| (the error of a correctly rounded output)."""
    import numpy as np
    from transformer_scaled_dot_flash_amd import inputs
    err = float(np.max(np.abs(got - want)))
    rel = float(np.linalg.norm(got - want) / np.linalg.norm(want))
    r = inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(want.astype(np.float32))).astype(np.float64)
    floor = float(np.max(np.abs(r - want)))
    return {"max_abs_err": float(f"{err:.4g}"), "rel_frobenius": float(f"{rel:.4g}"),
            "bf16_floor": float(f"{floor:.4g}"), "tolerance": 1.5e-2, "pass": err <= 1.5e-2}


KERNELS = {
    # name in profiles/ : (mangled kernel-name substring, source files)
    # prefill<D=128, causal, contiguous, RB=1, BN=128, 8 waves>; decode<D=128, contiguous / paged>
    "prefill_bf16_T8192_D128_gqa": ("prefill_bf16_kernelILi128ELb1ELb0ELi1ELi128ELi8E",
                                    ["prefill_bf16.hip", "kernel_common.h"]),
    "decode_bf16_B64_T4096_D128": ("decode_split_kernelILi128ELb0E", ["decode_bf16.hip", "kernel_common.h"]),
    "decode_paged_bf16_B64_T4096_D128_page16": ("decode_split_kernelILi128ELb1E",
                                                ["decode_bf16.hip", "kernel_common.h"]),
    "qkv_project_bf16_T8192_dmodel4096_N6144": ("qkv_project_kernelILi128E", ["qkv_bf16.hip", "kernel_common.h"]),
    # the sliding-window line runs the same instantiation as the main prefill (taken from a --only window run)
    "window_prefill_bf16_T8192_W4096_D128_gqa": ("prefill_bf16_kernelILi128ELb1ELb0ELi1ELi128ELi8E",
                                                 ["prefill_bf16.hip", "kernel_common.h"]),
    # prefill<D=128, causal, packed, RB=1, BN=64, 4 waves>
    "varlen_prefill_bf16_32K_tokens_D128_gqa": ("prefill_bf16_kernelILi128ELb1ELb1ELi1ELi64ELi4E",
                                                ["prefill_bf16.hip", "kernel_common.h"]),
    # prefill<D=64, causal, contiguous, RB=1, BN=64, 8 waves, 4 per EU, 2 key groups>: the GPT-2-small workload
    "prefill_bf16_gpt2s_B4_H12_T1024_D64": ("prefill_bf16_kernelILi64ELb1ELb0ELi1ELi64ELi8ELi4ELi2E",
                                            ["prefill_bf16.hip", "kernel_common.h"]),
    # long-context decode with split keys: split pass and combine pass
    "decode_split_bf16_B4_T32768_D128": ("decode_split_kernelILi128ELb0E", ["decode_bf16.hip", "kernel_common.h"]),
    "decode_combine_bf16_B4_T32768_D128": ("decode_combine_kernel<128>", ["decode_bf16.hip", "kernel_common.h"]),
}
# profiles --summarize writes when no names are given
DEFAULT_SUMMARY = ["prefill_bf16_T8192_D128_gqa", "decode_bf16_B64_T4096_D128",
                   "decode_paged_bf16_B64_T4096_D128_page16", "qkv_project_bf16_T8192_dmodel4096_N6144"]


def algorithmic_bytes(name):
    from transformer_scaled_dot_flash_amd.workloads import DECODE_HEADLINE as wd
    from transformer_scaled_dot_flash_amd.workloads import PREFILL_HEADLINE as wp
    if name.startswith("prefill_bf16_gpt2s"):
        from transformer_scaled_dot_flash_amd.workloads import BY_ORDINAL
        return BY_ORDINAL[3].bytes()
    if name.startswith("decode_split"):
        B, H_q, H_kv, T, D, S = LONG_DECODE
        return 2 * (2 * B * H_kv * T * D + B * H_q * D) + B * H_q * S * (D + 2) * 4  # K, V, Q; partials written
    if name.startswith("decode_combine"):
        B, H_q, H_kv, T, D, S = LONG_DECODE
        return B * H_q * S * (D + 2) * 4 + 2 * B * H_q * D  # partials read, O written
    if name.startswith("prefill") or name.startswith("window_prefill"):
        return wp.bytes()  # the window line reads and writes the same tensors
    if name.startswith("varlen_prefill"):
        H_q, H_kv, D = 32, 8, 128
        n_seq = len(varlen_lengths())
        return 2 * VARLEN_TOKENS * (2 * H_q + 2 * H_kv) * D + 2 * (n_seq + 1) * 4  # bf16 Q, O, K, V; cu_seqlens
    if name.startswith("decode_paged"):
        return wd.bytes() + wd.B * (wd.T_kv // PAGE_SIZE) * 4 + wd.B * 4  # + block table and lengths
    if name.startswith("decode"):
        return wd.bytes()
    if name.startswith("qkv"):
        M, dm, N = 8192, 4096, 6144
        return 2 * (M * dm + N * dm + M * N)  # X, W read once; Q, K, V written once
    raise KeyError(name)


def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def timed_dispatches(trace_dir, sub, n_timed):
    """Durations (us) of the last n_timed dispatches of the kernel whose name
    contains sub in a --kernel-trace run: the bench's timed calls come after
    its warm-up, so these are the dispatches its events measured."""
    import glob
    rows = _csv_rows(glob.glob(f"{trace_dir}/**/*kernel_trace.csv", recursive=True)[0])
    d = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows if sub in r["Kernel_Name"])
    return [(e - b) / 1e3 for b, e in d[-n_timed:]]


def bench_line_from_log(log_path):
    """The JSON line a profiled bench run printed (or None)."""
    try:
        for line in Path(log_path).read_text().splitlines():
            if line.startswith("{"):
                return json.loads(line)
    except OSError:
        pass
    return None


def bench_event_us(line, name):
    """The bench's HIP-event average for the line a profile covers."""
    if not line:
        return None
    path = {
        "prefill_bf16_T8192_D128_gqa": ("roofline", "avg_launch_us"),
        "decode_bf16_B64_T4096_D128": ("decode", "roofline", "avg_call_us"),
        "decode_paged_bf16_B64_T4096_D128_page16": ("paged_decode", "roofline", "avg_call_us"),
        "qkv_project_bf16_T8192_dmodel4096_N6144": ("qkv_projection", "roofline", "avg_launch_us"),
        "window_prefill_bf16_T8192_W4096_D128_gqa": ("window_prefill", "roofline", "avg_launch_us"),
        "varlen_prefill_bf16_32K_tokens_D128_gqa": ("varlen_prefill", "roofline", "avg_launch_us"),
        "prefill_bf16_gpt2s_B4_H12_T1024_D64": ("small_prefill", "gpt2s_causal_bf16_B4_H12_T1024_D64",
                                                "roofline", "avg_launch_us"),
        "decode_split_bf16_B4_T32768_D128": ("long_decode", "roofline", "avg_call_us"),
        "decode_combine_bf16_B4_T32768_D128": ("long_decode", "roofline", "avg_call_us"),
    }.get(name)
    d = line
    for k in path or ():
        if not isinstance(d, dict) or k not in d:
            return None
        d = d[k]
    return d if isinstance(d, (int, float)) else None


def summarize(trace_dir, fetch_dir, write_dir, copy_mib, command_note, names=None, n_timed=20):
    """Turn rocprofv3 CSV output (a --kernel-trace --stats run and two --pmc
    runs, FETCH_SIZE then WRITE_SIZE, each with a device copy of copy_mib MiB
    for calibration) into the summaries kept under profiles/.  Durations are
    reported over all dispatches and over the last n_timed (the bench's timed
    calls, after its warm-up)."""
    import glob
    stats = _csv_rows(glob.glob(f"{trace_dir}/**/*kernel_stats.csv", recursive=True)[0])

    def counter(d, name):
        out = {}
        for r in _csv_rows(glob.glob(f"{d}/**/*counter_collection.csv", recursive=True)[0]):
            if r["Counter_Name"] == name:
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in out.items()}

    def largest_copy(d, name):
        # the calibration copy is the largest copy dispatch of the run (small
        # host-to-device copies, e.g. of cu_seqlens, also run as copy kernels)
        vals = [float(r["Counter_Value"])
                for r in _csv_rows(glob.glob(f"{d}/**/*counter_collection.csv", recursive=True)[0])
                if r["Counter_Name"] == name and "copyBuffer" in r["Kernel_Name"]]
        return max(vals) if vals else None

    fetch = counter(fetch_dir, "FETCH_SIZE")
    write = counter(write_dir, "WRITE_SIZE")
    copy_bytes = copy_mib << 20

    def pick(d, sub):
        ks = [k for k in d if sub in k]
        return d[ks[0]] if ks else None

    f_copy = largest_copy(fetch_dir, "FETCH_SIZE")
    w_copy = largest_copy(write_dir, "WRITE_SIZE")
    f_scale = copy_bytes / (f_copy * 1024.0)
    w_scale = copy_bytes / (w_copy * 1024.0)
    csrc = ROOT / "transformer_scaled_dot_flash_amd" / "csrc"
    algo = {name: algorithmic_bytes(name) for name in (names or DEFAULT_SUMMARY)}
    for name in (names or DEFAULT_SUMMARY):
        sub, files = KERNELS[name]
        st = [r for r in stats if sub in r["Name"]]
        if not st or pick(fetch, sub) is None or pick(write, sub) is None:
            continue
        st = st[0]
        fk, wk = pick(fetch, sub), pick(write, sub)
        fetch_b = fk * 1024.0 * f_scale
        write_b = wk * 1024.0 * w_scale
        digest = source_digest([csrc / f for f in files])
        timed = timed_dispatches(trace_dir, sub, n_timed)
        tsorted = sorted(timed)
        rec = {
            "kernel": st["Name"],
            "source_sha256": digest,
            "calls": int(st["Calls"]),
            "avg_duration_us": round(float(st["AverageNs"]) / 1e3, 2),
            "min_duration_us": round(float(st["MinNs"]) / 1e3, 2),
            "timed_dispatches": len(timed),
            "avg_timed_us": round(sum(timed) / max(len(timed), 1), 2),
            "median_timed_us": round(tsorted[len(tsorted) // 2], 2) if timed else None,
            "fetch_size_kib_raw": fk,
            "write_size_kib_raw": wk,
            "copy_calibration": {"bytes_each_way": copy_bytes, "fetch_kib_raw": f_copy,
                                 "write_kib_raw": w_copy, "fetch_scale": round(f_scale, 4),
                                 "write_scale": round(w_scale, 4)},
            "hbm_fetch_bytes_per_launch": round(fetch_b),
            "hbm_write_bytes_per_launch": round(write_b),
            "hbm_bytes_per_launch": round(fetch_b + write_b),
            "algorithmic_bytes_per_launch": algo[name],
        }
        ev = bench_event_us(bench_line_from_log(f"{trace_dir}.log"), name)
        if ev is not None:
            rec["bench_event_avg_us_same_run"] = ev
        (PROFILES / f"{name}_traffic.json").write_text(json.dumps(rec, indent=1) + "\n")
        md = [f"# {name}", "", f"Kernel: `{st['Name']}`", "",
              "Commands (from the repository root on the GPU host):", "", "```", command_note, "```", "",
              "| figure | value |", "|---|---|",
              f"| dispatches | {rec['calls']} |",
              f"| average duration (kernel trace, all dispatches incl. warm-up) | {rec['avg_duration_us']} us |",
              f"| average / median of the last {rec['timed_dispatches']} dispatches (the bench's timed calls) | "
              f"{rec['avg_timed_us']} / {rec['median_timed_us']} us |",
              f"| minimum duration | {rec['min_duration_us']} us |",
              *([f"| the bench's own HIP-event average in the same run | {ev} us |"] if ev is not None else []),
              f"| FETCH_SIZE raw / dispatch | {fk:.0f} KiB |",
              f"| WRITE_SIZE raw / dispatch | {wk:.0f} KiB |",
              f"| copy calibration ({copy_mib} MiB read + written) | FETCH x{f_scale:.3f}, WRITE x{w_scale:.3f} |",
              f"| HBM bytes fetched / launch (scaled) | {fetch_b / 2**20:.1f} MiB |",
              f"| HBM bytes written / launch (scaled) | {write_b / 2**20:.1f} MiB |",
              f"| algorithmic bytes / launch | {algo[name] / 2**20:.1f} MiB |",
              f"| source sha256 (kernel + common header) | `{digest[:16]}...` |", ""]
        (PROFILES / f"{name}.md").write_text("\n".join(md))
        print(f"wrote profiles/{name}.md")


def summarize_counters(dirs, command_note, name="prefill_bf16_T8192_D128_gqa"):
    """Shader-counter summary of one kernel from rocprofv3 --pmc runs (each a
    directory of CSV output): averages per dispatch, plus the derived shader
    clock (GRBM_GUI_ACTIVE is summed over the 8 XCDs) and the fraction of SIMD
    cycles the matrix cores were busy."""
    import glob
    sub = KERNELS[name][0]
    per = {}
    dur = {}
    for d in dirs:
        for r in _csv_rows(glob.glob(f"{d}/**/*counter_collection.csv", recursive=True)[0]):
            if sub not in r["Kernel_Name"]:
                continue
            key = (d, r["Dispatch_Id"])
            per.setdefault(r["Counter_Name"], {}).setdefault(key, 0.0)
            per[r["Counter_Name"]][key] += float(r["Counter_Value"])
            dur[key] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    avg = {c: sum(v.values()) / len(v) for c, v in per.items()}
    n_simd = 1024
    gui = {k: v / 8 for k, v in per["GRBM_GUI_ACTIVE"].items()}  # cycles per XCD
    ghz = sum(gui[k] / dur[k] for k in gui) / len(gui)
    cyc = sum(gui.values()) / len(gui)
    rows = [f"| {c} | {avg[c]:.4g} |" for c in sorted(avg)]
    derived = [
        f"| dispatches sampled | {len(gui)} |",
        f"| kernel duration under counters | {sum(dur.values()) / len(dur) / 1e3:.1f} us |",
        f"| shader cycles per launch (GRBM_GUI_ACTIVE / 8 XCDs) | {cyc:.0f} |",
        f"| shader clock while it runs | {ghz:.2f} GHz |",
    ]
    if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
        derived.append(f"| matrix cores busy (SQ_VALU_MFMA_BUSY_CYCLES / (cycles x {n_simd} SIMDs)) | "
                       f"{avg['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * n_simd):.3f} |")
    if "SQ_VALU_MFMA_COEXEC_CYCLES" in avg:
        derived.append(f"| VALU issued while matrix cores busy (fraction of busy cycles) | "
                       f"{avg['SQ_VALU_MFMA_COEXEC_CYCLES'] / avg['SQ_VALU_MFMA_BUSY_CYCLES']:.3f} |")
    if "SQ_LDS_BANK_CONFLICT" in avg:
        derived.append(f"| LDS bank-conflict cycles / LDS active cycles | "
                       f"{avg['SQ_LDS_BANK_CONFLICT'] / max(avg['SQ_LDS_IDX_ACTIVE'], 1):.4f} |")
    md = [f"# {name}: shader counters", "", f"Kernel: `{sub}...`", "",
          "Commands (from the repository root on the GPU host):", "", "```", command_note, "```", "",
          "| derived | value |", "|---|---|", *derived, "",
          "| counter (sum over instances, average per dispatch) | value |", "|---|---|", *rows, ""]
    (PROFILES / f"{name}_counters.md").write_text("\n".join(md))
    files = KERNELS[name][1]
    csrc = ROOT / "transformer_scaled_dot_flash_amd" / "csrc"
    (PROFILES / f"{name}_counters.json").write_text(json.dumps({
        "kernel": sub, "source_sha256": source_digest([csrc / f for f in files]),
        "dispatches_sampled": len(gui), "shader_cycles_per_launch": round(cyc),
        "shader_clock_ghz": round(ghz, 3), "counters_per_dispatch": {c: avg[c] for c in sorted(avg)},
    }, indent=1) + "\n")
    print(f"wrote profiles/{name}_counters.md")


PAGE_SIZE = 16


def profile_traffic(name):
    """HBM bytes per launch from profiles/<name>_traffic.json, or None when the
    kernel source changed since the counters were taken."""
    _, files = KERNELS[name]
    csrc = ROOT / "transformer_scaled_dot_flash_amd" / "csrc"
    return traffic_from_profile(name, source_digest([csrc / f for f in files]))
LONG_DECODE = (4, 32, 8, 32768, 128, 24)  # B, H_q, H_kv, T_kv, D, default split count
WINDOW = 4096                 # sliding-window line: Mistral-style 4K window
VARLEN_TOKENS = 32768         # packed-batch line: total query tokens


def time_calls(torch, stream, run, warmup, settle, steps):
    """Average and minimum duration (ms) of ``run`` over ``steps`` calls, each
    bracketed by events on ``stream``, after warm-up."""
    t_settle = time.perf_counter() + settle
    done = 0
    while done < warmup or time.perf_counter() < t_settle:
        run()
        done += 1
        if done % 50 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    return sum(ms) / steps, min(ms)


def graph_call_us(torch, dev, run_on, out, n_calls=20, reps=7):
    """GPU time per call (us) with ``n_calls`` calls captured into one HIP
    graph and replayed (no host launch cost between kernels): the median over
    ``reps`` timed replays, after a warm-up replay.  Also returns whether
    every replay left ``out`` equal, bit for bit, to an eager call's output."""
    cur = torch.cuda.current_stream(dev)
    run_on(cur)
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream(device=dev)  # default priority
    side.wait_stream(cur)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for _ in range(n_calls):
            run_on(torch.cuda.current_stream(dev))
    torch.cuda.synchronize()
    times, same = [], True
    for i in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(cur)
        g.replay()
        e1.record(cur)
        torch.cuda.synchronize()
        same = same and bool(torch.equal(out.view(torch.int16), ref.view(torch.int16)))
        if i:
            times.append(e0.elapsed_time(e1) * 1e3 / n_calls)
    return sorted(times)[len(times) // 2], same


def mfma_line(metric, workload, flops, avg, mn, kernel):
    tf = flops / (avg * 1e-3) / 1e12
    return {"metric": metric, "value": round(tf, 1), "unit": "TFLOP/s",
            "config": {"workload": workload, "flops": flops},
            "roofline": {"bound": "mfma", "kernel": kernel, "achieved": round(tf, 1),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
                         "avg_launch_us": round(avg * 1e3, 2), "min_launch_us": round(mn * 1e3, 2)}}


def window_prefill_line(abi, torch, wp, qp, kp, vp, stream, warmup, settle, steps):
    """Causal sliding window W=4096 on the T=8192 GQA prefill inputs."""
    op = torch.empty_like(qp)
    T, W = wp.T_q, WINDOW
    pairs = sum(min(i + 1, W) for i in range(T))
    flops = 4 * wp.B * wp.H_q * wp.D * pairs

    def run():
        abi.attn_fwd_prefill_window(qp, kp, vp, op, wp.B, wp.H_q, wp.H_kv, T, wp.T_kv, wp.D, W,
                                    wp.scale, abi.ATTN_BF16, stream)
    log("window prefill")
    avg, mn = time_calls(torch, stream, run, warmup, settle, steps)
    line = mfma_line("sliding-window prefill TFLOP/s",
                     f"causal GQA B=1 H_q=32 H_kv=8 T=8192 D=128 bf16, window {W}", flops, avg, mn,
                     "prefill_bf16_kernel<D=128,causal,BN=128,8 waves> (window)")
    line["roofline"]["traffic"] = profile_traffic("window_prefill_bf16_T8192_W4096_D128_gqa")
    return line


def varlen_lengths():
    """Sequence lengths of the packed-batch line: drawn once from a seeded
    uniform on [128, 4096] until VARLEN_TOKENS tokens, the last one cut."""
    import numpy as np
    rng = np.random.default_rng(2024)
    lens = []
    while sum(lens) < VARLEN_TOKENS:
        lens.append(int(rng.integers(128, 4097)))
    lens[-1] -= sum(lens) - VARLEN_TOKENS
    return [x for x in lens if x > 0]


def varlen_prefill_line(abi, torch, np, stream, dev, warmup, settle, steps):
    """Packed causal GQA batch of mixed lengths (H_q=32, H_kv=8, D=128, bf16):
    lengths drawn once from a seeded uniform on [128, 4096], 32K tokens."""
    from transformer_scaled_dot_flash_amd import inputs
    lens = varlen_lengths()
    H_q, H_kv, D = 32, 8, 128
    total = sum(lens)
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device=dev)

    def mk(seed, h):
        bits = inputs.normal(seed, (total, h, D), "bf16")
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v = mk(7001, H_q), mk(7002, H_kv), mk(7003, H_kv)
    o = torch.empty_like(q)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    flops = sum(4 * H_q * D * t * (t + 1) // 2 for t in lens)

    def run():
        abi.attn_fwd_prefill_varlen(q, k, v, o, cu, cu, len(lens), H_q, H_kv, D, total, total,
                                    max(lens), max(lens), True, 0, scale, abi.ATTN_BF16, stream)
    log(f"varlen prefill ({len(lens)} sequences)")
    avg, mn = time_calls(torch, stream, run, warmup, settle, steps)
    line = mfma_line("packed variable-length prefill TFLOP/s",
                     f"{len(lens)} causal GQA sequences, lengths U[128, 4096] (seed 2024), "
                     f"{total} tokens, H_q=32 H_kv=8 D=128 bf16", flops, avg, mn,
                     "prefill_bf16_kernel<D=128,causal,packed,BN=64,4 waves>")
    line["config"]["lengths"] = lens
    line["roofline"]["traffic"] = profile_traffic("varlen_prefill_bf16_32K_tokens_D128_gqa")
    return line


def time_paged_decode(abi, torch, wd, kd, vd, qd, od_contig, stream, dev, warmup, settle, steps):
    """The decode workload over a paged cache: the same K/V values scattered
    into shuffled pools of 16-token pages (64 * 256 pages of 4 KiB per kv
    head), one block-table row per sequence.  Returns the JSON object."""
    B, H_kv, T, D = wd.B, wd.H_kv, wd.T_kv, wd.D
    per = T // PAGE_SIZE
    n_pages = B * per
    g = torch.Generator(device="cpu").manual_seed(5005)
    perm = torch.randperm(n_pages, generator=g).to(dev)
    def scatter(x):
        logical = x.view(B, H_kv, per, PAGE_SIZE, D).permute(0, 2, 1, 3, 4).reshape(n_pages, H_kv, PAGE_SIZE, D)
        pool = torch.empty_like(logical)
        pool[perm] = logical
        return pool
    kpool, vpool = scatter(kd), scatter(vd)
    pools = [(kpool, vpool), (kpool.clone(), vpool.clone())]  # alternated: no reuse through the Infinity Cache
    n_call = [0]
    table = perm.view(B, per).to(torch.int32).contiguous()
    lens = torch.full((B,), T, dtype=torch.int32, device=dev)
    q2 = qd.view(B, wd.H_q, D)
    o2 = torch.empty_like(q2)
    ws_bytes = abi.attn_fwd_decode_paged_workspace_bytes(B, wd.H_q, H_kv, D, PAGE_SIZE, per, 0)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

    def run():
        kp_, vp_ = pools[n_call[0] % 2]
        n_call[0] += 1
        abi.attn_fwd_decode_paged(q2, kp_, vp_, o2, table, lens, B, wd.H_q, H_kv, D, PAGE_SIZE,
                                  n_pages, per, wd.scale, abi.ATTN_BF16, 0, ws, ws_bytes, stream)

    log("paged decode: warmup")
    t_settle = time.perf_counter() + settle
    done = 0
    while done < warmup or time.perf_counter() < t_settle:
        run()
        done += 1
        if done % 50 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    avg = sum(ms) / steps
    nbytes = wd.bytes() + table.numel() * 4 + lens.numel() * 4
    gbs = nbytes / (avg * 1e-3) / 1e9
    same = None
    if od_contig is not None:
        same = bool(torch.equal(o2, od_contig.view(B, wd.H_q, D)))
    log(f"paged decode: {avg * 1e3:.1f} us, {gbs:.1f} GB/s")
    return {
        "metric": "paged-KV decode KV-read GB/s",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "config": {"workload": f"decode B={B} H_q={wd.H_q} H_kv={H_kv} T_kv={T} D={D} bf16, "
                               f"pages of {PAGE_SIZE} tokens in a shuffled pool of {n_pages} "
                               "(two identical pools, alternated call by call)",
                   "bytes": nbytes},
        "roofline": {"bound": "hbm", "kernel": "decode_split_kernel<128, paged>",
                     "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": profile_traffic("decode_paged_bf16_B64_T4096_D128_page16"),
                     "avg_call_us": round(avg * 1e3, 2), "min_call_us": round(min(ms) * 1e3, 2)},
        "equals_contiguous_decode": same,
    }


def qkv_projection_line(abi, torch, np, stream, dev, warmup, settle, steps):
    """Fused QKV projection at the Llama-3-8B shape: 8192 tokens, d_model
    4096, 32 q heads + 8 kv heads of 128 (N = 6144), bf16."""
    from transformer_scaled_dot_flash_amd import inputs
    B, T, dm, H_q, H_kv, D = 1, 8192, 4096, 32, 8, 128
    N = (H_q + 2 * H_kv) * D

    def mk(seed, shape):
        bits = inputs.normal(seed, shape, "bf16")
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    x = mk(8001, (B * T, dm))
    w = mk(8002, (N, dm))
    q = torch.empty(B, H_q, T, D, dtype=torch.bfloat16, device=dev)
    k = torch.empty(B, H_kv, T, D, dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k)
    flops = 2 * B * T * dm * N

    def run():
        abi.attn_qkv_project(x, w, q, k, v, B, T, dm, H_q, H_kv, D, abi.ATTN_BF16, stream)
    log("qkv projection")
    avg, mn = time_calls(torch, stream, run, warmup, settle, steps)
    line = mfma_line("fused QKV projection TFLOP/s",
                     f"X [8192 x 4096] W [6144 x 4096] -> Q [1,32,8192,128], K, V [1,8,8192,128] bf16",
                     flops, avg, mn, "qkv_project_kernel<128>")
    line["roofline"]["traffic"] = profile_traffic("qkv_project_bf16_T8192_dmodel4096_N6144")
    return line


def small_prefill_lines(abi, torch, np, stream, dev, warmup, settle, steps):
    """The three small workloads: B1 H1 T128 D64 fp32 non-causal, B1 H4 T128
    D64 bf16 causal, and the GPT-2-small shape B4 H12 T1024 D64 bf16 causal.
    Each is timed per call (the first two are launch-latency bound)."""
    from transformer_scaled_dot_flash_amd.workloads import BY_ORDINAL
    out = {}
    for ordinal in (1, 2, 3):
        w = BY_ORDINAL[ordinal]
        q, k, v = w.make_inputs()
        if w.dtype == "bf16":
            qd, kd, vd = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev) for x in (q, k, v))
        else:
            qd, kd, vd = (torch.from_numpy(x).to(dev) for x in (q, k, v))
        od = torch.empty_like(qd)
        code = abi.ATTN_BF16 if w.dtype == "bf16" else abi.ATTN_F32

        def run_on(st, qd=qd, kd=kd, vd=vd, od=od, w=w, code=code):
            abi.attn_fwd_prefill(qd, kd, vd, od, w.B, w.H_q, w.H_kv, w.T_q, w.T_kv, w.D, w.causal, w.scale,
                                 code, st)

        def run():
            run_on(stream)
        log(f"small prefill {w.name}")
        avg, mn = time_calls(torch, stream, run, max(warmup, 20), settle, max(steps, 50))
        g_us, g_same = graph_call_us(torch, dev, run_on, od)
        tf = w.flops() / (avg * 1e-3) / 1e12
        peak = PEAK_F32_VALU_TFLOPS if w.dtype == "f32" else PEAK_BF16_TFLOPS
        line = {"metric": "prefill call latency (us) and TFLOP/s", "value": round(avg * 1e3, 2), "unit": "us",
                "tflops": round(tf, 2),
                "config": {"workload": w.name, "flops": w.flops(), "bytes": w.bytes()},
                "roofline": {"bound": "alu" if w.dtype == "f32" else "mfma",
                             "kernel": "attn_f32_row_kernel<64> (one wave per row)" if w.dtype == "f32" else "prefill_bf16_kernel<D=64,causal,BN=64,8 waves in 2 key groups>",
                             "achieved": round(tf, 2), "peak": peak, "unit": "TFLOP/s",
                             "frac": round(tf / peak, 5), "traffic": None,
                             "avg_launch_us": round(avg * 1e3, 2), "min_launch_us": round(mn * 1e3, 2)},
                # 20 calls captured into one HIP graph and replayed: GPU time per call without the
                # host's launch cost between them; the replays' output equals an eager call's
                "graph_us_per_call": round(g_us, 2), "graph_output_equals_eager": g_same}
        if ordinal == 3:
            line["roofline"]["traffic"] = profile_traffic("prefill_bf16_gpt2s_B4_H12_T1024_D64")
        out[w.name] = line
    return out


def long_decode_line(abi, torch, np, stream, dev, warmup, settle, steps):
    """Long-context decode whose default plan splits the keys: B=4 H_q=32
    H_kv=8 T_kv=32768 D=128 bf16 (32 (batch, kv head) groups, 24 splits):
    the split pass writes per-split partials, the combine pass merges them."""
    from transformer_scaled_dot_flash_amd import inputs
    B, H_q, H_kv, T, D, S_expect = LONG_DECODE
    scale = float(np.float32(1.0 / math.sqrt(D)))

    def mk(seed, shape):
        bits = inputs.normal(seed, shape, "bf16")
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev), bits
    (q, qb), (k, kb), (v, vb) = mk(9001, (B, H_q, 1, D)), mk(9002, (B, H_kv, T, D)), mk(9003, (B, H_kv, T, D))
    o = torch.empty_like(q)
    splits = abi.attn_fwd_decode_default_splits(B, H_q, H_kv, T, D)
    ws_bytes = abi.attn_fwd_decode_workspace_bytes(B, H_q, H_kv, T, D, abi.ATTN_BF16, 0)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

    kv_sets = [(k, v), (k.clone(), v.clone())]  # alternated: no reuse through the Infinity Cache
    n_call = [0]

    def run():
        k_, v_ = kv_sets[n_call[0] % 2]
        n_call[0] += 1
        abi.attn_fwd_decode(q, k_, v_, o, B, H_q, H_kv, 1, T, D, False, scale, abi.ATTN_BF16, 0, ws, ws_bytes,
                            stream)
    log(f"long decode B={B} T_kv={T} ({splits} splits)")
    avg, mn = time_calls(torch, stream, run, warmup, settle, max(steps, 50))
    kv_bytes = 2 * 2 * B * H_kv * T * D
    nbytes = kv_bytes + 2 * 2 * B * H_q * D
    gbs = nbytes / (avg * 1e-3) / 1e9
    part_bytes = 2 * B * H_q * splits * (D + 2) * 4  # partials written by the split pass, read by the combine
    line = {"metric": "long-context decode KV-read GB/s", "value": round(gbs, 1), "unit": "GB/s",
            "config": {"workload": f"decode B={B} H_q={H_q} H_kv={H_kv} T_kv={T} D={D} bf16 (two identical "
                                   "K/V caches, alternated call by call)", "splits": splits,
                       "bytes": nbytes, "partials_bytes": part_bytes,
                       "partials_share_of_bytes": round(part_bytes / nbytes, 5)},
            "roofline": {"bound": "hbm", "kernel": "decode_split_kernel<128> + decode_combine_kernel<128>",
                         "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                         "avg_call_us": round(avg * 1e3, 2), "min_call_us": round(mn * 1e3, 2)}}
    sp = profile_record("decode_split_bf16_B4_T32768_D128")
    cb = profile_record("decode_combine_bf16_B4_T32768_D128")
    if sp and cb:
        line["roofline"]["traffic"] = sp["hbm_bytes_per_launch"] + cb["hbm_bytes_per_launch"]
        line["combine_share_of_time"] = round(cb["avg_timed_us"] / (sp["avg_timed_us"] + cb["avg_timed_us"]), 4)
        line["split_kernel_us"] = sp["avg_timed_us"]
        line["combine_kernel_us"] = cb["avg_timed_us"]
    # parity of this call against the oracle (every element)
    import oracle
    torch.cuda.synchronize()
    got = inputs.bf16_bits_to_f32(o.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    want = oracle.attention(inputs.as_f64(qb, "bf16"), inputs.as_f64(kb, "bf16"), inputs.as_f64(vb, "bf16"),
                            scale, False)
    line["parity"] = parity_stats(got, want)
    return line


def profile_record(name):
    """profiles/<name>_traffic.json when it belongs to the current source."""
    f = PROFILES / f"{name}_traffic.json"
    if not f.exists():
        return None
    d = json.loads(f.read_text())
    _, files = KERNELS[name]
    csrc = ROOT / "transformer_scaled_dot_flash_amd" / "csrc"
    return d if d.get("source_sha256") == source_digest([csrc / f_ for f_ in files]) else None


def ceilings(torch, stream, dev, run_prefill=None):
    """Measured ceilings beside the published peaks: a register-fed bf16 MFMA
    loop with low-entropy operands and the same with random bf16 operands
    (TFLOP/s and shader clock of each: the power limit, and so the clock,
    depends on the operand bits), a 1 GiB streaming read (GB/s, the decode
    kernel's load pattern), and the shader clock sampled while the prefill
    runs."""
    from transformer_scaled_dot_flash_amd import probe
    probe.load_library()
    n_wg = 1024
    out = torch.empty(n_wg * 512, dtype=torch.float32, device=dev)
    cyc = torch.zeros(n_wg * 8 * 2, dtype=torch.int64, device=dev)

    def mfma_rate(fn, iters, mfma_per_iter):
        # two warm-up launches, then the median of three timed ones
        runs = []
        for i in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn(n_wg, iters, out, cyc, stream)
            e1.record(stream)
            torch.cuda.synchronize()
            if i >= 2:
                c = cyc.view(-1, 2).double()
                runs.append((e0.elapsed_time(e1), float((c[:, 0] / (c[:, 1] * 10.0)).median())))  # ref: 100 MHz
        ms, clock = sorted(runs)[1]
        return n_wg * 8 * iters * mfma_per_iter * 32768 / (ms * 1e-3) / 1e12, clock

    mfma_tf, mfma_clock = mfma_rate(probe.attn_probe_mfma, 4000, 4)
    rand_tf, rand_clock = mfma_rate(probe.attn_probe_mfma_random, 500, 32)
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.empty(4096, dtype=torch.int32, device=dev)
    times = []
    for i in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        probe.attn_probe_stream_read(src, nbytes, sink, 4096, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        if i >= 2:
            times.append(e0.elapsed_time(e1))
    res = {"mfma_bf16_tflops": round(mfma_tf, 1), "mfma_clock_ghz": round(mfma_clock, 3),
           "mfma_bf16_random_tflops": round(rand_tf, 1), "mfma_random_clock_ghz": round(rand_clock, 3),
           "stream_read_gbs": round(nbytes / (sorted(times)[len(times) // 2] * 1e-3) / 1e9, 1),
           "published_bf16_tflops": PEAK_BF16_TFLOPS, "published_hbm_gbs": PEAK_HBM_GBS,
           "published_clock_ghz": 2.4}
    del src
    if run_prefill is not None:
        # clock while the prefill runs: a one-wave sampler on a second stream
        # (default priority) shares a CU with the prefill's workgroups
        side = torch.cuda.Stream(device=dev)
        clk = torch.zeros(2, dtype=torch.int64, device=dev)
        samples = []
        for _ in range(5):
            torch.cuda.synchronize()
            run_prefill()
            run_prefill()
            with torch.cuda.stream(side):
                probe.attn_probe_clock(clk, 20000, side)  # 200 us of reference ticks
            torch.cuda.synchronize()
            samples.append(float(clk[0]) / (float(clk[1]) * 10.0))
        res["prefill_clock_ghz"] = round(sorted(samples)[len(samples) // 2], 3)
    return res


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-counters":
        # python bench.py --summarize-counters "commands" DIR DIR [NAME]
        names = [a for a in sys.argv[3:] if a in KERNELS]
        dirs = [a for a in sys.argv[3:] if a not in KERNELS]
        summarize_counters(dirs, sys.argv[2], *(names[:1]))
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize":
        # python bench.py --summarize TRACE_DIR FETCH_DIR WRITE_DIR COPY_MIB "commands" [NAME ...]
        summarize(sys.argv[2], sys.argv[3], sys.argv[4], int(sys.argv[5]), sys.argv[6], sys.argv[7:] or None)
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle", type=float, default=1.0,
                    help="minimum seconds of untimed warm-up (GPU clock settle)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "paged", "window", "varlen", "qkv", "small",
                                       "long_decode", "ceilings"],
                    default=None, help="time one part only (for profiling runs)")
    ap.add_argument("--no-paged", action="store_true", help="skip the paged-KV decode line")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the sliding-window, packed-batch, QKV-projection, small-workload "
                         "and long-decode lines")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the measured ceilings")
    ap.add_argument("--no-parity", action="store_true",
                    help="skip the oracle comparison of the decode workload's output")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one device-to-device copy of this size (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the forward shards over (batch, kv head) with no exchange; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from transformer_scaled_dot_flash_amd import attn as abi
    from transformer_scaled_dot_flash_amd.workloads import DECODE_HEADLINE as wd
    from transformer_scaled_dot_flash_amd.workloads import PREFILL_HEADLINE as wp

    abi.load_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    log("generating inputs")
    qp, kp, vp = (to_dev(x) for x in wp.make_inputs())
    op = torch.empty_like(qp)
    qd, kd, vd = (to_dev(x) for x in wd.make_inputs())
    od = torch.empty_like(qd)
    ws_bytes = abi.attn_fwd_decode_workspace_bytes(wd.B, wd.H_q, wd.H_kv, wd.T_kv, wd.D, abi.ATTN_BF16, 0)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    n_splits = abi.attn_fwd_decode_default_splits(wd.B, wd.H_q, wd.H_kv, wd.T_kv, wd.D)
    torch.cuda.synchronize()

    do_p = args.only in (None, "prefill")
    do_d = args.only in (None, "decode")
    do_pg = args.only == "paged" or (args.only is None and not args.no_paged)

    def run_prefill():
        abi.attn_fwd_prefill(qp, kp, vp, op, wp.B, wp.H_q, wp.H_kv, wp.T_q, wp.T_kv, wp.D, wp.causal,
                             wp.scale, abi.ATTN_BF16, stream)

    # The decode calls alternate between two identical copies of the 1 GiB K/V cache, so no call
    # finds its cache in the 256 MB Infinity Cache from the call before.
    kv_sets = [(kd, vd), (kd.clone(), vd.clone())] if args.only in (None, "decode") else [(kd, vd)]
    n_dec = [0]

    def run_decode():
        k_, v_ = kv_sets[n_dec[0] % len(kv_sets)]
        n_dec[0] += 1
        abi.attn_fwd_decode(qd, k_, v_, od, wd.B, wd.H_q, wd.H_kv, 1, wd.T_kv, wd.D, False, wd.scale,
                            abi.ATTN_BF16, 0, ws, ws_bytes, stream)

    # Untimed warm-up: W steps, continued until the GPU clock has settled
    # (at least --settle seconds of back-to-back work).
    log(f"warmup {args.warmup} steps, >= {args.settle} s")
    t_settle = time.perf_counter() + args.settle
    done = 0
    while done < args.warmup or time.perf_counter() < t_settle:
        if do_p:
            run_prefill()
        if do_d:
            run_decode()
        done += 1
        if done % 50 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    log(f"timing {K} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        e = ev[i]
        e[0].record(stream)
        if do_p:
            run_prefill()
        e[1].record(stream)
        e[2].record(stream)
        if do_d:
            run_decode()
        e[3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log("timed region done")

    p_ms = [e[0].elapsed_time(e[1]) for e in ev]
    d_ms = [e[2].elapsed_time(e[3]) for e in ev]
    p_avg = sum(p_ms) / K
    d_avg = sum(d_ms) / K
    p_tflops = wp.flops() / (p_avg * 1e-3) / 1e12 if do_p else None
    d_gbs = wd.bytes() / (d_avg * 1e-3) / 1e9 if do_d else None

    extra = {}
    all_extra = args.only is None and not args.no_extra
    if all_extra or args.only == "window":
        extra["window_prefill"] = window_prefill_line(abi, torch, wp, qp, kp, vp, stream, args.warmup,
                                                      args.settle, min(K, 20))
    if all_extra or args.only == "varlen":
        extra["varlen_prefill"] = varlen_prefill_line(abi, torch, np, stream, dev, args.warmup,
                                                      args.settle, min(K, 20))
    if all_extra or args.only == "qkv":
        extra["qkv_projection"] = qkv_projection_line(abi, torch, np, stream, dev, args.warmup,
                                                      args.settle, min(K, 20))
    if all_extra or args.only == "small":
        extra["small_prefill"] = small_prefill_lines(abi, torch, np, stream, dev, args.warmup,
                                                     args.settle, min(K, 20))
    if all_extra or args.only == "long_decode":
        extra["long_decode"] = long_decode_line(abi, torch, np, stream, dev, args.warmup, args.settle,
                                                min(K, 20))
    if (args.only is None and not args.no_ceilings) or args.only == "ceilings":
        log("measured ceilings")
        extra["ceilings"] = ceilings(torch, stream, dev, run_prefill if args.only is None else None)
    paged = None
    if do_pg:
        paged = time_paged_decode(abi, torch, wd, kd, vd, qd, od if do_d else None, stream, dev,
                                  args.warmup, args.settle, K)

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {n} bytes read + {n} bytes written")

    csrc = ROOT / "transformer_scaled_dot_flash_amd" / "csrc"
    prefill_digest = source_digest([csrc / "prefill_bf16.hip", csrc / "kernel_common.h"])
    decode_digest = source_digest([csrc / "decode_bf16.hip", csrc / "kernel_common.h"])

    result = {
        "metric": METRIC,
        "value": round(p_tflops, 3) if p_tflops else None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "prefill: causal GQA B=1 H_q=32 H_kv=8 T=8192 D=128 bf16 (scale 1/sqrt(128)); "
                        "decode: B=64 H_q=32 H_kv=8 T_q=1 T_kv=4096 D=128 bf16 (two identical K/V caches, "
                        "alternated call by call)",
            "prefill_flops": wp.flops(),
            "decode_bytes": wd.bytes(),
            "decode_splits": n_splits,
            "inputs": "i.i.d. N(0,1), seeded SplitMix64 + Box-Muller, rounded to bf16",
        },
    }
    if do_p:
        result["roofline"] = {
            "bound": "mfma",
            "kernel": "prefill_bf16_kernel<D=128,causal,BN=128,8 waves>",
            "achieved": round(p_tflops, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(p_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic_from_profile("prefill_bf16_T8192_D128_gqa", prefill_digest),
            # matrix cores busy and shader clock under the committed counter runs (which run a few
            # percent slower than the timed calls): the published peak assumes 100% busy at 2.4 GHz
            "counters": counters_from_profile("prefill_bf16_T8192_D128_gqa", prefill_digest),
            "avg_launch_us": round(p_avg * 1e3, 2),
            "min_launch_us": round(min(p_ms) * 1e3, 2),
            **percentiles_us(p_ms, "launch"),
        }
    if do_d:
        result["decode"] = {
            "metric": "decode KV-read GB/s",
            "value": round(d_gbs, 1),
            "unit": "GB/s",
            "roofline": {
                "bound": "hbm",
                "kernel": "decode_split_kernel<128>" + (" + decode_combine_kernel<128>" if n_splits > 1 else ""),
                "achieved": round(d_gbs, 1),
                "peak": PEAK_HBM_GBS,
                "unit": "GB/s",
                "frac": round(d_gbs / PEAK_HBM_GBS, 4),
                "traffic": traffic_from_profile("decode_bf16_B64_T4096_D128", decode_digest),
                "avg_call_us": round(d_avg * 1e3, 2),
                "min_call_us": round(min(d_ms) * 1e3, 2),
                **percentiles_us(d_ms, "call"),
            },
        }
    if paged is not None:
        result["paged_decode"] = paged
    result.update(extra)
    c = extra.get("ceilings")
    if do_p and c and c.get("mfma_bf16_random_tflops"):
        # the same achieved rate against the measured random-operand MFMA ceiling (context; `frac`
        # stays against the published peak)
        result["roofline"]["frac_of_measured_random_mfma"] = round(p_tflops / c["mfma_bf16_random_tflops"], 4)
    parity = {}
    if do_d and not args.no_parity:
        # the decode workload's output of the timed calls, every element against the oracle
        import oracle
        from transformer_scaled_dot_flash_amd import inputs
        log("decode parity (oracle)")
        qb, kb, vb = wd.make_inputs()
        want = oracle.attention(*(inputs.as_f64(x, "bf16") for x in (qb, kb, vb)), wd.scale, False)
        got = inputs.bf16_bits_to_f32(od.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
        parity["decode"] = parity_stats(got, want)
    if not args.no_cpu_baseline and do_p:
        log("cpu baseline (oracle)")
        rec, heads = cpu_baseline()
        rec["gpu_over_oracle"] = round(p_tflops / rec["value"], 1) if rec["value"] else None
        result["cpu_baseline"] = rec
        # the prefill output of the timed calls against the oracle heads just computed
        from transformer_scaled_dot_flash_amd import inputs
        hs = sorted(heads)
        got = inputs.bf16_bits_to_f32(op[0, hs].view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
        want = np.stack([heads[h] for h in hs])
        parity["prefill"] = parity_stats(got, want)
        parity["prefill"]["heads_compared"] = f"{len(hs)} of {wp.H_q} q heads, every row and feature"
    if parity:
        result["parity"] = parity
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
