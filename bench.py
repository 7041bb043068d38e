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


def cpu_baseline(budget_s=15.0):
    """The CPU oracle, timed on this host on a bounded sample of the prefill
    workload: q heads in order, every query row of each, until the budget is
    spent (at least one head)."""
    import numpy as np
    import oracle
    from transformer_scaled_dot_flash_amd import inputs
    from transformer_scaled_dot_flash_amd.workloads import PREFILL_HEADLINE as w
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        threads = 1
    q, k, v = w.make_inputs()
    Q, K, V = (inputs.as_f64(x, w.dtype) for x in (q, k, v))
    rows = np.arange(0, w.T_q)
    flop_per_head = sum(4 * w.D * (int(i) + 1) for i in rows)
    done = 0
    t0 = time.perf_counter()
    for h in range(w.H_q):
        oracle.attention(Q, K, V, w.scale, w.causal, rows=rows, heads=[h])
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {
        "value": round(done * flop_per_head / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} of {w.H_q} q heads x all {rows.size} query rows of the "
                  f"T=8192 causal GQA prefill, float64 three-stage oracle, {dt:.1f} s",
    }


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
}
# profiles --summarize writes when no names are given
DEFAULT_SUMMARY = ["prefill_bf16_T8192_D128_gqa", "decode_bf16_B64_T4096_D128",
                   "decode_paged_bf16_B64_T4096_D128_page16", "qkv_project_bf16_T8192_dmodel4096_N6144"]


def algorithmic_bytes(name):
    from transformer_scaled_dot_flash_amd.workloads import DECODE_HEADLINE as wd
    from transformer_scaled_dot_flash_amd.workloads import PREFILL_HEADLINE as wp
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


def summarize(trace_dir, fetch_dir, write_dir, copy_mib, command_note, names=None):
    """Turn rocprofv3 CSV output (a --kernel-trace --stats run and two --pmc
    runs, FETCH_SIZE then WRITE_SIZE, each with a device copy of copy_mib MiB
    for calibration) into the summaries kept under profiles/."""
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
        rec = {
            "kernel": st["Name"],
            "source_sha256": digest,
            "calls": int(st["Calls"]),
            "avg_duration_us": round(float(st["AverageNs"]) / 1e3, 2),
            "min_duration_us": round(float(st["MinNs"]) / 1e3, 2),
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
        (PROFILES / f"{name}_traffic.json").write_text(json.dumps(rec, indent=1) + "\n")
        md = [f"# {name}", "", f"Kernel: `{st['Name']}`", "",
              "Commands (from the repository root on the GPU host):", "", "```", command_note, "```", "",
              "| figure | value |", "|---|---|",
              f"| dispatches | {rec['calls']} |",
              f"| average duration (kernel trace) | {rec['avg_duration_us']} us |",
              f"| minimum duration | {rec['min_duration_us']} us |",
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
    print(f"wrote profiles/{name}_counters.md")


PAGE_SIZE = 16


def profile_traffic(name):
    """HBM bytes per launch from profiles/<name>_traffic.json, or None when the
    kernel source changed since the counters were taken."""
    _, files = KERNELS[name]
    csrc = ROOT / "transformer_scaled_dot_flash_amd" / "csrc"
    return traffic_from_profile(name, source_digest([csrc / f for f in files]))
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
    table = perm.view(B, per).to(torch.int32).contiguous()
    lens = torch.full((B,), T, dtype=torch.int32, device=dev)
    q2 = qd.view(B, wd.H_q, D)
    o2 = torch.empty_like(q2)
    ws_bytes = abi.attn_fwd_decode_paged_workspace_bytes(B, wd.H_q, H_kv, D, PAGE_SIZE, per, 0)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

    def run():
        abi.attn_fwd_decode_paged(q2, kpool, vpool, o2, table, lens, B, wd.H_q, H_kv, D, PAGE_SIZE,
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
                               f"pages of {PAGE_SIZE} tokens in a shuffled pool of {n_pages}",
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


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-counters":
        # python bench.py --summarize-counters "commands" DIR [DIR ...]
        summarize_counters(sys.argv[3:], sys.argv[2])
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
    ap.add_argument("--only", choices=["prefill", "decode", "paged", "window", "varlen", "qkv"],
                    default=None, help="time one part only (for profiling runs)")
    ap.add_argument("--no-paged", action="store_true", help="skip the paged-KV decode line")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the sliding-window, packed-batch and QKV-projection lines")
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

    def run_decode():
        abi.attn_fwd_decode(qd, kd, vd, od, wd.B, wd.H_q, wd.H_kv, 1, wd.T_kv, wd.D, False, wd.scale,
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
                        "decode: B=64 H_q=32 H_kv=8 T_q=1 T_kv=4096 D=128 bf16",
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
    if not args.no_cpu_baseline and do_p:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
