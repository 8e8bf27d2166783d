"""Throughput of the vocab-parallel LM head + cross entropy on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-embed-bench]

One step = one pass of the whole hot path over one batch of the 8B-class
shard workload (N = 8192 tokens, H = 4096, V = 128256, T = 8, shard 0 =
[16032, 4096] bf16, Zipf(1.1) targets):

    masked lookup of the batch's ids on shard 0          (vp_embed_fwd)
    fused LM-head GEMM + statistics of shard 0           (vp_lmhead_ce_fwd)
    merge of the 8 shards' statistics -> loss, lse, mean  (vp_ce_combine)
    recompute, softmax - onehot, dX_0 and dW_0            (vp_lmhead_ce_bwd)

The other seven shards' statistics are the other GPUs' work in a real
deployment; they are computed once before timing.  Inputs are resident in HBM
before the timed region.  Prints one JSON line (rank 0, N = 1).

Also measured beside the step: the same CE sequence with the shard's logits stored
in HBM instead of fused (the pages' tensor-parallel baseline; --no-comparator skips
it); and, unless --no-embed-bench, the step's CE sequence on
the padded vocabulary (shard 0 = 16128 rows instead of 16032), the embedding-heavy
lookup (65536 Zipf ids on a [64000, 4096] shard) and its weight gradient, each
against HBM bandwidth; the same CE sequence at the small LM, the large-vocab shard
and the embedding-heavy T=1 cross entropy unless --no-other-workloads; and yardsticks (vendor
GEMM, copy, fill) unless --no-yardsticks.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 flop/clk/CU, dense
PEAK_HBM_GBS = 8000.0
METRIC = "tokens/sec fused LM-head+vocab-parallel CE fwd+bwd; % bf16 MFMA peak"


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "traffic_ce_step_shard_8b.txt")
COPY_BYTES = 2**30          # the yardsticks' device copy: 1 GiB read + 1 GiB written


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# the sources the CE sequence's kernels are compiled from (and the build flags)
CE_SOURCES = ("common.hpp", "gemm.hpp", "gemm_small.hpp", "launch.hpp", "ce_fwd.hip",
              "ce_combine.hip", "ce_bwd.hip")


# the sources the lookup's and its gradient's kernels are compiled from
LOOKUP_SOURCES = ("common.hpp", "launch.hpp", "embed.hip", "embed_bwd.hip")


def kernel_source_hash(sources=CE_SOURCES) -> str:
    """Hash of everything that decides the kernels' code: their sources (the CE sequence's
    by default, comments and layout stripped), the compile command and the device flags of
    the build script.  The counter summaries record it, so that a reading taken on other
    kernels is never reported."""
    import importlib.util
    import inspect
    spec = importlib.util.spec_from_file_location(
        "vp_build", os.path.join(ROOT, "vocab_lm_head_amd", "build.py"))
    build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(build)
    h = hashlib.sha256()
    for f in sources:
        h.update(f.encode())
        with open(os.path.join(ROOT, "vocab_lm_head_amd", "csrc", f)) as fh:
            src = fh.read()
        # comments and layout do not change the code: only the tokens are hashed
        src = re.sub(r"/\*.*?\*/|//[^\n]*", " ", src, flags=re.S)
        h.update(" ".join(src.split()).encode())
    h.update(inspect.getsource(build._compile).encode())
    h.update(repr((build.ARCH, build.DEVICE_FLAGS)).encode())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per CE launch from the committed counter summary, if the kernels are
    still the ones it was measured on; else None."""
    try:
        txt = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    h = re.search(r"^kernel_source_hash: (\w+)", txt, re.M)
    b = re.search(r"^traffic_bytes_per_launch: (\d+)", txt, re.M)
    if not h or not b or h.group(1) != kernel_source_hash():
        return None
    return int(b.group(1))


CE_KERNELS = ("CeStatsEpilogue", "merge_slices_kernel", "combine_kernel", "mean_kernel",
              "transpose_bf16_kernel", "DlogitsEpilogue", "StoreTransposedEpilogue",
              "gemm_nt_splitk_store_kernel", "sum_splits_kernel", "gemm_nt_small_kernel")


def short_kernel_name(name: str) -> str:
    """A kernel's short name in profiler output: the epilogue of a GEMM instance
    (gemm_nt_kernel<...Epilogue>), otherwise the function's own name."""
    m = re.search(r"gemm_nt_kernel<(?:[\w:]*::)?(?:\(anonymous namespace\)::)?(\w+)(?:<[^<>]*>)?\s*>",
                  name)
    if m:
        return m.group(1)
    m = re.search(r"(\w+)(?:<[^<>()]*>)?\(", name)
    return m.group(1) if m else name


LOOKUP_TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "traffic_lookup_embedding_heavy.txt")
EMBED_HEAVY_GRID = "4194304"   # the embedding-heavy lookup's launch: 65536 rows, 4 per workgroup
LOOKUP_GRAD_KERNELS = ("radix_count_kernel", "radix_scan_kernel", "radix_scatter_kernel",
                       "radix_count_kernel", "radix_scan_kernel", "radix_scatter_kernel",
                       "segment_sum_kernel", "segment_fixup_kernel")


def recorded_lookup_traffic():
    """HBM bytes of one embedding-heavy lookup and of one call of its weight gradient, from
    the committed counter summary, if the kernels are still the ones it was measured on."""
    try:
        txt = open(LOOKUP_TRAFFIC_PROFILE).read()
    except OSError:
        return {}
    h = re.search(r"^kernel_source_hash: (\w+)", txt, re.M)
    if not h or h.group(1) != kernel_source_hash(LOOKUP_SOURCES):
        return {}
    out = {}
    for key in ("lookup", "gradient"):
        b = re.search(rf"^{key}_traffic_bytes: (\d+)", txt, re.M)
        if b:
            out[key] = int(b.group(1))
    return out


def _pmc_rows_grid(path, counter):
    """[(dispatch id, short kernel name, grid size, value)] of one counter."""
    acc = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        k = int(r["Dispatch_Id"])
        acc.setdefault(k, [short_kernel_name(r["Kernel_Name"]), r.get("Grid_Size", ""), 0.0])[2] += \
            float(r["Counter_Value"])
    return sorted((k, v[0], v[1], v[2]) for k, v in acc.items())


def reduce_pmc_lookup(fetch_csv, write_csv, cmd_fetch, cmd_write):
    """Summarise two counter runs of this script (FETCH_SIZE, WRITE_SIZE) into
    LOOKUP_TRAFFIC_PROFILE: the last embedding-heavy lookup launch and the last call of its
    weight gradient (its eight kernels), each counter scaled by its reading for the 1 GiB
    device copy of the yardsticks."""
    sel = {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _pmc_rows_grid(path, name)
        copies = [v for _, k, _, v in rows if "copyBuffer" in k and v > 0.5 * COPY_BYTES / 1024]
        factor = (COPY_BYTES / 1024) / (sum(copies) / len(copies))
        i_look = max(i for i, (_, k, g, _) in enumerate(rows)
                     if k == "embed_kernel" and g == EMBED_HEAVY_GRID)
        i_fix = max(i for i, (_, k, _, _) in enumerate(rows) if k == "segment_fixup_kernel")
        grad = rows[i_fix - len(LOOKUP_GRAD_KERNELS) + 1:i_fix + 1]
        assert tuple(k for _, k, _, _ in grad) == LOOKUP_GRAD_KERNELS, "unexpected kernel sequence"
        sel[name] = (factor, rows[i_look][3], [(k, v) for _, k, _, v in grad], len(copies))
    f_f, look_f, grad_f, nf = sel["FETCH_SIZE"]
    f_w, look_w, grad_w, nw = sel["WRITE_SIZE"]
    look = (look_f * f_f + look_w * f_w) * 1024
    grad = (sum(v for _, v in grad_f) * f_f + sum(v for _, v in grad_w) * f_w) * 1024
    lines = ["# HBM traffic of the embedding-heavy lookup (65536 Zipf(1.0) ids on shard 0 = [64000, 4096]",
             "# of V=256000) and of one call of its weight gradient, from rocprofv3 counters.",
             "# commands (from the repository root):", f"#   {cmd_fetch}", f"#   {cmd_write}",
             "#   python3 bench.py --reduce-pmc-lookup <fetch csv> <write csv>   (writes this file)",
             "# Each counter is scaled by its reading for the 1 GiB device copy of the yardsticks.",
             f"kernel_source_hash: {kernel_source_hash(LOOKUP_SOURCES)}",
             f"copy_calibration: FETCH factor {f_f:.4f} ({nf} copies), WRITE factor {f_w:.4f} ({nw} copies)",
             "", "kernel                      FETCH_KiB    WRITE_KiB   (raw counter)",
             f"{'embed_kernel':26s} {look_f:12.0f} {look_w:12.0f}"]
    for (k, vf), (_, vw) in zip(grad_f, grad_w):
        lines.append(f"{k:26s} {vf:12.0f} {vw:12.0f}")
    lines += ["", f"lookup_traffic_bytes: {int(round(look))}",
              f"gradient_traffic_bytes: {int(round(grad))}"]
    with open(LOOKUP_TRAFFIC_PROFILE, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _pmc_rows(path, counter):
    """[(dispatch id, short kernel name, value)] of one counter, summed over its dimensions."""
    acc = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        k = int(r["Dispatch_Id"])
        acc.setdefault(k, [short_kernel_name(r["Kernel_Name"]), 0.0])[1] += float(r["Counter_Value"])
    return sorted((k, v[0], v[1]) for k, v in acc.items())


def reduce_pmc(fetch_csv, write_csv, cmd_fetch, cmd_write):
    """Summarise two counter runs of this script into TRAFFIC_PROFILE: the last step's CE
    kernels' FETCH_SIZE and WRITE_SIZE (KiB), each scaled by the same counter's reading
    for the 1 GiB device copy of known size."""
    out = {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _pmc_rows(path, name)
        copies = [v for _, k, v in rows if "copyBuffer" in k and v > 0.5 * COPY_BYTES / 1024]
        factor = (COPY_BYTES / 1024) / (sum(copies) / len(copies))
        last = max(i for i, (_, k, _) in enumerate(rows) if k == "CeStatsEpilogue")
        step = []
        for _, k, v in rows[last:]:
            if k == "embed_kernel" or k not in CE_KERNELS:
                break
            step.append((k, v))
        out[name] = (factor, step, len(copies))
    f_fetch, step_f, nf = out["FETCH_SIZE"]
    f_write, step_w, nw = out["WRITE_SIZE"]
    total = sum(v for _, v in step_f) * f_fetch * 1024 + sum(v for _, v in step_w) * f_write * 1024
    lines = ["# HBM traffic of one fused CE launch (vp_lmhead_ce_fwd + vp_ce_combine + vp_lmhead_ce_bwd)",
             "# at the 8B-class shard (N=8192, H=4096, shard [16032, 4096]), from rocprofv3 counters.",
             "# commands (from the repository root):",
             f"#   {cmd_fetch}", f"#   {cmd_write}",
             "#   python3 bench.py --reduce-pmc <fetch csv> <write csv>   (writes this file)",
             "# Each counter is scaled by its reading for the 1 GiB device copy of the yardsticks",
             "# (known: 1048576 KiB read and 1048576 KiB written).",
             f"kernel_source_hash: {kernel_source_hash()}",
             f"copy_calibration: FETCH factor {f_fetch:.4f} ({nf} copies), WRITE factor {f_write:.4f} ({nw} copies)",
             "", "kernel                      FETCH_KiB    WRITE_KiB   (raw counter, last step)"]
    for (k, vf), (_, vw) in zip(step_f, step_w):
        lines.append(f"{k:26s} {vf:12.0f} {vw:12.0f}")
    lines += ["", f"traffic_bytes_per_launch: {int(round(total))}",
              f"traffic_GB_per_launch: {total / 1e9:.4f}"]
    with open(TRAFFIC_PROFILE, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def reduce_trace(path, name, title, cmd, last=5, bench_log=None):
    """Summarise a rocprofv3 --kernel-trace CSV into profiles/<name>.txt: per kernel (short
    name and grid), the mean duration of its last `last` launches and its launch count, and
    the sum of those means over the library's kernels."""
    acc = {}
    for r in csv.DictReader(open(path)):
        grid = "x".join(r.get(k, "1") for k in ("Grid_Size_X", "Grid_Size_Y"))
        wg = r.get("Workgroup_Size_X", "")
        key = (short_kernel_name(r["Kernel_Name"]), grid, wg)
        acc.setdefault(key, []).append(
            (int(r["Start_Timestamp"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    ours = set(CE_KERNELS) | set(LOOKUP_GRAD_KERNELS) | {
        "embed_kernel", "logits_stats_kernel", "dlogits_from_logits_kernel", "rows_max_kernel"}
    rows = []
    for (k, grid, wg), v in acc.items():
        if k not in ours:
            continue
        v.sort()
        tail = [d for _, d in v[-last:]]
        rows.append((sum(tail) / len(tail), k, grid, wg, len(v)))
    rows.sort(reverse=True)
    lines = [f"# rocprofv3 kernel trace: {title}", "# command (from the repository root):",
             f"#   {cmd}",
             f"#   python3 bench.py --reduce-trace <kernel_trace csv> {name} '<title>' '<command>'",
             f"kernel_source_hash: {kernel_source_hash()}", "",
             f"## per-launch durations, mean of the last {last} launches of each kernel, microseconds"]
    for us, k, grid, wg, n in rows:
        lines.append(f"  {us:8.1f}  {k} [grid {grid} x {wg}]  (launches in run: {n})")
    lines += ["", f"sum of the listed kernels (one launch each): {sum(r[0] for r in rows):.1f} us"]
    # the CE sequence of each traced step: from the forward GEMM that follows a lookup to the
    # last kernel before the next lookup (the step's own order: lookup, fwd, combine, bwd)
    seq = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]),
                  short_kernel_name(r["Kernel_Name"])) for r in csv.DictReader(open(path)))
    spans = []
    for i, (_, _, k) in enumerate(seq):
        if k != "embed_kernel" or i + 1 >= len(seq) or seq[i + 1][2] != "CeStatsEpilogue":
            continue
        # the sequence ends with the backward's second gradient GEMM after its recompute
        j, grads = i + 1, -1
        while j + 1 < len(seq) and seq[j + 1][2] in CE_KERNELS and grads < 2:
            j += 1
            if seq[j][2] == "DlogitsEpilogue":
                grads = 0
            elif grads >= 0 and seq[j][2] in ("StoreTransposedEpilogue", "gemm_nt_splitk_store_kernel"):
                grads += 1
        if grads == 2:
            spans.append((seq[j][1] - seq[i + 1][0]) / 1e3)
    if spans:
        tail = spans[-last:]
        lines.append(f"CE sequence (forward GEMM start to dW GEMM end), last {len(tail)} steps: "
                     f"{sum(tail) / len(tail):.1f} us")
    if bench_log:   # the bench's own HIP-event figures from the same run
        for line in open(bench_log):
            if line.startswith("{") and '"roofline"' in line:
                d = json.loads(line)
                lines.append(f"bench.py HIP events in the same (profiled) run: CE sequence "
                             f"{d['roofline']['avg_launch_ms'] * 1e3:.1f} us, step "
                             f"{d['ms_per_step'] * 1e3:.1f} us")
    stats = os.path.join(os.path.dirname(path), os.path.basename(path).replace("kernel_trace", "kernel_stats"))
    if os.path.exists(stats) and stats != path:
        lines += ["", "## rocprofv3 --stats (every launch of the run, warm-up and untimed calls included)",
                  "calls  avg_us  min_us  max_us  kernel"]
        for r in csv.DictReader(open(stats)):
            k = short_kernel_name(r["Name"])
            if k in ours:
                lines.append(f"{int(r['Calls']):5d} {float(r['AverageNs']) / 1e3:7.1f} "
                             f"{float(r['MinNs']) / 1e3:7.1f} {float(r['MaxNs']) / 1e3:7.1f}  {k}")
    with open(os.path.join(ROOT, "profiles", f"{name}.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


MFMA_PROFILE = os.path.join(ROOT, "profiles", "mfma_util_shard_8b.txt")
MFMA_COUNTERS = "GRBM_GUI_ACTIVE SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA"


def reduce_mfma(path, cmd):
    """Summarise one counter run of this script (MFMA_COUNTERS with --kernel-trace) into
    MFMA_PROFILE: per GEMM kernel, its duration, the clock it ran at (GRBM_GUI_ACTIVE is
    summed over the 8 XCDs) and the share of SIMD cycles the MFMA unit was busy
    (SQ_VALU_MFMA_BUSY_CYCLES summed over 1024 SIMDs), for ours and the vendor GEMM."""
    acc = {}
    for r in csv.DictReader(open(path)):
        k = int(r["Dispatch_Id"])
        e = acc.setdefault(k, {"name": short_kernel_name(r["Kernel_Name"]),
                               "grid": r.get("Grid_Size", r.get("Grid_Size_X", "")),
                               "us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    rows = {}
    for k in sorted(acc):
        e = acc[k]
        if e.get("SQ_INSTS_MFMA", 0) == 0:
            continue
        cyc = e["GRBM_GUI_ACTIVE"] / 8
        rows.setdefault((e["name"], e["grid"]), []).append(
            (e["us"], cyc / e["us"] / 1e3, e["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024 / cyc))
    lines = ["# MFMA utilisation and clock of every GEMM kernel in one bench run (rocprofv3 counters)",
             "# command (from the repository root):", f"#   {cmd}",
             f"#   python3 bench.py --reduce-mfma <counter csv>   (writes this file)",
             "# clock = GRBM_GUI_ACTIVE / 8 XCDs / duration; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES /",
             "# 1024 SIMDs / (GRBM_GUI_ACTIVE / 8).  Durations are under the profiler (counters on).",
             "# The Cijk_* kernels are hipBLASLt's (torch.matmul yardsticks at the same shapes).",
             f"kernel_source_hash: {kernel_source_hash()}", "",
             "dispatches  avg_us  clock_GHz  mfma_busy  kernel [grid]"]
    for (name, grid), v in rows.items():
        n = len(v)
        us, ghz, busy = (sum(x[i] for x in v) / n for i in range(3))
        lines.append(f"{n:10d} {us:7.1f} {ghz:10.2f} {busy * 100:9.1f}%  {name[:70]} [{grid}]")
    with open(MFMA_PROFILE, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


LDS_PROFILE = os.path.join(ROOT, "profiles", "lds_counters_shard_8b.txt")
LDS_COUNTERS = "SQ_INSTS_MFMA SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_WAIT_INST_LDS SQ_WAVE_CYCLES"


def reduce_lds(path, cmd):
    """Summarise one counter run of this script (LDS_COUNTERS with --kernel-trace) into
    LDS_PROFILE: per GEMM kernel, LDS instructions per MFMA, the share of wave cycles spent
    waiting on LDS instructions, and the LDS bank-conflict cycles per LDS instruction."""
    acc = {}
    for r in csv.DictReader(open(path)):
        k = int(r["Dispatch_Id"])
        e = acc.setdefault(k, {"name": short_kernel_name(r["Kernel_Name"]),
                               "grid": r.get("Grid_Size", r.get("Grid_Size_X", ""))})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    rows = {}
    for k in sorted(acc):
        e = acc[k]
        if e.get("SQ_INSTS_MFMA", 0) == 0:
            continue
        rows.setdefault((e["name"], e["grid"]), []).append(
            (e["SQ_INSTS_LDS"] / e["SQ_INSTS_MFMA"], e["SQ_WAIT_INST_LDS"] / e["SQ_WAVE_CYCLES"],
             e["SQ_LDS_BANK_CONFLICT"], e["SQ_LDS_BANK_CONFLICT"] / max(1.0, e["SQ_INSTS_LDS"])))
    lines = ["# LDS use of every GEMM kernel in one bench run (rocprofv3 counters)",
             "# command (from the repository root):", f"#   {cmd}",
             f"#   python3 bench.py --reduce-lds <counter csv>   (writes this file)",
             "# lds/mfma = SQ_INSTS_LDS / SQ_INSTS_MFMA (the mainloop issues 24 ds_read_b128 per",
             "# 64 MFMAs, 0.375; epilogues add their own); lds_wait = SQ_WAIT_INST_LDS /",
             "# SQ_WAVE_CYCLES; bank_conflict = SQ_LDS_BANK_CONFLICT cycles, also per LDS instruction.",
             "# The Cijk_* kernels are hipBLASLt's (torch.matmul yardsticks at the same shapes).",
             f"kernel_source_hash: {kernel_source_hash()}", "",
             "dispatches  lds/mfma  lds_wait  bank_conflict_cycles  per_lds_inst  kernel [grid]"]
    for (name, grid), v in rows.items():
        n = len(v)
        ratio, wait, conf, per = (sum(x[i] for x in v) / n for i in range(4))
        lines.append(f"{n:10d} {ratio:9.3f} {wait * 100:8.1f}% {conf:21.0f} {per:13.4f}  "
                     f"{name[:70]} [{grid}]")
    with open(LDS_PROFILE, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _run_text(cmd, timeout=30):
    """stdout of a command, or None if it is missing or fails (information only)."""
    import subprocess
    try:
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout)
    except (OSError, subprocess.SubprocessError):
        return None
    return r.stdout if r.returncode == 0 else None


def _read(path):
    try:
        with open(path) as fh:
            return fh.read().strip()
    except OSError:
        return None


def gpu_clock_and_driver():
    """The GPU's clocks and driver as the system reports them: rocm-smi's current and
    supported engine clocks and its driver version, the amdgpu module version, the ROCm
    release; and the engine clock the CE GEMMs ran at under load, from the committed
    counter summary (GRBM_GUI_ACTIVE over the kernels' durations) when it was taken on
    the kernels as built."""
    out = {"rocm": _read("/opt/rocm/.info/version"),
           "amdgpu_module_version": _read("/sys/module/amdgpu/version")}
    txt = _run_text(["rocm-smi", "--showclocks", "--showdriverversion", "--json"])
    if txt:
        try:
            info = json.loads(txt)
            for card, d in info.items():
                if not isinstance(d, dict):
                    continue
                if card == "system":
                    out["driver_version"] = d.get("Driver version")
                    continue
                out.setdefault("clocks_at_query", {})[card] = {
                    k: v for k, v in d.items() if "clock" in k.lower() or "sclk" in k.lower()}
        except (ValueError, AttributeError):
            out["rocm_smi_raw"] = txt[:400]
    levels = _run_text(["rocm-smi", "--showclkfrq"])
    if levels:
        out["sclk_levels"] = " ".join(l.strip() for l in levels.splitlines()
                                      if "Mhz" in l or "MHz" in l)[:400]
    try:
        txt = open(MFMA_PROFILE).read()
        h = re.search(r"^kernel_source_hash: (\w+)", txt, re.M)
        if h and h.group(1) == kernel_source_hash():
            clk = {}
            for line in txt.splitlines():
                f = line.split()
                if len(f) >= 5 and f[0].isdigit() and "Epilogue" in line:
                    clk.setdefault(f[4], []).append(float(f[2]))
            out["gemm_clock_under_load_GHz"] = {k: round(sum(v) / len(v), 3) for k, v in clk.items()}
            out["gemm_clock_source"] = "profiles/mfma_util_shard_8b.txt (rocprofv3 counters)"
    except OSError:
        pass
    return out


def device_info(torch, dev):
    """The device and software versions the numbers were taken on."""
    p = torch.cuda.get_device_properties(dev)
    return {"device": p.name, "arch": getattr(p, "gcnArchName", ""),
            "compute_units": p.multi_processor_count, "hbm_GiB": round(p.total_memory / 2**30, 1),
            "hip": torch.version.hip, "torch": torch.__version__, **gpu_clock_and_driver()}


def host_cpu_info():
    """The host the oracle baseline ran on: CPU model, the cores visible to this process,
    and NumPy's BLAS (library, version, threads) as threadpoolctl sees it."""
    model = None
    txt = _read("/proc/cpuinfo") or ""
    m = re.search(r"^model name\s*:\s*(.+)$", txt, re.M)
    if m:
        model = m.group(1).strip()
    try:
        import threadpoolctl
        blas = [{k: d.get(k) for k in ("internal_api", "version", "num_threads",
                                         "threading_layer", "architecture", "filepath")}
                for d in threadpoolctl.threadpool_info()]
    except Exception:   # noqa: BLE001 -- information only
        blas = None
    return {"cpu_model": model, "logical_cpus": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS"), "numpy": np.__version__,
            "blas": blas}


def oracle_threads():
    """Threads for the oracle's BLAS: every core this process may run on, except where the
    environment sets the job's CPU share (OMP_NUM_THREADS, which a shared GPU host sets to
    the cores allotted to one GPU's job); then that share."""
    cores = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        cores = min(cores, int(env))
    return cores


def dev_bf16(torch, bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def cpu_baseline(inp, sample_tokens: int):
    """The oracle, as it stands, timed on host cores for a bounded sample of tokens."""
    import threadpoolctl

    import oracle
    import vp_inputs
    cores = oracle_threads()
    wl = inp.wl
    rng = np.random.default_rng(1234)
    rows = np.sort(rng.choice(wl.N, sample_tokens, replace=False))
    with threadpoolctl.threadpool_limits(limits=cores):
        x = vp_inputs.bf16_bits_to_f64(inp.x[rows])
        y = inp.targets[rows]
        shards = [oracle.shard_range(wl.V, wl.T, t) for t in range(wl.T)]
        w = [vp_inputs.bf16_bits_to_f64(inp.w[a:b]) for a, b in shards]
        # other shards' statistics: inputs of the timed unit (other GPUs' work), untimed
        others = [oracle.shard_stats(oracle.logits(x, w[t]), y, shards[t][0])
                  for t in range(1, wl.T)]
        g = oracle.mean_scale(inp.targets)
        t0 = time.perf_counter()
        z0 = oracle.logits(x, w[0])                                   # shard-0 forward
        st0 = oracle.shard_stats(z0, y, 0)
        stats = [st0] + others
        loss, lse, mean = oracle.combine_triples(*(np.stack(a) for a in zip(*stats)), y)
        dz0 = oracle.dz_rows(x, w[0], y, lse, 0, g)                   # shard-0 backward
        dx0, dw0 = oracle.shard_grads(x, w[0], dz0)
        dt = time.perf_counter() - t0
        host = host_cpu_info()   # inside the limits: the BLAS threads it actually used
    return {"value": sample_tokens / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "host": host,
            "sample": f"{sample_tokens} of the {wl.N} tokens (seeded choice): shard-0 forward + "
                      f"combine of 8 shards + shard-0 backward, NumPy fp64, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=8192)
    ap.add_argument("--no-embed-bench", action="store_true")
    ap.add_argument("--no-yardsticks", action="store_true")
    ap.add_argument("--no-comparator", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the small-LM, large-vocab and embedding-heavy CE timings")
    ap.add_argument("--shape-sweep", action="store_true",
                    help="time the CE sequence at the 8B-class shard over N and H instead "
                         "(one JSON line per shape) and exit")
    ap.add_argument("--reduce-mfma", metavar="COUNTER_CSV",
                    help="summarise a rocprofv3 --pmc run of this script with MFMA_COUNTERS and "
                         "--kernel-trace into profiles/ and exit (no GPU needed)")
    ap.add_argument("--reduce-lds", metavar="COUNTER_CSV",
                    help="summarise a rocprofv3 --pmc run of this script with LDS_COUNTERS and "
                         "--kernel-trace into profiles/ and exit (no GPU needed)")
    ap.add_argument("--reduce-pmc-lookup", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this "
                         "script's lookup benches into profiles/ and exit (no GPU needed)")
    ap.add_argument("--reduce-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this "
                         "script into profiles/ and exit (no GPU needed)")
    ap.add_argument("--reduce-trace", nargs=4, metavar=("TRACE_CSV", "NAME", "TITLE", "COMMAND"),
                    help="summarise a rocprofv3 --kernel-trace CSV into profiles/NAME.txt and exit "
                         "(no GPU needed)")
    ap.add_argument("--bench-log", help="with --reduce-trace: the bench output of the traced run")
    args = ap.parse_args()
    if args.reduce_trace:
        reduce_trace(*args.reduce_trace, bench_log=args.bench_log)
        return
    # the counter runs' commands, as recorded in the summaries: the output folder is the
    # one the given CSV files were written to (rocprofv3 -d <folder> -o run)
    run_args = "-o run -- python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline " \
               "--no-embed-bench --no-comparator --no-other-workloads"
    if args.reduce_mfma:
        reduce_mfma(args.reduce_mfma,
                    f"rocprofv3 --pmc {MFMA_COUNTERS} --kernel-trace --output-format csv -d "
                    f"{os.path.dirname(args.reduce_mfma)} {run_args}")
        return
    if args.reduce_lds:
        reduce_lds(args.reduce_lds,
                   f"rocprofv3 --pmc {LDS_COUNTERS} --kernel-trace --output-format csv -d "
                   f"{os.path.dirname(args.reduce_lds)} {run_args}")
        return
    if args.reduce_pmc:
        cmds = [f"rocprofv3 --pmc {c} --output-format csv -d {os.path.dirname(path)} {run_args}"
                for c, path in zip(("FETCH_SIZE", "WRITE_SIZE"), args.reduce_pmc)]
        reduce_pmc(args.reduce_pmc[0], args.reduce_pmc[1], cmds[0], cmds[1])
        return
    if args.reduce_pmc_lookup:
        look_args = "-o run -- python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline " \
                    "--no-comparator --no-other-workloads"
        cmds = [f"rocprofv3 --pmc {c} --output-format csv -d {os.path.dirname(path)} {look_args}"
                for c, path in zip(("FETCH_SIZE", "WRITE_SIZE"), args.reduce_pmc_lookup)]
        reduce_pmc_lookup(args.reduce_pmc_lookup[0], args.reduce_pmc_lookup[1], cmds[0], cmds[1])
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (each vocab "
              "shard would run on a GPU of its own). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import vocab_lm_head_amd as vp
    import vp_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    if args.shape_sweep:
        shape_sweep(torch, vp, dev)
        return

    t0 = time.time()
    inp = vp_inputs.make_inputs("shard_8b")
    wl = inp.wl
    log(f"inputs generated in {time.time() - t0:.1f}s")
    N, H, V, T, Vs = wl.N, wl.H, wl.V, wl.T, wl.Vs
    x_d = dev_bf16(torch, inp.x, dev)
    w_full = dev_bf16(torch, inp.w, dev)
    y_d = torch.from_numpy(inp.targets).to(dev)
    ids_d = torch.from_numpy(inp.ids).to(dev)
    ranges = [vp.vp_shard_range(V, T, t) for t in range(T)]
    w0 = w_full[ranges[0][0]:ranges[0][1]]
    n_valid = int((inp.targets != vp.DEFAULT_IGNORE_INDEX).sum())
    grad_scale = 1.0 / max(1, n_valid)

    # buffers and workspaces allocated once
    m = torch.empty((T, N), dtype=torch.float32, device=dev)
    s, zy = torch.empty_like(m), torch.empty_like(m)
    loss = torch.empty(N, dtype=torch.float32, device=dev)
    lse = torch.empty_like(loss)
    mean = torch.empty(1, dtype=torch.float32, device=dev)
    emb = torch.empty((N, H), dtype=torch.bfloat16, device=dev)
    dx = torch.empty((N, H), dtype=torch.float32, device=dev)
    dw = torch.empty((Vs, H), dtype=torch.float32, device=dev)
    ws_f = vp.alloc_workspace(vp.vp_lmhead_ce_fwd_workspace(N, H, 0, Vs), dev)
    ws_b = vp.alloc_workspace(vp.vp_lmhead_ce_bwd_workspace(N, H, 0, Vs), dev)

    # the other seven shards' statistics (untimed)
    for t in range(1, T):
        a, b = ranges[t]
        vp.vp_lmhead_ce_fwd(x_d, w_full[a:b], y_d, a, b, m[t], s[t], zy[t], workspace=ws_f)

    calls = ("embed", "fwd", "combine", "bwd")

    def step(marks=None, ce_marks=None):
        """One step.  With `marks`, an event is recorded on the launch stream before each
        call and after the last one (5 events: the per-call breakdown).  With `ce_marks`,
        one event before the CE sequence (fwd, combine, bwd) and one after it (2 events:
        the sequence's duration, with no marker between its calls)."""
        def mark(i):
            if marks is not None:
                marks[i].record(stream)
        mark(0)
        vp.vp_embed_fwd(ids_d, w0, 0, Vs, out=emb)
        mark(1)
        if ce_marks is not None:
            ce_marks[0].record(stream)
        vp.vp_lmhead_ce_fwd(x_d, w0, y_d, 0, Vs, m[0], s[0], zy[0], workspace=ws_f)
        mark(2)
        vp.vp_ce_combine(m, s, zy, y_d, loss=loss, lse=lse, loss_mean=mean)
        mark(3)
        vp.vp_lmhead_ce_bwd(x_d, w0, y_d, lse, 0, Vs, grad_scale, dx=dx, dw=dw, workspace=ws_b)
        if ce_marks is not None:
            ce_marks[1].record(stream)
        mark(4)

    # parity gate: no number is reported unless the loss matches the oracle
    step()
    torch.cuda.synchronize()
    gold_path = os.path.join(ROOT, "tests", "golden", "oracle_shard_8b.npz")
    parity = {"checked": False}
    if os.path.exists(gold_path):
        gold = np.load(gold_path)
        lerr = float(np.abs(loss.cpu().double().numpy() - gold["loss"]).max())
        parity = {"checked": True, "loss_max_abs_err": lerr, "bar": 2e-3,
                  "mean_abs_err": abs(float(mean.item()) - float(gold["mean"]))}
        if not lerr <= 2e-3:
            log(f"PARITY FAILED: loss max abs err {lerr}")
            print(json.dumps({"metric": METRIC, "value": None, "error": "parity failed",
                              "parity": parity}))
            sys.exit(1)
    log(f"parity: {parity}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K whole steps, bracketed by synchronisation.  Inside it, two HIP events
    # on the launch stream bracket each step's CE sequence (forward, combine, backward), so
    # the roofline's launch duration carries no marker between the sequence's own calls.
    ce_marks = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for k in range(args.steps):
        step(ce_marks=ce_marks[k])
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    ce_each = np.array([mk[0].elapsed_time(mk[1]) for mk in ce_marks])
    ce_ms = float(ce_each.mean())
    # per-call breakdown: the same K steps again with an event between every two calls
    # (each event adds a few microseconds between the calls; these numbers are the parts'
    # proportions, not the headline)
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        step(marks[k])
    torch.cuda.synchronize()
    avg = {c: float(np.mean([mk[i].elapsed_time(mk[i + 1]) for mk in marks]))
           for i, c in enumerate(calls)}
    per_step = np.array([mk[0].elapsed_time(mk[4]) for mk in marks])
    step_stats = {"median_ms": float(np.median(per_step)), "min_ms": float(per_step.min()),
                  "p90_ms": float(np.percentile(per_step, 90)), "steps": int(per_step.size),
                  "ce_sequence_median_ms": float(np.median(ce_each)),
                  "ce_sequence_min_ms": float(ce_each.min()),
                  "note": "median/min/p90: whole steps with per-call events; ce_sequence_*: "
                          "the timed region's CE sequences"}
    alg_flops = 6.0 * N * Vs * H
    achieved = alg_flops / (ce_ms * 1e-3) / 1e12
    exec_tflops = 8.0 * N * Vs * H / (ce_ms * 1e-3) / 1e12

    embed_bytes = N * H * 2 + len(np.unique(inp.ids[inp.ids < Vs])) * H * 2 + N * 8
    breakdown = {
        "embed_ms": avg["embed"], "fwd_ms": avg["fwd"], "combine_ms": avg["combine"],
        "bwd_ms": avg["bwd"],
        "fwd_gemm_tflops": 2.0 * N * Vs * H / (avg["fwd"] * 1e-3) / 1e12,
        "bwd_gemms_tflops_executed": 6.0 * N * Vs * H / (avg["bwd"] * 1e-3) / 1e12,
        "ce_executed_tflops": exec_tflops,
        "ce_executed_frac": exec_tflops / PEAK_BF16_TFLOPS,
        "embed_GBs": embed_bytes / (avg["embed"] * 1e-3) / 1e9,
        # combine: read the [T, N] triples and targets, write loss and lse, mean pass
        "combine_GBs": (12 * T * N + 8 * N + 8 * N + 12 * N) / (avg["combine"] * 1e-3) / 1e9,
    }

    extra = {}
    if not args.no_comparator:
        extra["materialised_logits_comparator"] = comparator_bench(
            torch, vp, dev, stream, args, x_d, w0, y_d, m, s, zy, loss, lse, mean, dx, dw,
            grad_scale, ce_ms, avg, ws_f, ws_b)
    if not args.no_embed_bench:
        extra["vocab_padding"] = padding_bench(torch, vp, dev, stream, args, x_d, w_full, y_d, m, s,
                                               zy, loss, lse, mean, dx, grad_scale, ce_ms)
    embed_inputs = {}
    if not args.no_embed_bench:
        extra["embedding_heavy_lookup"] = embed_bench(torch, vp, vp_inputs, dev, stream, args)
        extra["embedding_heavy_backward"] = embed_bwd_bench(torch, vp, vp_inputs, dev, stream, args,
                                                            keep=embed_inputs)
    if not args.no_other_workloads:
        extra["other_workloads"] = {}
        for name in ("small_lm", "large_vocab", "embedding_heavy"):
            extra["other_workloads"][name] = ce_workload_bench(torch, vp, vp_inputs, dev, stream,
                                                               args, name)
            torch.cuda.empty_cache()
    if not args.no_yardsticks:
        extra["yardsticks"] = yardsticks(torch, dev, stream, N, H, Vs)

    result = {
        "metric": METRIC,
        "value": N / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "shard_8b: N=8192 tokens, H=4096, V=128256, T=8, shard 0 = "
                               "[16032, 4096] bf16 (W~N(0,0.02), X~N(0,1)), Zipf(1.1) targets; "
                               "step = lookup + fwd + combine(T=8) + bwd of shard 0",
                   "global_batch": N, "hidden": H, "vocab": V, "shards": T,
                   "parallelism": "1 GPU (one vocab shard)"},
        "roofline": {"bound": "mfma", "kernel": "fused LM-head CE fwd+combine+bwd (vp_lmhead_ce_fwd + "
                     "vp_ce_combine + vp_lmhead_ce_bwd)", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": recorded_traffic(), "algorithmic_flops_per_launch": alg_flops,
                     "avg_launch_ms": ce_ms},
        "breakdown": breakdown,
        "step_stats": step_stats,
        "env": device_info(torch, dev),
        "parity": parity,
        **extra,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample ...")
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_sample)
        if "embedding_heavy_backward" in result:
            result["embedding_heavy_backward"]["cpu_baseline"] = cpu_baseline_embed_bwd(
                embed_inputs["ids"], embed_inputs["dout"])
    print(json.dumps(result))


def shape_sweep(torch, vp, dev, Vs=16032, T=8, steps=10, warmup=3):
    """Step time of shard 0's forward, the combine over T = 8 and shard 0's backward at the
    8B-class shard width (Vs = 16032) over token counts N and hidden sizes H
    (``vp_inputs.sweep_inputs``: X ~ N(0, 1), W ~ N(0, 0.02) in bf16, uniform targets; the
    other shards' statistics are fixed synthetic triples, m = 1, s = 1000, target logit 0:
    only their count matters to the combine's time).  Each shape is gated before it is
    timed on the oracle's expected values (``tests/golden/oracle_sweep.npz``, written by
    ``tests/golden/make_oracle_golden.py sweep``): every token's loss, and dX and dW on the
    rows ``vp_inputs.sweep_samples`` names."""
    import vp_inputs
    gold = np.load(os.path.join(ROOT, "tests", "golden", "oracle_sweep.npz"))
    for N, H in vp_inputs.SWEEP_SHAPES:
        x_bits, w_bits, y_h = vp_inputs.sweep_inputs(N, H, Vs, T)
        x, w = dev_bf16(torch, x_bits, dev), dev_bf16(torch, w_bits, dev)
        y = torch.from_numpy(y_h).to(dev)
        m = torch.full((T, N), 1.0, device=dev)
        s = torch.full((T, N), 1000.0, device=dev)
        zy = torch.zeros((T, N), device=dev)
        loss, lse = torch.empty(N, device=dev), torch.empty(N, device=dev)
        mean = torch.empty(1, device=dev)
        dx, dw = torch.empty((N, H), device=dev), torch.empty((Vs, H), device=dev)
        wf = vp.alloc_workspace(vp.vp_lmhead_ce_fwd_workspace(N, H, 0, Vs), dev)
        wb = vp.alloc_workspace(vp.vp_lmhead_ce_bwd_workspace(N, H, 0, Vs), dev)
        g = 1.0 / N

        def step():
            vp.vp_lmhead_ce_fwd(x, w, y, 0, Vs, m[0], s[0], zy[0], workspace=wf)
            vp.vp_ce_combine(m, s, zy, y, loss=loss, lse=lse, loss_mean=mean)
            vp.vp_lmhead_ce_bwd(x, w, y, lse, 0, Vs, g, dx=dx, dw=dw, workspace=wb)

        step()
        torch.cuda.synchronize()
        key = f"{N}x{H}"
        rows, cols = vp_inputs.sweep_samples(N, H, y_h, Vs)
        dx_ref, dw_ref = gold[f"{key}_dx"].astype(np.float64), gold[f"{key}_dw"].astype(np.float64)
        loss_err = float(np.abs(loss.cpu().double().numpy() - gold[f"{key}_loss"]).max())
        dx_got = dx[torch.from_numpy(rows).to(dev)].double().cpu().numpy()
        dw_got = dw[torch.from_numpy(cols).to(dev)].double().cpu().numpy()
        dx_err = float(np.abs(dx_got - dx_ref).max() / np.abs(dx_ref).max())
        dw_err = float(np.abs(dw_got - dw_ref).max() / np.abs(dw_ref).max())
        gate = {"loss_max_abs_err": loss_err, "dx_rows_rel_err": dx_err, "dw_rows_rel_err": dw_err}
        if not (loss_err <= 2e-3 and dx_err <= 1e-2 and dw_err <= 1e-2):
            print(json.dumps({"N": N, "H": H, "error": "oracle gate failed", **gate}))
            sys.exit(1)
        for _ in range(warmup):
            step()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(steps):
            step()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        print(json.dumps({"N": N, "H": H, "Vs": Vs, "ms": round(ms, 4),
                          "tokens_per_s": round(N / ms * 1e3), "oracle_gate": gate,
                          "frac": round(6.0 * N * Vs * H / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12), 4)}),
              flush=True)
        del x, w, dx, dw, wf, wb
        torch.cuda.empty_cache()


def yardsticks(torch, dev, stream, N, H, Vs, reps=10):
    """Measured ceilings on this machine, for context: the vendor GEMM (torch.matmul on
    hipBLASLt, bf16) at the three GEMM shapes of the step, and streaming copy / fill."""
    def timed(fn):
        for _ in range(3):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps
    g = torch.Generator(device=dev).manual_seed(0)
    x = torch.randn(N, H, device=dev, generator=g).to(torch.bfloat16)
    w = torch.randn(Vs, H, device=dev, generator=g).to(torch.bfloat16)
    dz = torch.randn(N, Vs, device=dev, generator=g).to(torch.bfloat16)
    dzt = dz.t().contiguous()
    out = {}
    fl = 2.0 * N * Vs * H
    for name, fn in (("matmul_fwd_XWt", lambda: torch.matmul(x, w.t())),
                     ("matmul_dX_dzW", lambda: torch.matmul(dz, w)),
                     ("matmul_dW_dztX", lambda: torch.matmul(dzt, x))):
        ms = timed(fn)
        out[name + "_tflops"] = fl / (ms * 1e-3) / 1e12
    del x, w, dz, dzt
    a = torch.empty(512 * 2**20, dtype=torch.int16, device=dev)   # 1 GiB
    b = torch.empty_like(a)
    ms = timed(lambda: b.copy_(a))
    out["copy_GBs"] = 2 * a.numel() * 2 / (ms * 1e-3) / 1e9
    ms = timed(lambda: a.fill_(1))
    out["fill_GBs"] = a.numel() * 2 / (ms * 1e-3) / 1e9
    return out


def ce_workload_bench(torch, vp, vp_inputs, dev, stream, args, name):
    """The fused CE sequence of shard 0 (forward, combine over the T shards, backward) at
    another workload: the small LM (N=4096, H=512, V=6400, T=2; launch-bound), the
    large-vocab shard (N=16384, H=8192, shard [19008, 8192], T=8, shards 1-7 given as
    synthetic statistics) or the embedding-heavy T=1 cross entropy (N=4096, H=4096,
    V=256000).  Gated on every token's loss against the oracle golden;
    the same algorithmic count (6 N Vs H) and peak as the headline roofline."""
    inp = vp_inputs.make_inputs(name)
    wl = inp.wl
    N, H, T, Vs = wl.N, wl.H, wl.T, wl.Vs
    x_d = dev_bf16(torch, inp.x, dev)
    w0 = dev_bf16(torch, inp.w_shard(0), dev)
    y = inp.targets
    y_d = torch.from_numpy(y).to(dev)
    m = torch.empty((T, N), dtype=torch.float32, device=dev)
    s, zy = torch.empty_like(m), torch.empty_like(m)
    if T > 1 and wl.synthetic_other_shards:   # the other shards' statistics, made up
        ms, ss, zs = vp_inputs.synthetic_triples(name, y)
        m[1:].copy_(torch.from_numpy(ms[1:]))
        s[1:].copy_(torch.from_numpy(ss[1:]))
        zy[1:].copy_(torch.from_numpy(zs[1:]))
    elif T > 1:   # computed from their weight rows, untimed (other GPUs' work)
        for t in range(1, T):
            wt = dev_bf16(torch, inp.w_shard(t), dev)
            vp.vp_lmhead_ce_fwd(x_d, wt, y_d, t * Vs, (t + 1) * Vs, m[t], s[t], zy[t])
    loss = torch.empty(N, dtype=torch.float32, device=dev)
    lse, mean = torch.empty_like(loss), torch.empty(1, dtype=torch.float32, device=dev)
    dx = torch.empty((N, H), dtype=torch.float32, device=dev)
    dw = torch.empty((Vs, H), dtype=torch.float32, device=dev)
    ws_f = vp.alloc_workspace(vp.vp_lmhead_ce_fwd_workspace(N, H, 0, Vs), dev)
    ws_b = vp.alloc_workspace(vp.vp_lmhead_ce_bwd_workspace(N, H, 0, Vs), dev)
    g = 1.0 / max(1, int((y != vp.DEFAULT_IGNORE_INDEX).sum()))

    def step(marks=None):
        if marks:
            marks[0].record(stream)
        vp.vp_lmhead_ce_fwd(x_d, w0, y_d, 0, Vs, m[0], s[0], zy[0], workspace=ws_f)
        vp.vp_ce_combine(m, s, zy, y_d, loss=loss, lse=lse, loss_mean=mean)
        vp.vp_lmhead_ce_bwd(x_d, w0, y_d, lse, 0, Vs, g, dx=dx, dw=dw, workspace=ws_b)
        if marks:
            marks[1].record(stream)

    step()
    torch.cuda.synchronize()
    gold = np.load(os.path.join(ROOT, "tests", "golden", f"oracle_{name}.npz"))
    lerr = float(np.abs(loss.cpu().double().numpy() - gold["loss"]).max())
    out = {"workload": f"{name}: N={N}, H={H}, V={wl.V}, T={T}, shard 0 = [{Vs}, {H}] bf16",
           "parity": {"loss_max_abs_err": lerr, "bar": 2e-3}}
    if not lerr <= 2e-3:
        out["error"] = "parity failed: no time reported"
        return out
    steps = max(1, min(args.steps, 10))
    for _ in range(min(args.warmup, 3)):
        step()
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        step(marks[k])
    torch.cuda.synchronize()
    t = np.array([mk[0].elapsed_time(mk[1]) for mk in marks])
    # the same step captured once in a HIP graph and replayed (no per-kernel launch cost)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    graph.replay()
    torch.cuda.synchronize()
    gt = []
    for _ in range(steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        graph.replay()
        b.record(stream)
        torch.cuda.synchronize()
        gt.append(a.elapsed_time(b))
    ms = float(np.median(t))
    tf = 6.0 * N * Vs * H / (ms * 1e-3) / 1e12
    out.update({"median_ms": ms, "min_ms": float(t.min()), "steps": steps,
                "graph_replay_median_ms": float(np.median(gt)),
                "tokens_per_s": N / (ms * 1e-3), "achieved_tflops": tf,
                "frac": tf / PEAK_BF16_TFLOPS, "executed_tflops": tf * 8.0 / 6.0})
    return out


def embed_bench(torch, vp, vp_inputs, dev, stream, args):
    """The embedding-heavy lookup: 65536 Zipf(1.0) ids on shard 0 ([64000, 4096] bf16) of
    V = 256000, T = 4; algorithmic HBM bytes = output + distinct on-shard rows + ids."""
    wl = vp_inputs.WORKLOADS["embedding_heavy"]
    inp = vp_inputs.make_inputs("embedding_heavy", with_weight=False)
    Vs_e = wl.embed_V // wl.embed_T
    w_bits = vp_inputs.make_weight_rows(wl, 0, Vs_e)
    w_d = dev_bf16(torch, w_bits, dev)
    ids_d = torch.from_numpy(inp.ids).to(dev)
    n, h = inp.ids.shape[0], wl.embed_H
    out = torch.empty((n, h), dtype=torch.bfloat16, device=dev)
    ids = inp.ids
    own = ids[(ids >= 0) & (ids < Vs_e)]
    distinct = len(np.unique(own))
    alg_bytes = n * h * 2 + distinct * h * 2 + n * 8
    # parity of this launch: bit-exact on a sample of rows
    vp.vp_embed_fwd(ids_d, w_d, 0, Vs_e, out=out)
    torch.cuda.synchronize()
    rows = np.random.default_rng(5).choice(n, 512, replace=False)
    got = out[torch.from_numpy(rows).to(dev)].view(torch.int16).cpu().numpy().view(np.uint16)
    want = np.zeros((rows.size, h), dtype=np.uint16)
    o = (ids[rows] >= 0) & (ids[rows] < Vs_e)
    want[o] = w_bits[ids[rows][o]]
    ok = bool(np.array_equal(got, want))
    flush = torch.ones(512 * 2**20 // 4, dtype=torch.float32, device=dev)
    times = []
    for i in range(args.warmup + args.steps):
        # evict L2 / MALL between repetitions with a read-only pass (a write pass would
        # leave dirty lines draining to HBM during the timed lookup)
        flush.sum()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        vp.vp_embed_fwd(ids_d, w_d, 0, Vs_e, out=out)
        b.record(stream)
        torch.cuda.synchronize()
        if i >= args.warmup:
            times.append(a.elapsed_time(b))
    ms = float(np.median(times))
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": gbs / PEAK_HBM_GBS, "traffic": recorded_lookup_traffic().get("lookup"),
            "median_ms": ms, "min_ms": float(np.min(times)),
            "algorithmic_bytes": alg_bytes, "distinct_on_shard_rows": distinct,
            "on_shard_ids": int(own.size), "bit_exact_sample": ok}


def comparator_bench(torch, vp, dev, stream, args, x_d, w0, y_d, m, s, zy, loss, lse, mean, dx, dw,
                     grad_scale, fused_ms, fused_avg, ws_f, ws_b):
    """The same CE sequence with shard 0's fp32 logits stored in HBM (the pages'
    tensor-parallel baseline) instead of fused: logits GEMM, statistics read back from them
    (in one read, or in the pages' order: maxima, all-reduce MAX, sums about the global
    maximum), combine, and the backward from the stored logits (no recompute).  Reports
    time and the device memory beyond the inputs and gradients, beside the fused path."""
    N, H = x_d.shape
    Vs = w0.shape[0]
    logits = torch.empty((N, vp.logits_ld(Vs)), dtype=torch.float32, device=dev)
    M = torch.empty(N, dtype=torch.float32, device=dev)

    def fwd(two_pass):
        vp.vp_lmhead_logits(x_d, w0, 0, Vs, logits=logits)
        vp.vp_logits_ce_stats(logits, y_d, 0, Vs, None, m[0], s[0], zy[0])
        if two_pass:
            vp.vp_ce_max(m, out=M)
            vp.vp_logits_ce_stats(logits, y_d, 0, Vs, M, m[0], s[0], zy[0])

    def step(two_pass, marks=None):
        if marks:
            marks[0].record(stream)
        fwd(two_pass)
        if marks:
            marks[1].record(stream)
        vp.vp_ce_combine(m, s, zy, y_d, loss=loss, lse=lse, loss_mean=mean)
        if marks:
            marks[2].record(stream)
        vp.vp_logits_ce_bwd(logits, x_d, w0, y_d, lse, 0, Vs, grad_scale, dx=dx, dw=dw,
                            workspace=ws_b)
        if marks:
            marks[3].record(stream)

    out = {}
    for two_pass in (False, True):
        for _ in range(args.warmup):
            step(two_pass)
        # the sequence's duration, bracketed by two events (as the fused path's), then the
        # parts with an event between every two calls
        whole = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for k in range(args.steps):
            whole[k][0].record(stream)
            step(two_pass)
            whole[k][1].record(stream)
        torch.cuda.synchronize()
        marks = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for k in range(args.steps):
            step(two_pass, marks[k])
        torch.cuda.synchronize()
        parts = [float(np.mean([mk[i].elapsed_time(mk[i + 1]) for mk in marks])) for i in range(3)]
        out["two_pass" if two_pass else "one_read"] = {
            "ms": float(np.mean([mk[0].elapsed_time(mk[1]) for mk in whole])),
            "fwd_ms": parts[0], "combine_ms": parts[1], "bwd_ms": parts[2]}
    flops = 6.0 * N * Vs * H   # same algorithmic count as the fused path's roofline
    for k in ("one_read", "two_pass"):
        tf = flops / (out[k]["ms"] * 1e-3) / 1e12
        out[k].update({"achieved_tflops": tf, "frac": tf / PEAK_BF16_TFLOPS})
    logits_bytes = logits.numel() * 4
    out.update({
        "fused_ms": fused_ms, "fused_fwd_ms": fused_avg["fwd"], "fused_bwd_ms": fused_avg["bwd"],
        "stored_logits_bytes": logits_bytes,
        "fused_fwd_workspace_bytes": ws_f.numel(),
        "bwd_workspace_bytes": ws_b.numel(),
        "extra_memory_vs_fused_bytes": logits_bytes - ws_f.numel(),
        "note": "the fused path never stores the [N, Vs] logits and recomputes them in the "
                "backward; the comparator stores them in fp32 and skips the recompute GEMM"})
    return out


def padding_bench(torch, vp, dev, stream, args, x_d, w_full, y_d, m, s, zy, loss, lse, mean, dx,
                  grad_scale, unpadded_ms):
    """The pages' padding tip at the 8B-class shard: V = 128256 padded for T = 8 to
    vp_padded_vocab(128256, 8, 128) = 129024, i.e. shard 0 = 16128 = 126 x 128 rows instead
    of 16032.  Times the same fwd + combine + bwd sequence at the padded size (rows of the
    same weight) beside the unpadded one: both shards are 63 vocabulary tiles of 256."""
    N, H = x_d.shape
    V_pad = vp.vp_padded_vocab(128256, 8, 128)
    vs = V_pad // 8
    w0 = w_full[:vs]
    dw = torch.empty((vs, H), dtype=torch.float32, device=dev)
    ws_f = vp.alloc_workspace(vp.vp_lmhead_ce_fwd_workspace(N, H, 0, vs), dev)
    ws_b = vp.alloc_workspace(vp.vp_lmhead_ce_bwd_workspace(N, H, 0, vs), dev)

    def step():
        vp.vp_lmhead_ce_fwd(x_d, w0, y_d, 0, vs, m[0], s[0], zy[0], workspace=ws_f)
        vp.vp_ce_combine(m, s, zy, y_d, loss=loss, lse=lse, loss_mean=mean)
        vp.vp_lmhead_ce_bwd(x_d, w0, y_d, lse, 0, vs, grad_scale, dx=dx, dw=dw, workspace=ws_b)

    for _ in range(args.warmup):
        step()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(args.steps):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    tf = 6.0 * N * vs * H / (ms * 1e-3) / 1e12
    return {"V": 128256, "V_pad": V_pad, "shard_rows": 16032, "padded_shard_rows": vs,
            "padded_achieved_tflops": tf, "padded_frac": tf / PEAK_BF16_TFLOPS,
            "unpadded_ms": unpadded_ms, "padded_ms": ms,
            "padded_over_unpadded": ms / unpadded_ms,
            "note": "same 63 vocabulary tiles either way: the kernels mask the shard's tail "
                    "rows in-tile, so padding buys no speed here"}


def embed_bwd_bench(torch, vp, vp_inputs, dev, stream, args, keep=None):
    """Weight gradient of the embedding-heavy lookup (65536 Zipf(1.0) ids, shard 0 =
    [64000, 4096] of V = 256000, T = 4), added into an fp32 gradient.  Algorithmic HBM
    bytes = ids + the owned tokens' bf16 gradient rows (read once) + every distinct owned
    row of the fp32 gradient (read and written once)."""
    wl = vp_inputs.WORKLOADS["embedding_heavy"]
    ids = vp_inputs.make_inputs("embedding_heavy", with_weight=False).ids
    Vs_e = wl.embed_V // wl.embed_T
    h = wl.embed_H
    dout = vp_inputs.make_embed_output_grad("embedding_heavy")
    if keep is not None:   # the CPU baseline reuses the same inputs
        keep.update(ids=ids, dout=dout)
    ids_d = torch.from_numpy(ids).to(dev)
    dout_d = dev_bf16(torch, dout, dev)
    dw = torch.zeros((Vs_e, h), dtype=torch.float32, device=dev)
    ws = vp.alloc_workspace(vp.vp_embed_bwd_workspace(ids.shape[0], h, 0, Vs_e), dev)
    own = (ids >= 0) & (ids < Vs_e)
    rows, counts = np.unique(ids[own], return_counts=True)
    alg_bytes = ids.shape[0] * 8 + int(own.sum()) * h * 2 + rows.size * h * 4 * 2
    # check of this launch: sampled rows against plain sums of their tokens' gradients,
    # and a second call on the same inputs giving the same bits
    vp.vp_embed_bwd(ids_d, dout_d, 0, Vs_e, dw=dw, workspace=ws)
    first = dw.clone()
    dw.zero_()
    vp.vp_embed_bwd(ids_d, dout_d, 0, Vs_e, dw=dw, workspace=ws)
    torch.cuda.synchronize()
    deterministic = bool(torch.equal(first, dw))
    pick = np.concatenate([rows[np.argsort(-counts)[:4]],
                           np.random.default_rng(9).choice(rows, 12, replace=False)])
    got = first[torch.from_numpy(pick).to(dev)].double().cpu().numpy()
    ref = np.stack([vp_inputs.bf16_bits_to_f64(dout[ids == r]).sum(axis=0) for r in pick])
    sample_err = float(np.abs(got - ref).max() / np.abs(ref).max())
    del first
    flush = torch.ones(512 * 2**20 // 4, dtype=torch.float32, device=dev)
    times = []
    for i in range(args.warmup + args.steps):
        flush.sum()          # evict L2 / MALL with a read-only pass
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        vp.vp_embed_bwd(ids_d, dout_d, 0, Vs_e, dw=dw, workspace=ws)
        b.record(stream)
        torch.cuda.synchronize()
        if i >= args.warmup:
            times.append(a.elapsed_time(b))
    ms = float(np.median(times))
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": gbs / PEAK_HBM_GBS, "traffic": recorded_lookup_traffic().get("gradient"),
            "median_ms": ms, "min_ms": float(np.min(times)),
            "algorithmic_bytes": alg_bytes, "owned_ids": int(own.sum()),
            "distinct_rows": int(rows.size), "most_repeated_row": int(counts.max()),
            "sample_max_rel_err": sample_err, "deterministic": deterministic}


def cpu_baseline_embed_bwd(ids, dout_bits, sample_ids: int = 65536):
    """The oracle's lookup gradient (np.add.at in fp64) on the first `sample_ids` ids of
    the embedding-heavy lookup, shard 0; reported in the same GB/s unit as the GPU."""
    import oracle
    import vp_inputs
    wl = vp_inputs.WORKLOADS["embedding_heavy"]
    ids = ids[:sample_ids]
    Vs_e = wl.embed_V // wl.embed_T
    dout = vp_inputs.bf16_bits_to_f64(dout_bits[:sample_ids])
    own = (ids >= 0) & (ids < Vs_e)
    alg_bytes = ids.size * 8 + int(own.sum()) * wl.embed_H * 2 + \
        np.unique(ids[own]).size * wl.embed_H * 4 * 2
    t0 = time.perf_counter()
    oracle.embed_shard_grad(ids, dout, 0, Vs_e)
    dt = time.perf_counter() - t0
    return {"value": alg_bytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"the first {sample_ids} of the 65536 ids (shard 0 of [256000, 4096]): "
                      f"np.add.at into an fp64 [64000, 4096] gradient, {dt:.2f} s"}


if __name__ == "__main__":
    main()
