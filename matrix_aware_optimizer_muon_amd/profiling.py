"""Summaries of rocprofv3 output for the Muon step kernels.

    python -m matrix_aware_optimizer_muon_amd.profiling trace DIR [--title T] [--command C ...]
        Markdown table of a `rocprofv3 --kernel-trace --stats --output-format csv`
        run (per-kernel calls, total and average duration, grid, LDS bytes).

    python -m matrix_aware_optimizer_muon_amd.profiling mfma DIR [--title T] [--command C ...]
        Markdown table of one `rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16
        SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE` pass: MFMA flops per
        dispatch, rate against the bf16 peak, MFMA busy share.

    python -m matrix_aware_optimizer_muon_amd.profiling traffic \
        --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR --copy-bytes N \
        [--out JSON] [--command C ...]
        HBM bytes per launch from two `rocprofv3 --pmc` passes (FETCH_SIZE, then
        WRITE_SIZE; KiB per dispatch), each scaled by what the same counter
        reads for device-to-device copies of a known size, as JSON.

Kernels are named by phase: gram (A = s X X^T), square (B = bA + cA^2),
bx (X <- s(aX + BX), weight update in the last iteration), momentum, update,
and the Newton-Muon kernels by their own names.
"""

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)


def kernel_source_hash():
    """Hash of the kernel sources (csrc/*.hip, *.h, *.cpp): counter figures
    are only valid for the sources they were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(PKG, "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def kernel_kind(name):
    # ns_gemm_kernel<f32, phase, tile shape, last iteration>
    m = re.search(r"ns_gemm_kernel<(\w+), (\d)[,>]", name) or re.search(r"ns_gemm_kernelILb(\d)ELi(\d)E", name)
    if m:
        f32 = m.group(1) in ("true", "1")
        return ["gram", "square", "bx"][int(m.group(2))] + ("/f32" if f32 else "")
    for k, v in (("momentum_kernel", "momentum"), ("(?<!syrk_)update_kernel", "update"), ("copyBuffer", "copy"),
                 ("fillBuffer", "fill")):
        if re.search(k, name):   # the Cholesky's syrk_update_kernel is not the update phase
            m2 = re.search(r"<(\w+)>", name) or re.search(r"ILb(\d)E", name)
            f32 = bool(m2) and m2.group(1) in ("true", "1")
            return v + ("/f32" if f32 and v in ("momentum", "update") else "")
    m = re.search(r"(\w+_kernel)", name)
    return m.group(1) if m else name[:40]


def _one(dirpath, pattern):
    hits = sorted(glob.glob(os.path.join(dirpath, "**", pattern), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no {pattern} under {dirpath}")
    return hits[0]


def _num(row, *keys, default=0.0):
    for k in keys:
        if k in row and row[k] not in ("", None):
            return float(row[k])
    return default


def _alone(spans):
    """For dispatches given as (start, end), whether each one overlapped no
    other dispatch in time (it had the GPU to itself)."""
    order = sorted(range(len(spans)), key=lambda i: spans[i][0])
    alone = [True] * len(spans)
    max_end = float("-inf")
    for pos, i in enumerate(order):
        s, e = spans[i]
        if max_end > s:
            alone[i] = False
        if pos + 1 < len(order) and spans[order[pos + 1]][0] < e:
            alone[i] = False
        max_end = max(max_end, e)
    return alone


def trace_table(dirpath):
    """Per-kernel rows from the kernel-trace CSV: calls, total/avg µs, grid
    workgroups, LDS bytes, and the average over the dispatches that ran alone
    (kernels of two streams overlap in time; a timing pass that keeps every
    launch on one stream gives dispatches that do not)."""
    path = _one(dirpath, "*kernel_trace.csv")
    recs = []
    with open(path) as f:
        for r in csv.DictReader(f):
            # workgroups over all grid dimensions (the Y and Z sizes are 1
            # when absent)
            wg = _num(r, "Workgroup_Size_X", "Workgroup_Size", default=1.0) or 1.0
            groups = int(_num(r, "Grid_Size_X", "Grid_Size", default=0.0) // wg)
            for d in ("Y", "Z"):
                wd = _num(r, f"Workgroup_Size_{d}", default=1.0) or 1.0
                groups *= max(1, int(_num(r, f"Grid_Size_{d}", default=1.0) // wd))
            recs.append((kernel_kind(r.get("Kernel_Name", "")), _num(r, "Start_Timestamp"),
                         _num(r, "End_Timestamp"), groups,
                         int(_num(r, "Group_Segment_Size", "LDS_Block_Size"))))
    alone = _alone([(a, b) for _, a, b, _, _ in recs])
    rows = {}
    for (kind, t0, t1, grid, lds), al in zip(recs, alone):
        dur = (t1 - t0) / 1e3
        e = rows.setdefault(kind, {"calls": 0, "total_us": 0.0, "grid": grid, "lds": lds,
                                   "alone_calls": 0, "alone_us": 0.0})
        e["calls"] += 1
        e["total_us"] += dur
        if al:
            e["alone_calls"] += 1
            e["alone_us"] += dur
    tot = sum(e["total_us"] for e in rows.values()) or 1.0
    for e in rows.values():
        e["avg_us"] = e["total_us"] / e["calls"]
        e["alone_avg_us"] = e["alone_us"] / e["alone_calls"] if e["alone_calls"] else float("nan")
        e["pct"] = 100.0 * e["total_us"] / tot
    return rows


def step_windows(dirpath):
    """Occupancy of each step in a kernel trace.  Every lane group's first
    launch of a step is its momentum launch, one per group, and the timed
    steps run the groups on queues of their own; so the number of queues the
    momentum launches use is the number per step, and a step starts at every
    such count of momentum launches and ends where the next starts (the last
    at its last dispatch).  Per step: its length, the time some kernel is
    running, the queues it used and, per queue, the idle time between
    consecutive dispatches on that queue (up to its first dispatch of the
    next step, where it has one)."""
    with open(_one(dirpath, "*kernel_trace.csv")) as f:
        ev = sorted((int(_num(r, "Start_Timestamp")), int(_num(r, "End_Timestamp")),
                     kernel_kind(r.get("Kernel_Name", "")), r.get("Queue_Id", "")) for r in csv.DictReader(f))
    mom = [e for e in ev if e[2].startswith("momentum")]
    per_step = max(1, len({e[3] for e in mom}))
    firsts = [e[0] for e in mom[::per_step]]
    out = []
    for k, a in enumerate(firsts):
        b = firsts[k + 1] if k + 1 < len(firsts) else None
        seg = [e for e in ev if e[0] >= a and (b is None or e[0] < b)]
        nxt = {e[3] for e in ev if b is not None and e[0] >= b and (k + 2 >= len(firsts) or e[0] < firsts[k + 2])}
        end = b if b is not None else max(e[1] for e in seg)
        busy, cs, ce = 0, seg[0][0], seg[0][1]
        for s0, e0, _, _ in seg[1:]:
            if s0 > ce:
                busy, cs, ce = busy + ce - cs, s0, e0
            else:
                ce = max(ce, e0)
        busy += min(ce, end) - cs
        gaps = {}
        for q in sorted({e[3] for e in seg}):
            qe = [(e[0], e[1]) for e in seg if e[3] == q]
            g = sum(max(0, qe[i + 1][0] - qe[i][1]) for i in range(len(qe) - 1))
            if q in nxt:   # idle until this queue's first launch of the next step
                g += max(0, end - max(e1 for _, e1 in qe))
            gaps[q] = g / 1e3
        out.append({"us": (end - a) / 1e3, "busy_us": busy / 1e3, "dispatches": len(seg), "queues": len(gaps),
                    "queue_gap_us": gaps})
    return out


def trace_markdown(dirpath, title, command):
    """`command`: one command line, or a list of them."""
    rows = trace_table(dirpath)
    lines = [command] if isinstance(command, str) else list(command)
    out = [f"# {title}", "", "Commands (repository root on one MI355X, `libmuon.so` built):", "", "```",
           *[c.strip() for c in lines], "```", "",
           "`alone`: dispatches that overlapped no other dispatch in time.", "",
           "| kernel | calls | total µs | avg µs | % | alone calls | alone avg µs | grid (workgroups) | LDS B |",
           "|---|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for k, e in sorted(rows.items(), key=lambda kv: -kv[1]["total_us"]):
        out.append(f"| {k} | {e['calls']} | {e['total_us']:.1f} | {e['avg_us']:.2f} | {e['pct']:.1f} | "
                   f"{e['alone_calls']} | {e['alone_avg_us']:.2f} | {e['grid']} | {e['lds']} |")
    steps = step_windows(dirpath)
    if 0 < len(steps) <= 40:   # a bench of a few whole steps (not a refresh-dominated run)
        out += ["", "Steps (from the first momentum launch of one step to that of the next, warm-up steps "
                "included): time some kernel is running, and idle time between consecutive dispatches of each "
                "queue. Steps on one queue are the timing pass's, one launch at a time.", "",
                "| step | µs | dispatches | queues | kernel running % | idle between dispatches per queue, µs |",
                "|---:|---:|---:|---:|---:|---|"]
        for i, st in enumerate(steps):
            gaps = ", ".join(f"{v:.1f}" for v in st["queue_gap_us"].values())
            out.append(f"| {i + 1} | {st['us']:.0f} | {st['dispatches']} | {st['queues']} | "
                       f"{100.0 * st['busy_us'] / st['us']:.1f} | {gaps} |")
    return "\n".join(out) + "\n"


def counter_per_dispatch(dirpath, counter):
    """Mean value of `counter` per dispatch, by kernel kind (values of the
    same dispatch are summed over the counter's instances)."""
    path = _one(dirpath, "*counter_collection.csv")
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") != counter:
                continue
            kind = kernel_kind(r.get("Kernel_Name", ""))
            d = per.setdefault(kind, {})
            key = r.get("Dispatch_Id") or r.get("Correlation_Id")
            d[key] = d.get(key, 0.0) + float(r["Counter_Value"])
    return {k: sum(v.values()) / len(v) for k, v in per.items()}


def _agent(dirpath):
    """SIMD count, XCD count and peak engine clock (MHz) of the GPU agent."""
    with open(_one(dirpath, "*agent_info.csv")) as f:
        for r in csv.DictReader(f):
            if int(_num(r, "Simd_Count")) > 0:
                return int(_num(r, "Simd_Count")), int(_num(r, "Num_Xcc", default=1.0)) or 1, \
                    _num(r, "Max_Engine_Clk_Fcompute")
    raise RuntimeError("no GPU agent in the run")


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")


def mfma_table(dirpath, peak_tflops):
    """Per kernel kind, from one `--pmc` pass of MFMA_COUNTERS (which also
    records each dispatch's start and end):
      gflop      MFMA flops per dispatch (the bf16 op counter counts units of
                 512 flops);
      avg_us     dispatch duration (dispatches run one at a time while
                 counters are collected);
      tflops     the two combined, and `frac` of `peak_tflops`;
      busy_pct   MFMA busy cycles as a share of the SIMD cycles of the
                 counter window (GRBM_GUI_ACTIVE arrives summed over the XCDs,
                 so one XCD's active cycles are the sum / Num_Xcc; the window
                 is somewhat longer than the dispatch, so this reads low)."""
    simds, xcc, _ = _agent(dirpath)
    disp = {}
    with open(_one(dirpath, "*counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            key = r.get("Dispatch_Id") or r.get("Correlation_Id")
            d = disp.setdefault(key, {"kind": kernel_kind(r.get("Kernel_Name", "")),
                                      "ns": _num(r, "End_Timestamp") - _num(r, "Start_Timestamp")})
            c = r.get("Counter_Name")
            d[c] = d.get(c, 0.0) + float(r["Counter_Value"])
    rows = {}
    for d in disp.values():
        e = rows.setdefault(d["kind"], {"dispatches": 0, "flop": 0.0, "ns": 0.0, "busy": 0.0, "gui": 0.0})
        e["dispatches"] += 1
        e["flop"] += 512.0 * d.get(MFMA_COUNTERS[0], 0.0)
        e["busy"] += d.get(MFMA_COUNTERS[1], 0.0)
        e["gui"] += d.get(MFMA_COUNTERS[2], 0.0) / xcc
        e["ns"] += d["ns"]
    out = {}
    for k, e in rows.items():
        if e["flop"] <= 0:
            continue
        n = e["dispatches"]
        tflops = e["flop"] / e["ns"] / 1e3 if e["ns"] > 0 else float("nan")
        out[k] = {"dispatches": n, "gflop": e["flop"] / n / 1e9, "avg_us": e["ns"] / n / 1e3,
                  "tflops": tflops, "frac": tflops / peak_tflops,
                  "busy_pct": 100.0 * e["busy"] / (e["gui"] * simds) if e["gui"] else float("nan")}
    return out


def mfma_markdown(dirpath, title, command, peak_tflops):
    rows = mfma_table(dirpath, peak_tflops)
    lines = [command] if isinstance(command, str) else list(command)
    out = [f"# {title}", "", "Commands (repository root on one MI355X, `libmuon.so` built):", "", "```",
           *[c.strip() for c in lines], "```", "",
           f"MFMA flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; peak {peak_tflops:.0f} TFLOP/s (dense bf16). "
           "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x SIMDs), over the counter window. "
           f"Kernel sources: {kernel_source_hash()}.", "",
           "| kernel | dispatches | MFMA GFLOP per dispatch | avg µs | MFMA TFLOP/s | % of peak | MFMA busy % |",
           "|---|---:|---:|---:|---:|---:|---:|"]
    for k, e in sorted(rows.items(), key=lambda kv: -kv[1]["gflop"] * kv[1]["dispatches"]):
        out.append(f"| {k} | {e['dispatches']} | {e['gflop']:.2f} | {e['avg_us']:.1f} | {e['tflops']:.0f} | "
                   f"{100 * e['frac']:.1f} | {e['busy_pct']:.1f} |")
    return "\n".join(out) + "\n"


def traffic(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_bytes, commands):
    fetch = counter_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = counter_per_dispatch(write_dir, "WRITE_SIZE")
    cf = counter_per_dispatch(copy_fetch_dir, "FETCH_SIZE").get("copy")
    cw = counter_per_dispatch(copy_write_dir, "WRITE_SIZE").get("copy")
    if not cf or not cw:
        raise RuntimeError("no copy kernel in the calibration runs")
    # a copy of N bytes reads N and writes N; KiB per dispatch -> bytes
    f_scale = copy_bytes / (cf * 1024.0)
    w_scale = copy_bytes / (cw * 1024.0)
    per = {}
    for k in sorted(set(fetch) | set(write)):
        if k in ("copy", "fill"):
            continue
        rd = fetch.get(k, 0.0) * 1024.0 * f_scale
        wr = write.get(k, 0.0) * 1024.0 * w_scale
        per[k] = int(round(rd + wr))
    return {
        "kernel_source_hash": kernel_source_hash(),
        "per_launch_bytes": per,
        "per_launch_read_bytes": {k: int(round(fetch.get(k, 0.0) * 1024.0 * f_scale)) for k in per},
        "per_launch_write_bytes": {k: int(round(write.get(k, 0.0) * 1024.0 * w_scale)) for k in per},
        "raw_kib_per_dispatch": {"FETCH_SIZE": fetch, "WRITE_SIZE": write},
        "calibration": {"copy_bytes": copy_bytes, "copy_FETCH_SIZE_kib": cf, "copy_WRITE_SIZE_kib": cw,
                        "fetch_scale": f_scale, "write_scale": w_scale},
        "commands": commands,
    }


LDS_COUNTERS = ["SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS", "SQ_INSTS_MFMA", "SQ_WAIT_INST_LDS",
                "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE"]


def lds_table(dirpath):
    """Per kernel kind, from one `--pmc` pass of LDS_COUNTERS:
      lds_busy_pct  cycles the CU's LDS serves indexed accesses, as a share
                    of the CU cycles of the counter window (the counter is
                    summed over every CU; GRBM_GUI_ACTIVE over the XCDs);
      conflict_pct  bank-conflict cycles as a share of those LDS cycles;
      lds_per_mfma  LDS instructions (the direct-to-LDS copies included) per
                    MFMA instruction;
      wait_lds_pct  wave time spent waiting to issue an LDS instruction, and
      wait_any_pct  waiting to issue any instruction, as shares of the wave
                    time (both counters and SQ_WAVE_CYCLES are in units of
                    four cycles)."""
    simds, xcc, _ = _agent(dirpath)
    cus = max(1, simds // 4)
    disp = {}
    with open(_one(dirpath, "*counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            key = r.get("Dispatch_Id") or r.get("Correlation_Id")
            d = disp.setdefault(key, {"kind": kernel_kind(r.get("Kernel_Name", "")),
                                      "ns": _num(r, "End_Timestamp") - _num(r, "Start_Timestamp")})
            c = r.get("Counter_Name")
            d[c] = d.get(c, 0.0) + float(r["Counter_Value"])
    rows = {}
    for d in disp.values():
        e = rows.setdefault(d["kind"], {"dispatches": 0, "ns": 0.0, **{c: 0.0 for c in LDS_COUNTERS}})
        e["dispatches"] += 1
        e["ns"] += d["ns"]
        for c in LDS_COUNTERS:
            e[c] += d.get(c, 0.0)
    out = {}
    for k, e in rows.items():
        gui = e["GRBM_GUI_ACTIVE"] / xcc
        idx, wave = e["SQ_LDS_IDX_ACTIVE"], e["SQ_WAVE_CYCLES"]
        out[k] = {"dispatches": e["dispatches"], "avg_us": e["ns"] / e["dispatches"] / 1e3,
                  "lds_busy_pct": 100.0 * idx / (gui * cus) if gui else float("nan"),
                  "conflict_pct": 100.0 * e["SQ_LDS_BANK_CONFLICT"] / idx if idx else float("nan"),
                  "lds_per_mfma": e["SQ_INSTS_LDS"] / e["SQ_INSTS_MFMA"] if e["SQ_INSTS_MFMA"] else float("nan"),
                  "wait_lds_pct": 100.0 * e["SQ_WAIT_INST_LDS"] / wave if wave else float("nan"),
                  "wait_any_pct": 100.0 * e["SQ_WAIT_INST_ANY"] / wave if wave else float("nan")}
    return out


def lds_markdown(dirpath, title, commands):
    rows = lds_table(dirpath)
    out = [f"# {title}", ""] + _command_block(commands) + [
        "LDS busy = SQ_LDS_IDX_ACTIVE / (GRBM_GUI_ACTIVE per XCD x CUs); conflicts = SQ_LDS_BANK_CONFLICT / "
        "SQ_LDS_IDX_ACTIVE; LDS per MFMA = SQ_INSTS_LDS / SQ_INSTS_MFMA (the direct-to-LDS copies count as LDS "
        "instructions); waits = SQ_WAIT_INST_LDS and SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES. Dispatches run one at a "
        f"time while counters are collected; the counter window is a little longer than a dispatch. Kernel "
        f"sources: {kernel_source_hash()}.", "",
        "| kernel | dispatches | avg µs | LDS busy % | bank conflicts % of LDS cycles | LDS instr. per MFMA | "
        "wave time waiting for LDS issue % | waiting for any issue % |",
        "|---|---:|---:|---:|---:|---:|---:|---:|"]
    for k, e in sorted(rows.items(), key=lambda kv: -kv[1]["avg_us"] * kv[1]["dispatches"]):
        if k in ("copy", "fill"):
            continue
        out.append(f"| {k} | {e['dispatches']} | {e['avg_us']:.1f} | {e['lds_busy_pct']:.1f} | "
                   f"{e['conflict_pct']:.1f} | {e['lds_per_mfma']:.2f} | {e['wait_lds_pct']:.1f} | "
                   f"{e['wait_any_pct']:.1f} |")
    return "\n".join(out) + "\n"


def _command_block(commands):
    return ["Commands (repository root on one MI355X, `libmuon.so` built):", "", "```", *commands, "```", ""]


def markers_markdown(trace_dir, title, commands):
    """Named host-side ranges (rocprofv3 --marker-trace): count and mean
    duration per range name, largest total first."""
    rows = {}
    with open(_one(trace_dir, "*marker_api_trace.csv")) as f:
        recs = list(csv.DictReader(f))
    for r in recs:
        e = rows.setdefault(r["Function"], [0, 0.0])
        e[0] += 1
        e[1] += (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    out = [f"# {title}", ""] + _command_block(commands) + [
        "The library pushes a named host-side range around each step and each launch (`Range` in "
        "`muon_host.cpp`). Durations are host time inside the enclosed enqueue calls. The host runs ahead of the "
        "GPU until the runtime's queue is full; from then on each enqueue waits for a slot, so these durations "
        "track the kernels' own (the kernel trace of the same run has those).", "",
        "| range | count | mean host µs |", "|---|---:|---:|"]
    for name, (n, us) in sorted(rows.items(), key=lambda kv: -kv[1][1]):
        out.append(f"| `{name}` | {n} | {us / n:.1f} |")
    return "\n".join(out) + "\n"


BLAS_LABELS = {
    "gpt2s": "GPT-2-small (72 units: 48 of 768x768, 24 of 768x3072)",
    "square": "one 4096x4096 unit",
    "gpt2xl": "GPT-2-XL (288 units: 192 of 1600x1600, 96 of 1600x6400)",
}


def blas_markdown(bench_lines, commands):
    """Vendor BLAS beside the library's Newton-Schulz phases, from bench.py
    --blas-context lines (workload name = file stem after "blas_")."""
    recs = []
    for path in bench_lines:
        with open(path) as f:
            line = [l for l in f.read().splitlines() if l.startswith("{")][-1]
        w = os.path.splitext(os.path.basename(path))[0].split("blas_", 1)[-1]
        recs.append((w, json.loads(line)))
    lib = recs[0][1]["blas_context"]["library"]
    out = ["# Vendor BLAS beside the library's Newton-Schulz phases (context, not part of the step)", "",
           "The same products as one Newton-Schulz iteration, timed with the vendor BLAS: one batched `torch.bmm` "
           "in bf16 per distinct unit shape (hipBLASLt underneath), for X X^T (full product), A A and B X of every "
           "bf16 unit, 20 repetitions after 3 warm-up calls, on the bench's stream. `library ms` is the library's "
           "time for the same phase, all lanes, one launch at a time (the bench's timing pass, averaged over the "
           "five iterations). The library's Gram and square compute only the tiles on and above the diagonal and "
           "store the rest mirrored; its B X also folds in a X, reads and writes the int8 master corrections and, "
           f"in the last iteration, applies the weight update. Library: {lib}.", ""] + _command_block(commands) + [
           f"Kernel sources: {kernel_source_hash()}.", "",
           "| workload | phase | vendor ms | vendor TFLOP/s | vendor % of bf16 peak | library ms | "
           "vendor / library time |", "|---|---|---:|---:|---:|---:|---:|"]
    for w, d in recs:
        for ph in ("gram", "square", "bx"):
            e = d["blas_context"][ph]
            out.append(f"| {BLAS_LABELS.get(w, w)} | {ph} | {e['vendor_ms']:.4f} | {e['vendor_tflops']:.0f} | "
                       f"{100 * e['vendor_frac_bf16_peak']:.1f} | {e['library_ms']:.4f} | "
                       f"{e['vendor_ms'] / e['library_ms']:.2f} |")
    out += ["", "Shader clock read during each run's timed steps (MHz): " +
            ", ".join(f"{w} {d.get('gpu_clock_mhz')}" for w, d in recs) + "."]
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(prog="python -m matrix_aware_optimizer_muon_amd.profiling")
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--title", default="Kernel trace")
    t.add_argument("--command", action="append", default=[])
    t.add_argument("--out")
    m = sub.add_parser("mfma")
    m.add_argument("dir")
    m.add_argument("--title", default="MFMA counters")
    m.add_argument("--command", action="append", default=[])
    m.add_argument("--peak-tflops", type=float, default=2500.0)
    m.add_argument("--out")
    c = sub.add_parser("traffic")
    for a in ("--fetch", "--write", "--copy-fetch", "--copy-write"):
        c.add_argument(a, required=True)
    c.add_argument("--copy-bytes", type=int, required=True)
    c.add_argument("--command", action="append", default=[])
    c.add_argument("--out")
    l = sub.add_parser("lds")
    l.add_argument("dir")
    l.add_argument("--title", default="LDS counters")
    l.add_argument("--command", action="append", default=[])
    l.add_argument("--out")
    k = sub.add_parser("markers")
    k.add_argument("dir")
    k.add_argument("--title", default="roctx ranges")
    k.add_argument("--command", action="append", default=[])
    k.add_argument("--out")
    b = sub.add_parser("blas")
    b.add_argument("lines", nargs="+", help="bench.py --blas-context outputs named blas_<workload>.json")
    b.add_argument("--command", action="append", default=[])
    b.add_argument("--out")
    args = ap.parse_args(argv)
    if args.cmd == "trace":
        text = trace_markdown(args.dir, args.title, args.command)
    elif args.cmd == "mfma":
        text = mfma_markdown(args.dir, args.title, args.command, args.peak_tflops)
    elif args.cmd == "lds":
        text = lds_markdown(args.dir, args.title, args.command)
    elif args.cmd == "markers":
        text = markers_markdown(args.dir, args.title, args.command)
    elif args.cmd == "blas":
        text = blas_markdown(args.lines, args.command)
    else:
        text = json.dumps(traffic(args.fetch, args.write, args.copy_fetch, args.copy_write, args.copy_bytes,
                                  args.command), indent=1) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    else:
        sys.stdout.write(text)


if __name__ == "__main__":
    main()
