"""Benchmark of the MI355X Muon step.

Workload: one grouped Muon step over the GPT-2-small hidden weight set
(12 layers x {Q, K, V, attn-out 768x768, MLP-up 3072x768, MLP-down
768x3072} = 72 bf16 matrices, Gaussian gradients with per-matrix scale, zero
initial momentum), mu 0.95 Nesterov, 5 quintic Newton-Schulz iterations,
lr 0.02, wd 0.01.  Inputs are generated once and stay resident in HBM.

Prints ONE JSON line: steps/s of the whole step, plus the roofline of the
dominant kernel (per-launch duration from HIP events recorded between the
launches on the launch stream) and the float64 CPU oracle timed on a bounded
sample of the same workload.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E

METRIC = "Muon steps/sec over a GPT-2-small weight set; NS TFLOP/s as % of bf16 MFMA peak"
STEP_TEXT = "one grouped Muon step (mu 0.95 Nesterov, 5 quintic NS, lr 0.02, wd 0.01)"
WORKLOAD_TEXT = {
    "gpt2s": "gpt2s: GPT-2-small hidden weights, 12 layers x {Q,K,V,O 768x768, MLP-up 3072x768, "
             "MLP-down 768x3072} = 72 bf16 matrices; " + STEP_TEXT,
    "square": "square: one 4096x4096 bf16 matrix, rank-32 + noise gradient; " + STEP_TEXT,
    "gpt2xl": "gpt2xl: GPT-2-XL hidden weights, 48 layers x {Q,K,V,O 1600x1600, MLP-up 6400x1600, "
              "MLP-down 1600x6400} = 288 bf16 matrices; " + STEP_TEXT,
    "gpt2s_aux": "gpt2s_aux: the gpt2s hidden matrices (Muon) plus every other GPT-2-small parameter with AdamW "
                 "(embeddings 50257x768 and 1024x768, 98 gain and bias vectors; 39.5M parameters, bf16); "
                 + STEP_TEXT + "; AdamW lr 3e-4, betas (0.9, 0.95), wd 0.01",
    "conv": "conv: 3x3 convolution filters of a CIFAR-10-style network as out x (in*9) matrices, 6 bf16 "
            "filters (64x288, 64x576, 256x576, 3 x 256x2304); " + STEP_TEXT,
    "tiny": "tiny: one 256x512 fp32 matrix; " + STEP_TEXT,
    "nmuon": "nmuon: one Newton-Muon layer at d=768 (QKV 2304x768 as three 768x768 blocks, O 768x768 and MLP-up "
             "3072x768 sharing one S^-1; MLP-down 768x3072 with four 768x768 S^-1 blocks; activations 16384x768 "
             "bf16 per S); preconditioned step: P = G S^-1 (fp32), then " + STEP_TEXT,
}


def ns_flops(m, n):
    """Algorithmic flops of the three NS products of one iteration, using the
    symmetry of A and B: Gram m(m+1)n, square m^2(m+1), update 2 m^2 n."""
    return {"gram": m * (m + 1) * n, "square": m * m * (m + 1), "bx": 2 * m * m * n}


def ns_bytes(m, n, es, w_es, ns_steps):
    """Algorithmic HBM bytes per launch of the three NS phases (averaged over
    the ns_steps iterations of a step) for an m x n unit whose NS buffers
    hold `es`-byte elements (bf16: the X master is bf16 hi + one int8
    correction, 3 bytes; float32: X is one float) and whose weight has
    `w_es`-byte elements.  Gram reads X (hi) and writes A; the square reads
    A and writes B; B X reads B, X (hi, the operand) and the master's
    correction, and writes the next X master -- except in the last
    iteration, which reads and writes the weight instead."""
    xm = es + 1 if es == 2 else es          # bytes of one X master element
    bx_in = es * m * m + es * m * n + (xm - es) * m * n
    bx = ((ns_steps - 1) * (bx_in + xm * m * n) + (bx_in + 2 * w_es * m * n)) / ns_steps
    return {"gram": es * m * n + es * m * m, "square": 2 * es * m * m, "bx": bx}


def load_traffic(kernel, src_hash, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (written by `python -m matrix_aware_optimizer_muon_amd.profiling
    traffic`), if it was taken on the current kernel sources and on this
    workload (the summary covers the GPT-2-small step)."""
    if workload != "gpt2s":
        return None
    p = os.path.join(ROOT, "profiles", "traffic_gpt2s.json")
    try:
        with open(p) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_hash") != src_hash:
        return None
    return d.get("per_launch_bytes", {}).get(kernel)


def cpu_baseline(wl, hp, budget_s):
    """The float64 oracle on whole layers of the same workload, cycling
    through the layers until the time budget is spent (at most three passes);
    steps/s scaled from the layers done."""
    import numpy as np
    from threadpoolctl import threadpool_info
    import synth
    from oracle import muon_oracle as orc
    layers = sorted({t.layer for t in wl.tensors})
    done, spent = 0, 0.0
    for layer in layers * 3:
        specs = [t for t in wl.tensors if t.layer == layer]
        inputs = [(orc.bf16_bits_to_f64(synth.weight(wl, s)), orc.bf16_bits_to_f64(synth.gradient(wl, s)),
                   synth.momentum0(wl, s)) for s in specs]
        t0 = time.perf_counter()
        for (W, G, M) in inputs:
            orc.muon_step(W, G, M, lr=float(hp.lr), weight_decay=float(hp.weight_decay),
                          momentum=float(hp.momentum), eps=float(hp.eps))
        spent += time.perf_counter() - t0
        done += 1
        if spent >= budget_s:
            break
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    threads = max([i.get("num_threads", 1) for i in blas] or [1])
    frac = done / len(layers)
    return {"value": frac / spent, "unit": "steps/s", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 oracle on {done} layer steps ({6 * done} matrix steps; one whole step is "
                      f"{len(layers)} layers, {len(wl.tensors)} matrices) in {spent:.1f} s, scaled to one "
                      f"whole step",
            "cpu_model": cpu_model(), "affinity_cores": len(os.sched_getaffinity(0)),
            "blas": [{"name": i.get("internal_api"), "version": i.get("version"), "threads": i.get("num_threads"),
                      "architecture": i.get("architecture")} for i in blas]}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def gpu_clock_mhz(run_steps, seconds=2.0):
    """Shader clock (MHz) as rocm-smi reports it while the step runs: a
    thread keeps stepping for about `seconds` while rocm-smi is read once.
    None if rocm-smi is unavailable or its output is not understood."""
    import re
    import subprocess
    import threading
    done = threading.Event()

    def busy():
        t0 = time.perf_counter()
        while not done.is_set() and time.perf_counter() - t0 < seconds + 5.0:
            run_steps()

    th = threading.Thread(target=busy, daemon=True)
    th.start()
    time.sleep(0.3)
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], stdout=subprocess.PIPE,
                           stderr=subprocess.DEVNULL, text=True, timeout=20)
        text = r.stdout
    except (OSError, subprocess.SubprocessError):
        text = ""
    finally:
        done.set()
        th.join()
    try:
        d = json.loads(text)
    except ValueError:
        return None
    for card in d.values():
        if not isinstance(card, dict):
            continue
        for k, v in card.items():
            if "sclk" in k.lower():
                m = re.search(r"(\d+)\s*mhz", str(v).lower())
                if m:
                    return int(m.group(1))
    return None


def blas_context(units, ns_ms, dev, reps=20):
    """The vendor BLAS (torch.bmm in bf16, hipBLASLt on this stack) timed on
    the same products as the Newton-Schulz phases, one batched call per
    shape: the full X X^T, A A and B X of every bf16 unit.  Context for the
    GEMM kernels' rates only; the step never calls it.  ns_ms: the library's
    milliseconds per iteration of each phase (all lanes, one launch at a
    time)."""
    import torch
    from collections import Counter
    shapes = Counter((m, n) for m, n, es, _ in units if es == 2)
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        for _ in range(3):
            fn()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        return e0.elapsed_time(e1) / reps

    ms = {"gram": 0.0, "square": 0.0, "bx": 0.0}
    fl = {"gram": 0.0, "square": 0.0, "bx": 0.0}
    for (m, n), b in sorted(shapes.items()):
        X = torch.randn(b, m, n, device=dev, generator=gen).to(torch.bfloat16)
        Xt = X.transpose(1, 2).contiguous()
        A = torch.randn(b, m, m, device=dev, generator=gen).to(torch.bfloat16)
        ms["gram"] += timed(lambda: torch.bmm(X, Xt))
        ms["square"] += timed(lambda: torch.bmm(A, A))
        ms["bx"] += timed(lambda: torch.bmm(A, X))
        fl["gram"] += 2.0 * b * m * m * n
        fl["square"] += 2.0 * b * m ** 3
        fl["bx"] += 2.0 * b * m * m * n
        del X, Xt, A
    out = {"library": f"torch.bmm bf16 (torch {torch.__version__})", "shapes": len(shapes)}
    for k in ms:
        out[k] = {"vendor_ms": round(ms[k], 4), "vendor_tflops": round(fl[k] / (ms[k] * 1e-3) / 1e12, 1),
                  "vendor_frac_bf16_peak": round(fl[k] / (ms[k] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                  "library_ms": round(ns_ms[k], 4)}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true", help="skip reading the shader clock (profiled runs)")
    ap.add_argument("--graph", action="store_true", help="time replays of the step captured in a HIP graph")
    ap.add_argument("--workload", default="gpt2s", choices=["gpt2s", "gpt2s_aux", "square", "gpt2xl", "conv", "tiny", "nmuon"],
                    help="weight set to step (the headline metric is quoted on gpt2s)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run 3 device-to-device copies of BYTES each (HBM counter calibration)")
    ap.add_argument("--blas-context", action="store_true",
                    help="also time the vendor BLAS on the same Newton-Schulz products (context)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the Muon step here runs on one GPU only (no collectives); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import matrix_aware_optimizer_muon_amd as mm
    from matrix_aware_optimizer_muon_amd.profiling import kernel_source_hash
    import synth

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    wl = synth.workload(args.workload)
    hp = mm.default_hparams()
    keep, descs = [], []
    for s in wl.tensors:
        G, W, M = synth.gradient(wl, s), synth.weight(wl, s), synth.momentum0(wl, s)
        if s.dtype == "bf16":
            tg = torch.from_numpy(G.view(np.int16).copy()).view(torch.bfloat16).to(dev)
            tw = torch.from_numpy(W.view(np.int16).copy()).view(torch.bfloat16).to(dev)
        else:
            tg, tw = torch.from_numpy(G).to(dev), torch.from_numpy(W).to(dev)
        tm = torch.from_numpy(M).to(dev)
        if s.kind == "adamw":               # embeddings, gains, biases: AdamW in the same step
            shape = s.shape or (s.rows, s.cols)
            tg, tw, tm = tg.view(shape), tw.view(shape), tm.view(shape)
            tv = torch.zeros_like(tm)
            keep += [tg, tw, tm, tv]
            descs.append(mm.adam_tensor_desc(tw, tg, tm, tv))
            continue
        keep += [tg, tw, tm]
        descs.append(mm.tensor_desc(tw, tg, tm, split_rows=s.split_rows, precond=s.precond))
    # Newton-Muon slots: one per preconditioner index, d = the activation width
    slots = sorted({s.precond for s in wl.tensors if s.precond >= 0})
    preconds = []
    for sl in slots:
        pc = mm.MuonPrecond()
        pc.d = wl.act_dim
        pc.nblocks = max(s.precond_blocks for s in wl.tensors if s.precond == sl)
        preconds.append(pc)
    st = mm.MuonStep(descs, hp, preconds=preconds, device=dev)
    stream = torch.cuda.current_stream(dev)
    acts = []          # (slot, block, activations) in the order the workload draws them
    for sl, pc in zip(slots, preconds):
        for blk in range(pc.nblocks):
            A = synth.activations(wl, len(acts))
            acts.append((sl, blk, torch.from_numpy(A.view(np.int16).copy()).view(torch.bfloat16).to(dev)))
    for sl, blk, a in acts:
        st.precond_refresh(sl, blk, a, damping=1e-4)

    for _ in range(args.warmup):
        st.step()
    torch.cuda.synchronize(dev)
    run_step = st.step
    if args.graph:
        # the whole step (both lanes' fork and join included) captured once
        # in a HIP graph and replayed: no host launch work between kernels
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream(dev)
        with torch.cuda.graph(graph, stream=cap):
            st.step()
        torch.cuda.synchronize(dev)
        run_step = graph.replay
        for _ in range(max(1, args.warmup)):
            run_step()
        torch.cuda.synchronize(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        run_step()
    ev1.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps

    # per-launch durations: HIP events recorded between launches on the
    # launch stream, over a second run of the same steps
    per = {}
    nprof = max(3, min(args.steps, 20))
    for _ in range(nprof):
        for name, ms in st.step_timed():
            kind = name.split("/")[0]
            per.setdefault(kind, []).append(ms)
    assert st.flags() == 0, "non-finite values in the benchmark step"
    precond_info = None
    if acts:
        # refresh (S = X^T X / N + damping I from one activation batch, then
        # its float64 Cholesky inverse) and one micro-batch accumulation,
        # each timed alone per block
        reps = 10
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            for sl, blk, a in acts:
                st.precond_refresh(sl, blk, a, damping=1e-4)
        e1.record(stream)
        torch.cuda.synchronize(dev)
        refresh_ms = e0.elapsed_time(e1) / (reps * len(acts))
        e0.record(stream)
        for _ in range(reps):
            for sl, blk, a in acts:
                st.precond_accumulate(sl, blk, a, beta=1.0)
        e1.record(stream)
        torch.cuda.synchronize(dev)
        acc_ms = e0.elapsed_time(e1) / (reps * len(acts))
        n, d = wl.act_rows, wl.act_dim
        syrk_flop = n * d * (d + 1)             # upper tiles of X^T X (symmetric)
        precond_info = {"blocks": len(acts), "act_rows": n, "d": d,
                        "refresh_ms_per_block": round(refresh_ms, 4),
                        "accumulate_ms_per_block": round(acc_ms, 4),
                        "accumulate_tflops": round(syrk_flop / (acc_ms * 1e-3) / 1e12, 2)}
        assert st.flags() == 0, "non-finite values in the preconditioner timing"
    def burst():
        for _ in range(10):
            st.step()
        torch.cuda.synchronize(dev)

    clock = None if args.no_clock else gpu_clock_mhz(burst)
    peak_mem = torch.cuda.max_memory_allocated(dev)
    ws_bytes = st.workspace_bytes
    st.close()

    units = []
    for s in wl.tensors:
        if s.kind != "muon":
            continue
        h = s.split_rows or s.rows
        m = min(h, s.cols)
        es = 4 if (s.dtype == "f32" or m < 128) else 2     # NS precision of the unit
        w_es = 4 if s.dtype == "f32" else 2
        units += [(m, max(h, s.cols), es, w_es)] * (s.rows // h)
    flops = {"gram": 0, "square": 0, "bx": 0}
    nbytes = {"gram": 0, "square": 0, "bx": 0}
    for m, n, es, w_es in units:
        for k, v in ns_flops(m, n).items():
            flops[k] += v
        for k, v in ns_bytes(m, n, es, w_es, max(1, hp.ns_steps)).items():
            nbytes[k] += v
    elems = sum(s.rows * s.cols for s in wl.tensors if s.kind == "muon")
    # P = G S^-1: per preconditioned tensor rows x (cols/d blocks) x d x d
    # multiply-adds of a float32 GEMM; G read (stored dtype), P written
    # (float32).  The kernel forms it from bf16 plane products: three per
    # float32 product for a bf16 G, six for a float32 G (apply_mfma_flops).
    flops["precond_apply"] = sum(2 * s.rows * s.cols * wl.act_dim for s in wl.tensors if s.precond >= 0)
    apply_mfma_flops = sum((6 if s.dtype == "f32" else 3) * 2 * s.rows * s.cols * wl.act_dim
                           for s in wl.tensors if s.precond >= 0)
    nbytes["precond_apply"] = sum(s.rows * s.cols * ((4 if s.dtype == "f32" else 2) + 4)
                                  for s in wl.tensors if s.precond >= 0)
    nbytes["momentum"] = 13 * elems          # G (bf16) + M read, M + X master (hi, int8) written
    nbytes["update"] = 8 * elems
    # AdamW: W read and written, G read, both float32 moments read and written
    nbytes["adamw"] = sum(s.rows * s.cols * (3 * (4 if s.dtype == "f32" else 2) + 16)
                          for s in wl.tensors if s.kind == "adamw")
    totals = {k: sum(v) / nprof for k, v in per.items()}          # ms per step by kernel kind
    avg = {k: sum(v) / len(v) for k, v in per.items()}             # ms per launch
    launches = {k: len(v) // nprof for k, v in per.items()}        # launches per step (two per phase with lanes)
    # algorithmic work per step of each kind (NS phases run ns_steps times)
    iters = {k: (hp.ns_steps if k in ("gram", "square", "bx") else 1) for k in per}
    ns_ms = sum(totals[k] for k in ("gram", "square", "bx"))
    ns_tflop = hp.ns_steps * sum(flops[k] for k in ("gram", "square", "bx")) / 1e12
    dom = max(totals, key=totals.get)
    src_hash = kernel_source_hash()
    # The Newton-Schulz products are dense contractions: their roofline is
    # the MFMA peak of their type, whatever their intensity; the element-wise
    # kernels are bound by HBM.  The apply is priced by the bf16 MFMA work it
    # issues.  Either way the HBM view is reported beside it.
    intensity = flops.get(dom, 0) / nbytes[dom]
    # per launch: the kind's work per step over its launches per step (with
    # two lanes each phase is two launches of about half the work)
    per_launch_flops = flops.get(dom, 0) * iters[dom] / launches[dom]
    per_launch_bytes = nbytes[dom] * iters[dom] / launches[dom]
    # the NS phases run on bf16 MFMA unless every unit takes the float32 path
    # (float32 matrices, or a short side under 128); the apply issues bf16
    # plane products
    ns_f32_only = bool(units) and all(es == 4 for _, _, es, _ in units)
    peak = PEAK_F32_TFLOPS if (ns_f32_only and dom in ("gram", "square", "bx")) else PEAK_BF16_TFLOPS
    if dom == "precond_apply":                 # priced by the bf16 MFMA work it issues
        intensity = apply_mfma_flops / nbytes[dom]
        per_launch_flops = apply_mfma_flops / launches[dom]
    hbm_gbs = per_launch_bytes / (avg[dom] * 1e-3) / 1e9
    if dom in flops:
        achieved = per_launch_flops / (avg[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(hbm_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(hbm_gbs / PEAK_HBM_GBS, 4)}
    roof["traffic"] = load_traffic(dom, src_hash, args.workload)
    roof["kernel"] = dom
    roof["avg_launch_ms"] = round(avg[dom], 5)
    roof["launches_per_step"] = launches[dom]
    roof["algorithmic_bytes"] = int(per_launch_bytes)
    if dom in flops:
        roof["algorithmic_flops"] = int(per_launch_flops)
        roof["intensity_flop_per_byte"] = round(intensity, 1)
        roof["hbm_view"] = {"achieved": round(hbm_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(hbm_gbs / PEAK_HBM_GBS, 4)}

    out = {
        "metric": METRIC,
        "value": round(1000.0 / ms_per_step, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.workload],
                   "matrices": sum(1 for s in wl.tensors if s.kind == "muon"), "params": elems,
                   "adamw_params": sum(s.rows * s.cols for s in wl.tensors if s.kind == "adamw"),
                   "parallelism": "single GPU", "launch": "graph" if args.graph else "eager"},
        "matrices_per_s": round(sum(1 for s in wl.tensors if s.kind == "muon") * 1000.0 / ms_per_step, 1),
        "ns_tflops": round(ns_tflop / (ns_ms * 1e-3), 2),
        "ns_frac_bf16_peak": round(ns_tflop / (ns_ms * 1e-3) / PEAK_BF16_TFLOPS, 4),
        "phase_ms_per_step": {k: round(v, 4) for k, v in totals.items()},
        "phase_avg_launch_ms": {k: round(v, 5) for k, v in avg.items()},
        "wall_s_timed": round(wall, 3),
        "kernel_source_hash": src_hash,
        "roofline": roof,
        "phase_hbm_gbs": {k: round(nbytes[k] * iters[k] / (totals[k] * 1e-3) / 1e9, 1) for k in avg if k in nbytes},
        "ns_kernel_frac_bf16_peak": {k: round(flops[k] * iters[k] / launches[k] / (avg[k] * 1e-3) / 1e12
                                              / PEAK_BF16_TFLOPS, 4)
                                     for k in ("gram", "square", "bx") if k in avg},
        "gpu_clock_mhz": clock,
        "peak_device_memory_gb": round(peak_mem / 1e9, 3),
        "workspace_gb": round(ws_bytes / 1e9, 3),
        "cpu_baseline": None,
    }
    if precond_info is not None:
        t_apply = totals["precond_apply"] * 1e-3
        precond_info["apply_tflops"] = round(flops["precond_apply"] / t_apply / 1e12, 2)          # float32 GEMM work
        precond_info["apply_mfma_tflops"] = round(apply_mfma_flops / t_apply / 1e12, 2)           # bf16 plane products
        out["precond"] = precond_info
    if args.workload != "gpt2s":
        out["metric"] = f"Muon steps/sec, {args.workload} weight set (not the headline workload)"
        out["dtype"] = "f32" if args.workload == "tiny" else "bf16"
    if args.blas_context and any(es == 2 for _, _, es, _ in units):
        out["blas_context"] = blas_context(units, {k: totals[k] / hp.ns_steps for k in ("gram", "square", "bx")}, dev)
    if not args.no_cpu_baseline and args.workload == "gpt2s":
        out["cpu_baseline"] = cpu_baseline(wl, hp, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
