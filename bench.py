#!/usr/bin/env python3
"""Throughput of the LongCat-Flash zero-computation-expert MoE layer on one MI355X.

One step = one lcmoe_forward call (router, biased top-K, permutation, grouped
SiLU-gated expert GEMMs, combine) on a resident batch of synthetic tokens at
the model's layer shape (d_model 6144, 512 FFN + 256 zero-computation
experts, K=12, expert intermediate 2048; "LongCat-Flash" llm-wiki entity
page, section 1 table). The headline value is the prefill batch (T=8192,
bf16); the decode batch (T=64, bf16), the fp8-weight batch (T=16384), the
same batch with fp8 activations as well, and a 32768-token bf16 batch are
measured in the same run and reported alongside.

Per-stage kernel durations come from HIP events recorded between the
library's launches on the same stream (lcmoe_forward_staged) inside the timed
region. The CPU oracle is timed on a bounded sample of the prefill workload.
Prints one JSON line.
"""
import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

METRIC = "MoE-layer tokens/sec at 1 GPU (decode & prefill); % HBM / MFMA roofline"
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "mixture_experts_layer_biased_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COPY_BYTES = 4 << 30      # the calibration copy of copy_bandwidth()
PEAK_HBM = 8.0e12          # B/s, MI355X HBM3E
PEAK_BF16 = 2.5e15         # FLOP/s, dense bf16 MFMA (fp8 weights run bf16 MFMA)
PEAK_FP8 = 5.0e15          # FLOP/s, dense fp8 MFMA (fp8 weights and fp8 activations)


def mfma_peak(cfg):
    """Peak of the contraction's own dtype."""
    return PEAK_FP8 if cfg.wdtype == "fp8a8" else PEAK_BF16


def _hip():
    lib = ctypes.CDLL("libamdhip64.so")
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return lib


GEMM_SOURCES = ("common.h", "kernels.h", "gemm.hip")


def source_hash():
    """Hash of the grouped-GEMM kernels' sources: the counter-derived traffic
    the bench line reports (the dominant grouped-GEMM kernel's) is used only
    while those kernels are unchanged since the counters were taken."""
    import hashlib
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as fh:
            h.update(name.encode() + fh.read())
    return h.hexdigest()[:16]


def stage_of_kernel(name):
    """Map a kernel symbol to its forward stage name."""
    if "gemm_big" in name:
        return "gateup" if "<true" in name else "down"
    if "quant_rows" in name:  # fp8 activations: x in the permute stage, H in the down stage
        return "quant (fp8 activations)"
    if "stats_partial" in name or "stats_final" in name:
        return "router statistics (outside the layer step)"
    for key, stage in (("router_gemm", "router"), ("topk", "topk"), ("combine", "combine"),
                       ("hist_kernel", "permute"), ("colscan", "permute"),
                       ("schedule_kernel", "permute"), ("scatter", "permute")):
        if key in name:
            return stage
    return None


BWD_OPS = {2: "w2t_dy", 3: "dx_rows", 4: "dw2", 5: "dw13", 6: "router_grads", 7: "router_grads"}


def bwd_stage_of_kernel(name):
    """Map a kernel symbol of a backward-only run to its backward stage."""
    if "gemm_big_dma_kernel<true, false, true>" in name:
        return "u_silu"
    for kname in ("bwd_dgrad_kernel<", "bwd_wgrad_stream_kernel<", "bwd_wgrad_f32_kernel<"):
        if kname in name:
            op = int(name.split(kname)[1].split(">")[0].split(",")[-1])
            return BWD_OPS.get(op)
    for key, stage in (("gather_rows", "route_gather"), ("router_gemm", "route_gather"),
                       ("topk", "route_gather"), ("hist_kernel", "route_gather"),
                       ("colscan", "route_gather"), ("schedule_kernel", "route_gather"),
                       ("scatter", "route_gather"), ("tile_prefix", "route_gather"),
                       ("bwd_dg_reduce", "dz"), ("bwd_zero_dg", "dz"),
                       ("bwd_router_dz", "dz"), ("router_w_split", "router_grads"),
                       ("bwd_dx", "dx")):
        if key in name:
            return stage
    return None


def measured_traffic(workload, stage):
    """HBM bytes per launch of `stage` from profiles/traffic.json, or None if
    absent or taken on different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != source_hash():
        return None
    e = t.get("workloads", {}).get(workload, {}).get(stage)
    return None if e is None else e["bytes"]


def pmc_summary(fetch_dir, write_dir, workload, cmd):
    """Fold two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per
    dispatch) into profiles/traffic.json. Each counter is scaled by what it
    reads for the 4 GiB device copy in the same run (true bytes / counted)."""
    import csv
    import collections

    def per_kernel(d, counter):
        rows = list(csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))))
        vals = collections.defaultdict(list)
        copy = []
        for r in rows:
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"]) * 1024.0
            if "copyBuffer" in r["Kernel_Name"]:
                copy.append(v)
            else:
                st = stage_of_kernel(r["Kernel_Name"])
                if st:
                    vals[(st, r["Kernel_Name"])].append(v)
        calib = max(copy) if copy else None
        return vals, calib

    fv, fcal = per_kernel(fetch_dir, "FETCH_SIZE")
    wv, wcal = per_kernel(write_dir, "WRITE_SIZE")
    fscale = COPY_BYTES / fcal if fcal else 1.0
    wscale = COPY_BYTES / wcal if wcal else 1.0
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        t = {}
    if t.get("source_hash") != source_hash():
        t = {"workloads": {}}
    t.update(source_hash=source_hash(), fetch_scale=fscale, write_scale=wscale,
             calibration=f"FETCH_SIZE/WRITE_SIZE of a {COPY_BYTES >> 30} GiB device copy "
                         f"read {COPY_BYTES / fscale / 2**30:.3f} / "
                         f"{COPY_BYTES / wscale / 2**30:.3f} GiB")
    wl = {}
    for (st, kname), v in fv.items():
        fb = float(np.mean(v)) * fscale
        wb = float(np.mean(wv.get((st, kname), [0.0]))) * wscale
        prev = wl.get(st)
        if prev is None or fb + wb > prev["bytes"]:
            wl[st] = dict(kernel=kname, fetch_bytes=fb, write_bytes=wb, bytes=fb + wb,
                          dispatches=len(v))
    t["workloads"][workload] = wl
    t.setdefault("commands", {})[workload] = cmd
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(t, f, indent=1, sort_keys=True)
    print(json.dumps({k: {"bytes": v["bytes"], "kernel": v["kernel"][:60]} for k, v in wl.items()},
                     indent=1))


def trace_summary(trace_dir, workload, cmd, out_path, work_path=None):
    """Write the rocprofv3 --kernel-trace --stats summary of the layer's
    kernels (calls, average / min / max duration) as a markdown table. With
    the work file the profiled bench run wrote (--work-out), also each
    grouped-GEMM stage's roofline fraction from the rocprof durations of the
    timed launches (the `steps` dispatches of its kernel before the
    `trailing` ones the run made after its timed loop), next to the bench's
    own event timing of the same launches."""
    import csv
    mapper = bwd_stage_of_kernel if workload.startswith("backward") else stage_of_kernel
    rows = list(csv.DictReader(open(os.path.join(trace_dir, "run_kernel_stats.csv"))))
    lines = [f"# rocprofv3 kernel statistics: {workload} workload", "",
             f"GEMM source hash (common.h, kernels.h, gemm.hip): `{source_hash()}`", "",
             "Command (from the repository root on the GPU host):", "", "```", cmd, "```", "",
             "| kernel | stage | calls | average us | min us | max us | share % |",
             "|---|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"]
        st = mapper(name)
        if st is None and "copyBuffer" not in name:
            continue
        short = name.split("(")[0].replace("void ", "")
        lines.append(f"| `{short}` | {st or 'device copies (input setup and the copy calibration; no entry point of the layer enqueues one)'} | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                     f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
    if work_path and os.path.exists(work_path):
        work = json.load(open(work_path))
        steps = int(work["steps"])
        trace = list(csv.DictReader(open(os.path.join(trace_dir, "run_kernel_trace.csv"))))
        trace.sort(key=lambda r: int(r["Start_Timestamp"]))
        durs = {}
        prev = None  # (stage, duration) of the dispatch before this one
        for r in trace:
            st = mapper(r["Kernel_Name"])
            dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            if st is not None:
                # with fp8 activations the down stage begins with the
                # quantization of H (the dispatch right before it)
                extra = prev[1] if st == "down" and prev and prev[0] == "quant (fp8 activations)" else 0
                durs.setdefault(st, []).append((int(r["Start_Timestamp"]), dur + extra))
            prev = (st, dur)
        lines += ["", f"Roofline of the grouped-GEMM stages over the {steps} timed launches "
                  "(algorithmic bytes: touched experts' weights once, plus the token rows once for "
                  "gate/up; spills are the gathered per-slot rows, H and Y; peaks 8 TB/s HBM, "
                  f"{mfma_peak_name(work['wdtype'])} MFMA):", "",
                  "| stage | rocprof mean ms | bench event mean ms | algorithmic GB | spill GB | "
                  "TFLOP | bound | achieved | frac (rocprof) | frac (bench) |",
                  "|---|---|---|---|---|---|---|---|---|---|"]
        for st, w in work["stage_work"].items():
            if st not in durs or w["flops"] == 0:
                continue
            seq = [x[1] for x in sorted(durs[st])]
            tail = int(work.get("trailing", 0))
            d = seq[max(0, len(seq) - tail - steps):len(seq) - tail]
            ms = float(np.mean(d)) / 1e6
            peak_m = PEAK_FP8 if work["wdtype"] == "fp8a8" else PEAK_BF16
            bound = "hbm" if w["flops"] / max(w["bytes"], 1) < peak_m / PEAK_HBM else "mfma"
            if bound == "hbm":
                ach, peak, unit = w["bytes"] / (ms / 1e3) / 1e9, PEAK_HBM / 1e9, "GB/s"
                fb = w["bytes"] / (w["ms"] / 1e3) / 1e9 / peak
            else:
                ach, peak, unit = w["flops"] / (ms / 1e3) / 1e12, peak_m / 1e12, "TFLOP/s"
                fb = w["flops"] / (w["ms"] / 1e3) / 1e12 / peak
            lines.append(f"| {st} | {ms:.3f} | {w['ms']:.3f} | {w['bytes'] / 1e9:.2f} | "
                         f"{w['spill_bytes'] / 1e9:.2f} | {w['flops'] / 1e12:.2f} | {bound} | "
                         f"{ach:.0f} {unit} | {ach / peak:.3f} | {fb:.3f} |")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def mfma_peak_name(wdtype):
    return "5.0 PFLOP/s fp8" if wdtype == "fp8a8" else "2.5 PFLOP/s bf16"


def counter_summary(dirs, workload, cmd, out_path, regex="gemm_big"):
    """Fold rocprofv3 --pmc runs (one counter set per directory) into a
    markdown table per kernel (mean per launch) with derived figures: the
    average clock over the launch, the MFMA pipes' busy share of all SIMD
    cycles, the share of wave cycles spent waiting and issuing VALU work, and
    the texture-data unit's busy and L2-stall shares. Stamped with the GEMM
    source hash."""
    import collections
    import csv
    vals = collections.defaultdict(list)
    kern_ms = {}
    for d in dirs:
        for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
            k = r["Kernel_Name"].split("(")[0].replace("void ", "")
            vals[(k, r["Counter_Name"])].append(float(r["Counter_Value"]))
            kern_ms.setdefault(k, []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6)
    kernels = sorted({k for k, _ in vals})
    counters = sorted({c for _, c in vals})
    m = {(k, c): float(np.mean(v)) for (k, c), v in vals.items()}
    lines = [f"# rocprofv3 counters: {workload} workload", "",
             f"GEMM source hash (common.h, kernels.h, gemm.hip): `{source_hash()}`", "",
             "Commands (from the repository root on the GPU host; one counter set per run):", "",
             "```"] + cmd.split(" ;; ") + ["```", "", "Mean per launch:", "",
             "| counter | " + " | ".join(f"`{k}`" for k in kernels) + " |",
             "|---|" + "---|" * len(kernels)]
    for c in counters:
        lines.append(f"| {c} | " + " | ".join(f"{m.get((k, c), float('nan')):.4g}" for k in kernels)
                     + " |")
    lines += ["", "Derived (GRBM_GUI_ACTIVE is the sum over the 8 XCDs, SQ_VALU_MFMA_BUSY_CYCLES over "
              "the 1024 SIMDs, TA/TD sums over the 256 CUs; wave-cycle shares are of SQ_WAVE_CYCLES):", ""]
    for k in kernels:
        g = m.get((k, "GRBM_GUI_ACTIVE"))
        if not g:
            continue
        cyc = g / 8
        ms = float(np.median(kern_ms[k]))
        parts = [f"clock {cyc / (ms / 1e3) / 1e9:.2f} GHz over {ms:.2f} ms"]
        if (k, "SQ_VALU_MFMA_BUSY_CYCLES") in m:
            parts.append(f"MFMA pipes busy {100 * m[(k, 'SQ_VALU_MFMA_BUSY_CYCLES')] / 1024 / cyc:.1f}% "
                         "of SIMD cycles")
        wc = m.get((k, "SQ_WAVE_CYCLES"))
        if wc:
            for c, what in (("SQ_WAIT_ANY", "waiting"), ("SQ_ACTIVE_INST_VALU", "issuing VALU"),
                            ("SQ_ACTIVE_INST_LDS", "issuing LDS")):
                if (k, c) in m:
                    parts.append(f"{what} {100 * m[(k, c)] / wc:.1f}% of wave cycles")
        if (k, "SQ_INSTS_MFMA") in m and (k, "SQ_INSTS_VALU") in m:
            mf = m[(k, "SQ_INSTS_MFMA")]
            parts.append(f"{(m[(k, 'SQ_INSTS_VALU')] - mf) / mf:.2f} other VALU instructions per MFMA")
            if (k, "SQ_INSTS_VALU_CVT") in m:
                parts.append(f"{m[(k, 'SQ_INSTS_VALU_CVT')] / mf:.2f} conversions per MFMA")
        for c, what in (("TA_TA_BUSY_sum", "TA busy"), ("TD_TD_BUSY_sum", "TD busy"),
                        ("TD_TC_STALL_sum", "TD stalled on L2 data")):
            if (k, c) in m:
                parts.append(f"{what} {100 * m[(k, c)] / 256 / cyc:.1f}% of CU cycles")
        lines.append(f"- `{k}`: " + "; ".join(parts) + ".")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def make_event_sets(hip, n_sets, n_events):
    sets = []
    for _ in range(n_sets):
        arr = (ctypes.c_void_p * n_events)()
        for i in range(n_events):
            ev = ctypes.c_void_p()
            assert hip.hipEventCreate(ctypes.byref(ev)) == 0
            arr[i] = ev
        sets.append(arr)
    return sets


def step_ms(hip, sets, n_stages):
    """Per-step duration (first to last stage event) of every timed step."""
    out = []
    for arr in sets:
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), arr[0], arr[n_stages]) == 0
        out.append(ms.value)
    return np.array(out)


def stage_ms(hip, sets, n_stages):
    out = np.zeros((len(sets), n_stages))
    for s, arr in enumerate(sets):
        for i in range(n_stages):
            ms = ctypes.c_float()
            assert hip.hipEventElapsedTime(ctypes.byref(ms), arr[i], arr[i + 1]) == 0
            out[s, i] = ms.value
    return out.mean(axis=0)


def kernel_work(cfg, counts, idx=None):
    """Algorithmic bytes and MFMA flops of each grouped-GEMM stage.

    What the method must move: each touched expert's weights read once (bf16
    2 B, fp8 1 B plus the 128x128 block scales), and for gate/up the token
    rows that feed it read once (the distinct tokens with an FFN slot;
    every token when idx is not given). The gathered per-slot copies of
    those rows, H and Y are the implementation's intermediates: reported as
    spill_bytes, not counted. Flops 2 * rows * (weights per expert).
    """
    N, d, I = cfg.n_ffn, cfg.d, cfg.inter
    c = counts[:N].astype(np.int64)
    sw = 1 if cfg.wdtype in ("fp8", "fp8a8") else 2
    sc = (4 / (128 * 128)) if cfg.wdtype in ("fp8", "fp8a8") else 0.0
    sel = c > 0
    et, rows = int(sel.sum()), int(c.sum())
    if idx is None:
        toks = cfg.tokens if rows else 0
    else:
        toks = int((idx < N).any(axis=1).sum())
    return {
        "gateup": dict(bytes=et * 2 * I * d * (sw + sc) + toks * d * 2,
                       spill_bytes=max(rows - toks, 0) * d * 2 + rows * I * 2,
                       flops=2.0 * rows * 2 * I * d, experts=et, rows=rows),
        "down": dict(bytes=et * d * I * (sw + sc),
                     spill_bytes=rows * I * 2 + rows * d * 2,
                     flops=2.0 * rows * I * d, experts=et, rows=rows),
    }


def layer_bytes(cfg, counts, T):
    """Whole-layer algorithmic bytes: touched experts' weights once, the router
    weights once, x read once and y written once."""
    N, d, I, E = cfg.n_ffn, cfg.d, cfg.inter, cfg.n_experts
    sw = 1 if cfg.wdtype in ("fp8", "fp8a8") else 2
    et = int((counts[:N] > 0).sum())
    return et * 3 * I * d * sw + E * d * 4 + 2 * T * d * 2


def measure(cfg, steps, warmup, hip):
    import torch
    from mixture_experts_layer_biased_amd import inputs, lcmoe

    L = inputs.make_layer(cfg, "cuda")
    x = inputs.make_tokens(cfg, "cuda")
    shape = lcmoe.shape_of(cfg)
    T = cfg.tokens
    ws = lcmoe.workspace(shape, T)
    out = dict(y=torch.empty(T, cfg.d, dtype=torch.bfloat16, device="cuda"),
               idx=torch.empty(T, cfg.k, dtype=torch.int32, device="cuda"),
               gate=torch.empty(T, cfg.k, dtype=torch.float32, device="cuda"),
               counts=torch.empty(cfg.n_experts, dtype=torch.int32, device="cuda"))
    nst = lcmoe.NUM_STAGES
    sets = make_event_sets(hip, steps, nst + 1)

    def step(ev=None):
        lcmoe.forward(shape, x, L["w_router"], L["bias"], L["w13"], L["w2"], L["w13_scale"],
                      L["w2_scale"], ws=ws, out=out, stage_events=ev)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record()
    for s in range(steps):
        step(sets[s])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    per_stage = stage_ms(hip, sets, nst)
    per_step = step_ms(hip, sets, nst)
    for arr in sets:
        for i in range(nst + 1):
            hip.hipEventDestroy(arr[i])
    counts = out["counts"].cpu().numpy()
    ms = total_ms / steps
    work = kernel_work(cfg, counts, out["idx"].cpu().numpy())
    stages = {name: float(per_stage[i]) for i, name in enumerate(lcmoe.STAGES)}
    gemm = [k for k in work if work[k]["rows"] > 0]
    dom = max(gemm, key=lambda k: stages[k])
    wk = work[dom]
    dom_s = stages[dom] / 1e3
    peak_mfma = mfma_peak(cfg)
    bound = "hbm" if wk["flops"] / wk["bytes"] < peak_mfma / PEAK_HBM else "mfma"
    if bound == "hbm":
        ach, peak, unit = wk["bytes"] / dom_s / 1e9, PEAK_HBM / 1e9, "GB/s"
    else:
        ach, peak, unit = wk["flops"] / dom_s / 1e12, peak_mfma / 1e12, "TFLOP/s"
    gemm_s = sum(stages[k] for k in work) / 1e3
    gemm_flops = sum(w["flops"] for w in work.values())
    gemm_bytes = sum(w["bytes"] for w in work.values())
    lb = layer_bytes(cfg, counts, T)
    res = dict(
        tokens=T, ms_per_step=ms, tokens_per_s=T / (ms / 1e3), wall_s=wall,
        step_ms_median=float(np.median(per_step)), step_ms_min=float(per_step.min()),
        mean_ffn_experts_per_token=float(counts[: cfg.n_ffn].sum() / T),
        touched_experts=int((counts[: cfg.n_ffn] > 0).sum()),
        max_rows_per_expert=int(counts[: cfg.n_ffn].max()),
        stages_ms=stages,
        dominant_kernel=dom,
        roofline=dict(bound=bound, achieved=ach, peak=peak, unit=unit, frac=ach / peak,
                      traffic=measured_traffic(cfg.name, dom), algorithmic_bytes=wk["bytes"],
                      spill_bytes=wk["spill_bytes"], flops=wk["flops"], kernel_ms=stages[dom]),
        stage_work={k: dict(bytes=v["bytes"], spill_bytes=v["spill_bytes"], flops=v["flops"],
                            ms=stages[k]) for k, v in work.items()},
        grouped_gemm=dict(ms=gemm_s * 1e3, mfma_frac=gemm_flops / gemm_s / peak_mfma,
                          hbm_frac=gemm_bytes / gemm_s / PEAK_HBM),
        layer=dict(algorithmic_bytes=lb, hbm_frac=lb / (ms / 1e3) / PEAK_HBM,
                   mfma_frac=gemm_flops / (ms / 1e3) / peak_mfma),
    )
    # Router-side statistics (outside the layer step): one routing call that
    # exports the logits, then lcmoe_router_stats timed on its own.
    r = lcmoe.route(shape, x, L["w_router"], L["bias"], ws=ws, logits=True)
    D = 8 if cfg.n_ffn % 8 == 0 else 1
    k_e = cfg.k * cfg.n_ffn / cfg.n_experts
    sws = torch.empty(lcmoe.router_stats_workspace_bytes(shape, D), dtype=torch.uint8,
                      device="cuda")
    lcmoe.router_stats(shape, x, r["logits"], r["counts"], D, k_e, ws=sws)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    reps = 5
    a.record()
    for _ in range(reps):
        lcmoe.router_stats(shape, x, r["logits"], r["counts"], D, k_e, ws=sws)
    b.record()
    torch.cuda.synchronize()
    st_ms = a.elapsed_time(b) / reps
    st_bytes = T * cfg.n_experts * 4 + T * cfg.d * 2
    res["router_stats"] = dict(ms=st_ms, groups=D, algorithmic_bytes=st_bytes,
                               hbm_frac=st_bytes / (st_ms / 1e3) / PEAK_HBM)
    del r, sws
    if "bias_steps" in cfg.extra:
        res["bias_loop"] = bias_loop(cfg, L, shape, ws, out)
    return res, (L, x, out)


def bias_loop(cfg, L, shape, ws, out):
    """The bias-controller loop of a configuration that names one (the fp8
    LongCat-shape batch: 20 steps, mu = 1e-3, K_e = 8): from the layer's
    bias, each step runs lcmoe_forward on a fresh seeded batch (generator
    stream 100 + j) and then lcmoe_bias_update with that call's counts.
    Reports each step's mean FFN experts per token, the largest relative
    deviation from K_e (the pages' convergence criterion is 1%), and the time
    of the forward plus update (batch generation outside the timed pair)."""
    import torch
    from mixture_experts_layer_biased_amd import inputs, lcmoe

    mu, k_e, n = cfg.extra["mu"], cfg.extra["k_e"], cfg.extra["bias_steps"]
    T = cfg.tokens
    bias = L["bias"].clone()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    means, ms = [], []
    for j in range(n):
        xj = inputs.make_tokens(cfg, "cuda", stream=100 + j)
        torch.cuda.synchronize()
        a.record()
        lcmoe.forward(shape, xj, L["w_router"], bias, L["w13"], L["w2"], L["w13_scale"],
                      L["w2_scale"], ws=ws, out=out)
        lcmoe.bias_update(shape, out["counts"], mu, k_e, bias, T)
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
        means.append(float(out["counts"][: cfg.n_ffn].sum().item()) / T)
        del xj
    dev = float(np.max(np.abs(np.array(means) - k_e)) / k_e)
    return dict(steps=n, mu=mu, k_e=k_e, mean_ffn_experts_per_token=means,
                max_rel_deviation=dev, within_1pct=dev < 0.01,
                step_ms_median=float(np.median(ms)),
                bias_ffn_absmax=float(bias[: cfg.n_ffn].abs().max().item()))


def measure_small(steps, warmup):
    """The small bf16 layer (d=1024, 64 FFN + 32 zero experts, K=6, I=512,
    T=4096): its 201 MB of expert weights fit in the 256 MB MALL, so each
    call is timed warm (weights may stay in the MALL between calls) and cold
    (a 1 GiB scratch buffer written between calls, outside the timed region),
    and warm once more as a replayed HIP graph of the same call (this layer is
    small enough for the launch gaps between its kernels to show). Median per
    call, tokens/s, and the fraction of the HBM roof from the layer's
    algorithmic bytes."""
    import torch
    from mixture_experts_layer_biased_amd import inputs, lcmoe

    cfg = inputs.CONFIGS["small"]
    L = inputs.make_layer(cfg, "cuda")
    x = inputs.make_tokens(cfg, "cuda")
    shape = lcmoe.shape_of(cfg)
    T = cfg.tokens
    ws = lcmoe.workspace(shape, T)
    out = dict(y=torch.empty(T, cfg.d, dtype=torch.bfloat16, device="cuda"),
               idx=torch.empty(T, cfg.k, dtype=torch.int32, device="cuda"),
               gate=torch.empty(T, cfg.k, dtype=torch.float32, device="cuda"),
               counts=torch.empty(cfg.n_experts, dtype=torch.int32, device="cuda"))
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")

    def call():
        lcmoe.forward(shape, x, L["w_router"], L["bias"], L["w13"], L["w2"], ws=ws, out=out)

    # The same call captured once into a HIP graph (the forward enqueues
    # kernels only), replayed warm: the launch gaps between its kernels go.
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    res = {}
    for mode in ("warm", "cold", "graph"):
        for _ in range(warmup):
            graph.replay() if mode == "graph" else call()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for i, (a, b) in enumerate(evs):
            if mode == "cold":
                scratch.fill_(i & 255)
            a.record()
            if mode == "graph":
                graph.replay()
            else:
                call()
            b.record()
        torch.cuda.synchronize()
        ms = np.array([a.elapsed_time(b) for a, b in evs])
        res[mode] = dict(ms_median=float(np.median(ms)), ms_min=float(ms.min()),
                         tokens_per_s=T / (float(np.median(ms)) / 1e3))
    counts = out["counts"].cpu().numpy()
    lb = layer_bytes(cfg, counts, T)
    for mode in res:
        res[mode]["hbm_frac"] = lb / (res[mode]["ms_median"] / 1e3) / PEAK_HBM
    res.update(tokens=T, algorithmic_bytes=lb,
               touched_experts=int((counts[: cfg.n_ffn] > 0).sum()),
               config=(f"T={T}, d_model={cfg.d}, {cfg.n_ffn} FFN + {cfg.n_zero} zero experts, "
                       f"K={cfg.k}, I={cfg.inter}, bf16, router bias ~ N(0, {cfg.bias_std})"))
    del L, x, ws, out, scratch, graph
    torch.cuda.empty_cache()
    return res


def backward_work(cfg, counts, T):
    """Algorithmic bytes and flops of each backward stage (bf16 operands,
    fp32 slot-row intermediates): per FFN slot the operand rows are read once
    and the results written once, each touched expert's weights are read
    once per GEMM that uses them, and every expert's weight gradient is
    written (zeros for an untouched expert)."""
    N, d, I, E = cfg.n_ffn, cfg.d, cfg.inter, cfg.n_experts
    c = counts[:N].astype(np.int64)
    S, et = int(c.sum()), int((c > 0).sum())
    w13, w2 = 2 * I * d * 2, d * I * 2
    return {
        "route_gather": dict(bytes=T * d * 2 + E * d * 4 + T * E * 4 + 2 * S * d * 2 * 2, flops=0.0),
        "w2t_dy": dict(bytes=et * w2 + S * (d * 2 + I * 4), flops=2.0 * S * I * d),
        # u = W13 x with the SiLU backward fused: reads Q, writes dU and g h
        "u_silu": dict(bytes=et * w13 + S * (d * 2 + I * 4 + 2 * I * 2 + I * 2),
                       flops=2.0 * S * 2 * I * d),
        "dz": dict(bytes=T * E * 4 + T * E * 6 * 2, flops=0.0),
        "dx_rows": dict(bytes=et * w13 + S * (2 * I * 2 + d * 4), flops=2.0 * S * 2 * I * d),
        "dw2": dict(bytes=N * w2 + S * (d * 2 + I * 2), flops=2.0 * S * d * I),
        "dw13": dict(bytes=N * w13 + S * (2 * I * 2 + d * 2), flops=2.0 * S * 2 * I * d),
        # algorithmic: the fp32 GEMMs dz^T x and dz W_r (the MFMA runs 18 T Ep d on planes)
        "router_grads": dict(bytes=T * E * 4 + T * d * 2 + 2 * E * d * 4 + T * d * 4,
                             flops=4.0 * T * E * d),
        "dx": dict(bytes=S * d * 4 + T * d * (2 + 4 + 4), flops=0.0),
    }


def measure_backward(cfg, L, x, steps, warmup, hip):
    """The layer backward (gradients of <dy, y> for x, W_r, W13, W2) on the
    same layer and batch, dy ~ N(0, 1) in bf16, timed per stage."""
    import torch
    from mixture_experts_layer_biased_amd import inputs, lcmoe

    shape = lcmoe.shape_of(cfg)
    T = x.shape[0]
    dy = inputs.make_upstream_grad(cfg, "cuda", tokens=T)
    ws = torch.empty(lcmoe.backward_workspace_bytes(shape, T), dtype=torch.uint8, device="cuda")
    out = dict(dx=torch.empty(T, cfg.d, dtype=torch.float32, device="cuda"),
               dw_router=torch.empty(cfg.n_experts, cfg.d, dtype=torch.float32, device="cuda"),
               dw13=torch.empty(cfg.n_ffn, 2 * cfg.inter, cfg.d, dtype=torch.bfloat16,
                                device="cuda"),
               dw2=torch.empty(cfg.n_ffn, cfg.d, cfg.inter, dtype=torch.bfloat16, device="cuda"))
    nst = len(lcmoe.BWD_STAGES)
    sets = make_event_sets(hip, steps, nst + 1)

    def step(ev=None):
        lcmoe.backward(shape, x, L["w_router"], L["bias"], L["w13"], L["w2"], dy, ws=ws, out=out,
                       stage_events=ev)

    # lcmoe_backward (the weight-gradient GEMMs on a second stream beside the
    # data-gradient GEMM) for the step time; then the staged entry point, which
    # runs the same kernels one after another on one stream with events
    # between them, for the per-stage times
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for s in range(steps):
        step()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    a.record()
    for s in range(steps):
        step(sets[s])
    b.record()
    torch.cuda.synchronize()
    seq_ms = a.elapsed_time(b) / steps
    per_stage = stage_ms(hip, sets, nst)
    for arr in sets:
        for i in range(nst + 1):
            hip.hipEventDestroy(arr[i])
    counts = lcmoe.route(shape, x, L["w_router"], L["bias"])["counts"].cpu().numpy()
    work = backward_work(cfg, counts, T)
    stages = {name: float(per_stage[i]) for i, name in enumerate(lcmoe.BWD_STAGES)}
    roof = {}
    for k, w in work.items():
        sec = stages[k] / 1e3
        roof[k] = dict(ms=stages[k], hbm_frac=w["bytes"] / sec / PEAK_HBM,
                       mfma_frac=w["flops"] / sec / PEAK_BF16)
    dom = max(work, key=lambda k: stages[k])
    w = work[dom]
    sec = stages[dom] / 1e3
    bound = "hbm" if w["flops"] / w["bytes"] < PEAK_BF16 / PEAK_HBM else "mfma"
    if bound == "hbm":
        ach, peak, unit = w["bytes"] / sec / 1e9, PEAK_HBM / 1e9, "GB/s"
    else:
        ach, peak, unit = w["flops"] / sec / 1e12, PEAK_BF16 / 1e12, "TFLOP/s"
    flops = sum(v["flops"] for v in work.values())
    # the training pair: the forward that also stores u (fp32) and the
    # backward that reads it instead of recomputing u = W13 x
    u = torch.empty(lcmoe.u_rows(shape, T), 2 * cfg.inter, dtype=torch.float32, device="cuda")
    fws = lcmoe.workspace(shape, T)

    def timed(fn, n):
        for _ in range(min(warmup, 2)):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    fwd_train_ms = timed(lambda: lcmoe.forward(shape, x, L["w_router"], L["bias"], L["w13"],
                                               L["w2"], ws=fws, u_save=u), steps)
    bwd_saved_ms = timed(lambda: lcmoe.backward(shape, x, L["w_router"], L["bias"], L["w13"],
                                                L["w2"], dy, ws=ws, out=out, u_saved=u), steps)
    del ws, out, dy, u, fws
    torch.cuda.empty_cache()
    return dict(tokens=T, ms_per_step=ms, tokens_per_s=T / (ms / 1e3), sequential_ms=seq_ms,
                stages_ms=stages,
                training_pair=dict(forward_train_ms=fwd_train_ms, backward_saved_ms=bwd_saved_ms,
                                   step_ms=fwd_train_ms + bwd_saved_ms),
                stage_roofline=roof, dominant_kernel=dom,
                roofline=dict(bound=bound, achieved=ach, peak=peak, unit=unit, frac=ach / peak,
                              algorithmic_bytes=w["bytes"], flops=w["flops"],
                              kernel_ms=stages[dom]),
                mfma_frac=flops / (ms / 1e3) / PEAK_BF16)


def copy_bandwidth(nbytes=4 << 30, reps=5):
    """Achievable HBM bandwidth of a plain device-to-device copy (read + write
    bytes per second), for reference next to the 8 TB/s peak."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    gbps = 2 * nbytes * reps / (a.elapsed_time(b) / 1e3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbps


def vendor_gemm(cfg, counts, stages, reps=5):
    """The vendor library's dense batched product (torch.bmm, i.e. hipBLASLt)
    at the layer's grouped shape, next to the grouped kernels' own figures:
    every touched expert gets the mean row count of the touched experts,
    rounded up to 32; bf16 operands [batch][k][n] with a contiguous right
    operand; fp32 accumulation. Context only: a dense product, with no row
    gather, no ragged row counts and no SiLU epilogue. bf16 weights only."""
    import torch
    rows = counts[: cfg.n_ffn]
    big = rows[rows > 0]
    if cfg.wdtype != "bf16" or big.size == 0:
        return None
    nb = int(big.size)
    m = int(-(-int(np.ceil(big.mean())) // 32) * 32)
    work = kernel_work(cfg, counts)
    out = {"experts": nb, "rows_per_expert": m}
    g = torch.Generator(device="cuda").manual_seed(0)
    for name, k, n in (("gateup", cfg.d, 2 * cfg.inter), ("down", cfg.inter, cfg.d)):
        a = torch.randn(nb, m, k, device="cuda", dtype=torch.bfloat16, generator=g)
        b = torch.randn(nb, k, n, device="cuda", dtype=torch.bfloat16, generator=g)
        c = torch.bmm(a, b)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch.bmm(a, b, out=c)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        flops = 2.0 * nb * m * k * n
        own = work[name]
        own_ms = stages[name]
        out[name] = dict(vendor_ms=ms, vendor_tflops=flops / ms / 1e9,
                         vendor_frac=flops / (ms / 1e3) / PEAK_BF16,
                         grouped_ms=own_ms, grouped_tflops=own["flops"] / own_ms / 1e9,
                         grouped_frac=own["flops"] / (own_ms / 1e3) / PEAK_BF16)
        del a, b, c
        torch.cuda.empty_cache()
    return out


def cpu_baseline(cfg, L, x, out, n_experts_sample):
    """The oracle on a bounded sample of the same workload: the full router,
    selection and gates for all T tokens, plus the SiLU-gated FFN of a sample
    of touched experts on all their routed tokens; the expert part is scaled by
    (touched experts / sampled experts)."""
    import oracle
    from tests.helpers import bf16_values, expert_getter
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    T = cfg.tokens
    t0 = time.perf_counter()
    xv = bf16_values(x)
    r = oracle.route(xv, L["w_router"].cpu().numpy(), L["bias"].cpu().numpy(), cfg.k)
    t_route = time.perf_counter() - t0
    idx = r["idx"]
    touched = [e for e in range(cfg.n_ffn) if (idx == e).any()]
    sample = touched[:: max(1, len(touched) // n_experts_sample)][:n_experts_sample]
    get = expert_getter(L, cfg.wdtype)
    t1 = time.perf_counter()
    for e in sample:
        rows, ks = np.nonzero(idx == e)
        w13, w2 = get(e)
        _ = r["g"][rows, ks][:, None] * oracle.expert_ffn(xv[rows], w13, w2)
    t_exp = time.perf_counter() - t1
    est = t_route + t_exp * len(touched) / max(1, len(sample))
    return dict(value=T / est, unit="tokens/s", cores=int(threads), kind="oracle", projected=True,
                sample=(f"projected from a sample of the {cfg.name} workload (T={T}): router, "
                        f"selection and gates for all "
                        f"tokens ({t_route:.1f} s) + SiLU-gated FFN of {len(sample)} of "
                        f"{len(touched)} touched experts on all their routed tokens "
                        f"({t_exp:.1f} s), expert time scaled by {len(touched)}/{len(sample)}; "
                        f"the combine (per token a sum of K rows) not timed"),
                measured_s=t_route + t_exp)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", choices=["prefill", "decode", "fp8", "fp8a8", "prefill32k", "ep8_shard"],
                    default=None,
                    help="measure a single configuration (for profiling runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward measurement on the bf16 prefill batch")
    ap.add_argument("--backward-only", action="store_true",
                    help="measure only the backward on the prefill batch (for profiling runs)")
    ap.add_argument("--cpu-experts", type=int, default=240)
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="also time the vendor library's dense batched product at the grouped "
                         "shape of each bf16 workload (context, not part of the layer)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="fold rocprofv3 FETCH_SIZE / WRITE_SIZE runs into profiles/traffic.json")
    ap.add_argument("--trace-summary", metavar="TRACE_DIR",
                    help="write a rocprofv3 --stats summary to profiles/")
    ap.add_argument("--counter-summary", nargs="+", metavar="PMC_DIR",
                    help="fold rocprofv3 --pmc runs into profiles/counters_<workload>.md")
    ap.add_argument("--workload", default="prefill")
    ap.add_argument("--cmd", default="", help="the profiling command, recorded in the summary")
    ap.add_argument("--work-out", default=None,
                    help="write the measured workload's per-stage algorithmic work and event "
                         "timings to this JSON file (read by --trace-summary --work)")
    ap.add_argument("--work", default=None, help="work file for --trace-summary")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.workload, args.cmd)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary, args.workload, args.cmd,
                      os.path.join(ROOT, "profiles", f"kernel_stats_{args.workload}.md"), args.work)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary, args.workload, args.cmd,
                        os.path.join(ROOT, "profiles", f"counters_{args.workload}.md"))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark measures one GPU (the layer has no multi-GPU path "
                                   "here); --gpus must be 1"}))
        sys.exit(2)

    import torch
    from mixture_experts_layer_biased_amd import inputs, lcmoe
    lcmoe.lib()  # fail loudly if the HIP library is missing
    assert torch.cuda.is_available(), "no GPU visible"
    hip = _hip()
    if args.backward_only:
        cfg = inputs.CONFIGS["prefill"]
        L = inputs.make_layer(cfg, "cuda")
        x = inputs.make_tokens(cfg, "cuda")
        bw = measure_backward(cfg, L, x, args.steps, args.warmup, hip)
        print(json.dumps({"backward": bw}))
        return
    copy_gbps = copy_bandwidth()
    print(f"[bench] device copy: {copy_gbps:.0f} GB/s (read+write)", file=sys.stderr, flush=True)
    results = {}
    baseline = None
    names = [args.only] if args.only else ["prefill", "decode", "fp8", "fp8a8", "prefill32k",
                                           "ep8_shard"]
    for name in names:
        cfg = inputs.CONFIGS[name]
        res, keep = measure(cfg, args.steps, args.warmup, hip)
        results[name] = res
        if args.work_out and name == names[0]:
            os.makedirs(os.path.dirname(os.path.abspath(args.work_out)), exist_ok=True)
            with open(args.work_out, "w") as f:
                # trailing: layer calls made after the timed loop (the bias
                # loop's forwards), which the trace summary leaves out
                json.dump(dict(workload=name, wdtype=cfg.wdtype, steps=args.steps,
                               warmup=args.warmup, trailing=int(cfg.extra.get("bias_steps", 0)),
                               stage_work=res["stage_work"]), f, indent=1)
        if args.vendor_gemm:
            res["vendor_gemm"] = vendor_gemm(cfg, keep[2]["counts"].cpu().numpy(), res["stages_ms"])
            if res["vendor_gemm"]:
                vg = res["vendor_gemm"]
                print(f"[bench] {name} vendor dense bmm ({vg['experts']} x {vg['rows_per_expert']} "
                      f"rows): gate/up {vg['gateup']['vendor_tflops']:.0f} TFLOP/s vs grouped "
                      f"{vg['gateup']['grouped_tflops']:.0f}; down {vg['down']['vendor_tflops']:.0f} "
                      f"vs {vg['down']['grouped_tflops']:.0f}", file=sys.stderr, flush=True)
        print(f"[bench] {name}: {res['ms_per_step']:.3f} ms/step, "
              f"{res['tokens_per_s']:.0f} tok/s, dominant {res['dominant_kernel']} "
              f"{res['roofline']['frac']:.3f} of {res['roofline']['bound']}; router stats "
              f"{res['router_stats']['ms']:.3f} ms", file=sys.stderr, flush=True)
        if "bias_loop" in res:
            bl = res["bias_loop"]
            print(f"[bench] {name} bias loop: {bl['steps']} steps (mu={bl['mu']}, K_e={bl['k_e']}), "
                  f"mean FFN experts/token {min(bl['mean_ffn_experts_per_token']):.4f}.."
                  f"{max(bl['mean_ffn_experts_per_token']):.4f}, max deviation "
                  f"{100 * bl['max_rel_deviation']:.2f}% (within 1%: {bl['within_1pct']}), "
                  f"forward + update {bl['step_ms_median']:.3f} ms/step", file=sys.stderr, flush=True)
        if name == names[0] and not args.no_cpu_baseline:
            baseline = cpu_baseline(cfg, keep[0], keep[1], keep[2], args.cpu_experts)
        if name == "prefill" and not args.no_backward:
            res["backward"] = measure_backward(cfg, keep[0], keep[1], args.steps, args.warmup,
                                               hip)
            bw = res["backward"]
            print(f"[bench] {name} backward: {bw['ms_per_step']:.3f} ms/step (stages in sequence {bw['sequential_ms']:.3f}), dominant "
                  f"{bw['dominant_kernel']} {bw['roofline']['frac']:.3f} of "
                  f"{bw['roofline']['bound']}; training pair: forward with saved u "
                  f"{bw['training_pair']['forward_train_ms']:.3f} ms + backward from it "
                  f"{bw['training_pair']['backward_saved_ms']:.3f} ms", file=sys.stderr, flush=True)
        del keep
        torch.cuda.empty_cache()

    if not args.only:
        sm = measure_small(args.steps, args.warmup)
        results["small"] = sm
        print(f"[bench] small (d=1024, T=4096): warm {sm['warm']['ms_median']:.3f} ms, cold "
              f"{sm['cold']['ms_median']:.3f} ms ({sm['cold']['hbm_frac']:.3f} of HBM), graph "
              f"replay {sm['graph']['ms_median']:.3f} ms", file=sys.stderr, flush=True)

    main_name = names[0]
    m = results[main_name]
    cfg = inputs.CONFIGS[main_name]
    line = {
        "metric": METRIC,
        "value": m["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8-e4m3 weights, bf16 MFMA",
                  "fp8a8": "fp8-e4m3 weights and activations, fp8 MFMA"}[cfg.wdtype],
        "data": "synthetic",
        "config": {"workload": (f"LongCat-shape MoE layer, {main_name} batch: T={cfg.tokens}, "
                                f"d_model={cfg.d}, {cfg.n_ffn} FFN + {cfg.n_zero} zero experts, "
                                f"K={cfg.k}, I={cfg.inter}, {cfg.wdtype} weights, fp32 router"),
                   "tokens": cfg.tokens, "parallelism": "single GPU"},
        "roofline": {k: m["roofline"][k] for k in ("bound", "achieved", "peak", "unit",
                                                     "frac", "traffic")},
        "dominant_kernel": m["dominant_kernel"],
        "cpu_baseline": baseline,
        "backward": ({k: results["prefill"]["backward"][k] for k in
                      ("tokens", "ms_per_step", "sequential_ms", "tokens_per_s",
                       "dominant_kernel", "roofline", "training_pair")}
                     if "backward" in results.get("prefill", {}) else None),
        "copy_gbps": copy_gbps,
        "detail": results,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
