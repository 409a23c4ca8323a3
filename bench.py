"""Benchmark of the MI355X sparse-MoE layer forward (one GPU).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-decode] [--no-cpu]

One step = one moe_forward over the whole batch (router, dispatch, routed and shared SwiGLU experts,
combine) with every input resident in HBM. The default workload is the GLM-4.5-shaped prefill layer with
skewed expert load (N=8192, D=5120, E=160, k=8, d=1536), the prefill shape the MFMA target is quoted on;
the GLM-5-shaped decode step (N=32 on the GLM-5 prefill weights, D=6144, E=256 in 8 groups, keep 4, k=8,
d=2048) is measured after it and reported under "decode" with its HBM roofline.

Prints one JSON line. `roofline` covers the dominant kernel (the grouped gate_up GEMM + SwiGLU), timed
with HIP events recorded by the library on the launch stream over the timed steps; `traffic` comes from
rocprofv3 FETCH_SIZE / WRITE_SIZE summaries under profiles/ when they were taken on the current kernel
source. `cpu_baseline` times the oracle (routing + per-expert loop form) on the host on a bounded sample
of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

P_BF16 = 2516.6e12  # dense bf16 MFMA, FLOP/s
P_F32 = 157.3e12
HBM = 8.0e12  # B/s
METRIC = "MoE-layer tokens/s + % bf16 MFMA peak (prefill), % HBM BW (decode)"
DOMINANT = "experts_gate_up"
KERNEL_SOURCES = ["sparse_moe_layer_gate_amd/csrc/gemm_bf16.hip", "sparse_moe_layer_gate_amd/csrc/gemm_decode.hip",
                  "sparse_moe_layer_gate_amd/csrc/gemm.hip", "sparse_moe_layer_gate_amd/csrc/dispatch.hip",
                  "sparse_moe_layer_gate_amd/csrc/moe_internal.h"]  # kernels, launch choice, tile lists


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str) -> dict | None:
    """HBM bytes per launch of the dominant kernel from a committed rocprofv3 counter summary, if it was
    taken on the current kernel source. Format: 'key: value' lines."""
    path = os.path.join(ROOT, "profiles", f"{DOMINANT}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != kernel_source_hash():
        return None
    try:
        return {"bytes": float(kv["hbm_bytes_per_launch"]), "fetch": float(kv["fetch_bytes_per_launch"]),
                "write": float(kv["write_bytes_per_launch"])}
    except KeyError:
        return None


KERNEL_NAMES = {  # library stage -> substrings of the HIP kernel symbols that run it (first match wins)
    "experts_gate_up": [("grouped_bf16_w8<true>", "")],
    "experts_down": [("grouped_bf16_w8<false>", "")],
    "experts_gate_up_decode": [("grouped_bf16_decode<true", "")],
    "experts_down_decode": [("grouped_bf16_decode<false", "")],
}


def _csv_rows(path):
    import csv

    with open(path) as f:
        return list(csv.DictReader(f))


def _find(dirpath, suffix):
    for root, _, files in os.walk(dirpath):
        for fn in files:
            if fn.endswith(suffix):
                return os.path.join(root, fn)
    raise FileNotFoundError(f"no *{suffix} under {dirpath}")


def profile_summary(pdir: str, workload: str, decode: bool) -> str:
    """Markdown summary of a profiling directory laid out as
         trace/        rocprofv3 --kernel-trace --stats -f csv (this bench, this workload)
         FETCH_SIZE/   rocprofv3 --pmc FETCH_SIZE -f csv   (this bench, this workload; optional)
         WRITE_SIZE/   rocprofv3 --pmc WRITE_SIZE -f csv   (optional)
         FETCH_SIZE_copy/, WRITE_SIZE_copy/   the same counters on `bench.py --copy-calibration`
         MFMA/         rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_INSTS_MFMA
                       TCC_HIT_sum TCC_MISS_sum (optional)
         LOADS/        rocprofv3 --pmc GRBM_GUI_ACTIVE TA_TA_BUSY TA_BUFFER_READ_LDS_WAVEFRONTS
                       SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_VMEM_RD (optional)
       Byte counters are scaled by bytes-copied / counter-reading of the 1 GiB copy; with them, also writes
       the dominant kernel's traffic file read by the benchmark."""
    stats = _csv_rows(_find(os.path.join(pdir, "trace"), "_kernel_stats.csv"))
    lines = [f"# rocprofv3 kernel summary: {workload}", "",
             "| kernel | calls | avg ms | total % |", "|---|---:|---:|---:|"]
    for r in stats:
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e6:.4f} | "
                     f"{float(r['Percentage']):.2f} |")

    def per_kernel(sub, counter=None):
        rows = _csv_rows(_find(os.path.join(pdir, sub), "_counter_collection.csv"))
        acc = {}
        for r in rows:
            if counter and r["Counter_Name"] != counter:
                continue
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in acc.items()}

    if os.path.isdir(os.path.join(pdir, "FETCH_SIZE")):
        copy_bytes = float(1 << 30)
        cf = per_kernel("FETCH_SIZE_copy")
        cw = per_kernel("WRITE_SIZE_copy")
        kcopy = next(k for k in cf if "copyBuffer" in k)
        f_scale = copy_bytes / (cf[kcopy] * 1024.0)  # counters in KiB
        w_scale = copy_bytes / (cw[kcopy] * 1024.0)
        fetch = {k: v * 1024.0 for k, v in per_kernel("FETCH_SIZE").items()}
        write = {k: v * 1024.0 for k, v in per_kernel("WRITE_SIZE").items()}
        lines += ["", "## HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE, calibrated)", "",
                  f"Calibration on a 1 GiB device copy: FETCH_SIZE x {f_scale:.3f}, WRITE_SIZE x {w_scale:.3f}.", "",
                  "| kernel | fetch GB | write GB |", "|---|---:|---:|"]
        for k in fetch:
            if k in write:
                lines.append(f"| `{k[:90]}` | {fetch[k] * f_scale / 1e9:.3f} | {write[k] * w_scale / 1e9:.3f} |")
        dom = [k for a, b in KERNEL_NAMES["experts_gate_up_decode" if decode else "experts_gate_up"]
               for k in fetch if a in k and b in k]
        if dom:
            k = dom[0]
            fb, wb = fetch[k] * f_scale, write.get(k, 0.0) * w_scale
            path = os.path.join(ROOT, "profiles", f"{DOMINANT}_{workload}_traffic.txt")
            with open(path, "w") as f:
                f.write(f"# {DOMINANT} on {workload}: HBM bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE,\n"
                        f"# each scaled by bytes / counter on a 1 GiB device copy (bench.py --copy-calibration).\n"
                        f"# Commands: see profiles/README.md. Valid while kernel_source_sha matches.\n")
                f.write(f"kernel: {k}\nkernel_source_sha: {kernel_source_hash()}\n")
                f.write(f"fetch_scale: {f_scale:.4f}\nwrite_scale: {w_scale:.4f}\n")
                f.write(f"fetch_bytes_per_launch: {fb:.0f}\nwrite_bytes_per_launch: {wb:.0f}\n")
                f.write(f"hbm_bytes_per_launch: {fb + wb:.0f}\n")

    if os.path.isdir(os.path.join(pdir, "MFMA")):
        rows = _csv_rows(_find(os.path.join(pdir, "MFMA"), "_counter_collection.csv"))
        acc, dur = {}, {}
        for r in rows:
            k = r["Kernel_Name"]
            acc.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            dur.setdefault(k, set()).add((r["Dispatch_Id"], int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
        lines += ["", "## MFMA utilisation and clock (rocprofv3 --pmc, one pass)", "",
                  "GRBM_GUI_ACTIVE is summed over the 8 XCDs: cycles = GRBM_GUI_ACTIVE / 8, clock = cycles / "
                  "duration. MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs); at the measured clock "
                  "that is busy x clock / 2.4 GHz of the 2,516.6 TFLOP/s bf16 peak. L2 hit = TCC_HIT / "
                  "(TCC_HIT + TCC_MISS).", "",
                  "| kernel | avg ms (under counters) | clock GHz | MFMA busy | implied TFLOP/s | L2 hit |",
                  "|---|---:|---:|---:|---:|---:|"]
        for k, c in acc.items():
            mf = sum(c.get("SQ_VALU_MFMA_BUSY_CYCLES", [0.0]))
            if mf == 0:
                continue
            n = len(c["GRBM_GUI_ACTIVE"])
            cyc = sum(c["GRBM_GUI_ACTIVE"]) / n / 8
            ns = sum(d for _, d in dur[k]) / len(dur[k])
            busy = mf / n / (cyc * 1024)
            ghz = cyc / ns
            hit = sum(c.get("TCC_HIT_sum", [0.0])) / max(1.0, sum(c.get("TCC_HIT_sum", [0.0])) +
                                                          sum(c.get("TCC_MISS_sum", [0.0])))
            lines.append(f"| `{k[:70]}` | {ns / 1e6:.4f} | {ghz:.3f} | {busy:.1%} | "
                         f"{busy * ghz / 2.4 * P_BF16 / 1e12:.0f} | {hit:.1%} |")

    if os.path.isdir(os.path.join(pdir, "LOADS")):
        rows = _csv_rows(_find(os.path.join(pdir, "LOADS"), "_counter_collection.csv"))
        acc, dur = {}, {}
        for r in rows:
            k = r["Kernel_Name"]
            acc.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            dur.setdefault(k, set()).add((r["Dispatch_Id"], int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
        lines += ["", "## Direct loads and LDS (rocprofv3 --pmc, one pass)", "",
                  "Each load-to-LDS wavefront moves 64 lanes x 16 bytes: L2 -> LDS bytes = 1 KiB x "
                  "(TA_BUFFER_READ_LDS_WAVEFRONTS + TA_FLAT_READ_LDS_WAVEFRONTS), per CU and clock over the "
                  "kernel's cycles (GRBM_GUI_ACTIVE / 8) and 256 CUs. TA busy = TA_TA_BUSY / (cycles x 256). "
                  "LDS bank conflicts = SQ_LDS_BANK_CONFLICT / (SQ_LDS_IDX_ACTIVE - SQ_LDS_BANK_CONFLICT), "
                  "conflict cycles per conflict-free LDS cycle.", "",
                  "| kernel | avg ms (under counters) | L2 -> LDS GB | B / clock / CU | TA busy | LDS bank conflicts |",
                  "|---|---:|---:|---:|---:|---:|"]
        for k, c in acc.items():
            waves = sum(c.get("TA_BUFFER_READ_LDS_WAVEFRONTS", [0.0])) + sum(c.get("TA_FLAT_READ_LDS_WAVEFRONTS",
                                                                                    [0.0]))
            if waves == 0:
                continue
            n = len(c["GRBM_GUI_ACTIVE"])
            cyc = sum(c["GRBM_GUI_ACTIVE"]) / n / 8
            ns = sum(d for _, d in dur[k]) / len(dur[k])
            nbytes = waves / n * 1024.0
            ta = sum(c.get("TA_TA_BUSY", [0.0])) / n / (cyc * 256)
            conf = sum(c.get("SQ_LDS_BANK_CONFLICT", [0.0])) / n
            idx = sum(c.get("SQ_LDS_IDX_ACTIVE", [0.0])) / n
            lines.append(f"| `{k[:70]}` | {ns / 1e6:.4f} | {nbytes / 1e9:.2f} | {nbytes / (cyc * 256):.1f} | "
                         f"{ta:.1%} | {conf / max(1.0, idx - conf):.3f} |")
    return "\n".join(lines) + "\n"


def flops(w: synth.Workload, N: int) -> dict:
    """Algorithmic work of one forward: router (fp32) and the expert GEMMs (bf16)."""
    f32 = 2.0 * N * w.D * w.E
    gate_up = 4.0 * w.D * (N * w.k * w.d + N * w.d_sh)  # 2 (M) (D) (2 d): routed + shared
    down = 2.0 * w.D * (N * w.k * w.d + N * w.d_sh)
    return {"router": f32, "gate_up": gate_up, "down": down, "bf16": gate_up + down}


def algorithmic_bytes(w: synth.Workload, N: int, distinct: int) -> dict:
    es = 2 if w.dtype == "bf16" else 4
    expert = 3 * w.D * w.d * es
    weights = distinct * expert + w.n_shared * 3 * w.D * w.d * es
    router = 4 * w.E * w.D + 4 * w.E
    act = es * N * w.D * 2  # x in, y out
    gate_up = (distinct + w.n_shared) * 2 * w.d * w.D * es + es * N * w.D  # gate/up weights + x
    return {"layer": weights + router + act, "gate_up": gate_up}


def is_decode(w: synth.Workload) -> bool:
    """Batches under 4 rows per expert on average run the weight-streaming kernels."""
    return w.N * w.k < 4 * w.E


def measure(w: synth.Workload, r: dict) -> dict:
    """Layer-level rates and the dominant kernel's roofline from one timed run."""
    distinct = int(np.count_nonzero(r["counts"]))
    fl = flops(w, w.N)
    by = algorithmic_bytes(w, w.N, distinct)
    t_layer = r["ms_per_step"] * 1e-3
    gu_ms, gu_n = r["stages"][DOMINANT]
    gu_avg = gu_ms / max(gu_n, 1)
    traffic = read_traffic(w.name)
    traffic = None if traffic is None else traffic["bytes"]
    if is_decode(w):
        achieved = by["gate_up"] / (gu_avg * 1e-3)
        roof = {"bound": "hbm", "achieved": round(achieved / 1e9, 1), "peak": HBM / 1e9, "unit": "GB/s",
                "frac": round(achieved / HBM, 4), "traffic": traffic, "kernel": DOMINANT, "avg_ms": round(gu_avg, 4),
                "per_launch": f"gate/up weights of {distinct} routed + {w.n_shared} shared experts + x = "
                              f"{by['gate_up'] / 1e9:.4f} GB"}
    else:
        achieved = fl["gate_up"] / (gu_avg * 1e-3)
        roof = {"bound": "mfma", "achieved": round(achieved / 1e12, 2), "peak": P_BF16 / 1e12, "unit": "TFLOP/s",
                "frac": round(achieved / P_BF16, 4), "traffic": traffic, "kernel": DOMINANT,
                "avg_ms": round(gu_avg, 4),
                "per_launch": f"4 D (N k d + N d_sh) = {fl['gate_up'] / 1e12:.4f} TFLOP"}
    layer = {"tflops": round((fl["bf16"] + fl["router"]) / t_layer / 1e12, 2),
             "mfma_frac": round(fl["bf16"] / t_layer / P_BF16, 4),
             "hbm_frac": round(by["layer"] / t_layer / HBM, 4),
             "algorithmic_bytes": by["layer"],
             "distinct_experts": distinct, "max_rows_per_expert": int(r["counts"].max()),
             "stage_ms": {k: round(v[0] / max(v[1], 1), 4) for k, v in r["stages"].items() if v[1]}}
    return {"ms": r["ms_per_step"], "layer": layer, "roofline": roof}


def setup(w: synth.Workload):
    import torch

    import sparse_moe_layer_gate_amd as moe

    dev = synth.experts_device(w)
    wg, b = synth.router_host(w)
    dev["w_router"] = torch.from_numpy(wg).cuda()
    dev["e_bias"] = torch.from_numpy(b).cuda()
    x = synth.x_host(w)
    xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda() if x.dtype == np.uint16 else \
        torch.from_numpy(x).cuda()
    cfg = moe.config_of(w)
    ws = moe.alloc_workspace(cfg, w.N)
    y = torch.empty_like(xd)
    counts = torch.empty(w.E, dtype=torch.int32, device="cuda")
    if w.dtype == "bf16":
        # the router weight's bf16 split is taken once per weight, as when a checkpoint is loaded
        dev["w_router_prepared"] = moe.moe_router_prepare(cfg, dev["w_router"])
    weights = moe.weights_struct(cfg, dev)
    torch.cuda.synchronize()
    return {"cfg": cfg, "dev": dev, "weights": weights, "x": xd, "y": y, "ws": ws, "counts": counts}


def time_forward(w: synth.Workload, st: dict, steps: int, warmup: int) -> dict:
    import torch

    import sparse_moe_layer_gate_amd as moe

    def step(counts=None):
        moe.moe_forward(st["cfg"], w.N, st["x"], st["weights"], st["y"], st["ws"], counts_out=counts)

    step(st["counts"])
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # timed region: only the dominant kernel carries an event pair (events around every kernel add
    # ~3% to a decode step)
    moe.profile_begin([DOMINANT])
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    timed = moe.profile_end()
    # separate pass for the per-stage breakdown
    moe.profile_begin()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    stages = moe.profile_end()
    stages[DOMINANT] = timed[DOMINANT]
    counts = st["counts"].cpu().numpy()
    return {"ms_per_step": (t1 - t0) * 1e3 / steps, "stages": stages, "counts": counts}


def decode_sweep(w: synth.Workload, sizes: list, steps: int, warmup: int) -> list:
    """Token-count sweep at a decode shape ("Module 02 -- MoE: Capacity, Work, and Traffic", sections 1 and
    5: traffic, set by the distinct experts a batch touches, governs decode). Weights are generated once;
    batch N takes the first N tokens of the workload's x stream. Per N: time per step, distinct experts,
    collision rate (share of (token, slot) pairs whose expert another pair of the batch also uses), the
    algorithmic bytes and the achieved HBM rate."""
    import torch

    import sparse_moe_layer_gate_amd as moe

    wmax = w.with_tokens(max(sizes))
    st = setup(wmax)
    rows = []
    for N in sizes:
        wn = w.with_tokens(N)
        sub = {**st, "cfg": moe.config_of(wn), "x": st["x"][:N].contiguous(), "y": st["y"][:N].contiguous(),
               "ws": moe.alloc_workspace(moe.config_of(wn), N)}
        r = time_forward(wn, sub, steps, warmup)
        m = measure(wn, r)
        distinct = m["layer"]["distinct_experts"]
        by = m["layer"]["algorithmic_bytes"]
        uniform = w.E * (1.0 - (1.0 - w.k / w.E) ** N)  # expected distinct experts under uniform routing
        rows.append({"N": N, "ms_per_step": round(m["ms"], 4), "tokens_per_s": round(N / (m["ms"] * 1e-3), 1),
                     "distinct_experts": distinct, "uniform_expectation": round(uniform, 1),
                     "collision_rate": round(1.0 - distinct / (N * w.k), 4),
                     "algorithmic_gb": round(by / 1e9, 3), "gb_per_s": round(by / (m["ms"] * 1e-3) / 1e9, 1),
                     "hbm_frac": m["layer"]["hbm_frac"], "gate_up_ms": m["layer"]["stage_ms"].get(DOMINANT),
                     "gate_up_hbm_frac": m["roofline"]["frac"] if m["roofline"]["bound"] == "hbm" else None})
        print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
        del sub
    del st
    torch.cuda.empty_cache()
    return rows


def dense_bench(w, steps: int, warmup: int) -> dict:
    """The dense SwiGLU FFN (moe_dense_forward) at its full width: time per step, TFLOP/s and the MFMA
    fraction of each GEMM (algorithmic work 6 N D dff: gate_up 4 N D dff, down 2 N D dff)."""
    import torch

    import sparse_moe_layer_gate_amd as moe

    dev = synth.dense_device(w)
    x = synth.x_host(w)
    xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda() if x.dtype == np.uint16 else \
        torch.from_numpy(x).cuda()
    y = torch.empty_like(xd)
    ws = torch.empty(moe.moe_dense_workspace_size(w.N, w.D, w.dff, w.dtype), dtype=torch.uint8, device="cuda")

    def step():
        moe.moe_dense_forward(w.N, xd, dev["gate"], dev["up"], dev["down"], y, ws, limit=w.limit)

    for _ in range(warmup + 1):
        step()
    torch.cuda.synchronize()
    moe.profile_begin()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stages = moe.profile_end()
    ms = (t1 - t0) * 1e3 / steps
    fl = 6.0 * w.N * w.D * w.dff
    out = {"workload": w.name, "N": w.N, "D": w.D, "dff": w.dff, "ms_per_step": round(ms, 4),
           "tokens_per_s": round(w.N / (ms * 1e-3), 1), "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
           "mfma_frac": round(fl / (ms * 1e-3) / P_BF16, 4)}
    for name, share in (("experts_gate_up", 4.0), ("experts_down", 2.0)):
        t, n = stages[name]
        avg = t / max(n, 1)
        out[name.replace("experts_", "") + "_ms"] = round(avg, 4)
        out[name.replace("experts_", "") + "_mfma_frac"] = round(share * w.N * w.D * w.dff / (avg * 1e-3) / P_BF16, 4)
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w: synth.Workload, tokens: int, runs: int = 3) -> dict:
    """The oracle (routing + per-expert loop form) on the first `tokens` tokens of the workload: the
    median wall time of `runs` runs, with the host's threads and CPU model."""
    import oracle

    sub = w.with_tokens(tokens)
    x = synth.x_host(w, 0, tokens)
    wg, b = synth.router_host(w)
    times = []
    table = None
    for _ in range(runs):
        t0 = time.perf_counter()
        s = oracle.scores(sub, x, wg)
        idx, wt = oracle.select(sub, s, b)
        t_route = time.perf_counter() - t0
        if table is None:  # weight generation is set-up, not timed
            needed = {int(e): synth.expert_host(w, int(e)) for e in np.unique(idx)}
            table = oracle.ExpertTable(sub, needed, synth.shared_host(w))
        t1 = time.perf_counter()
        oracle.forward_expert_loop(sub, x, table, idx, wt)
        times.append(t_route + time.perf_counter() - t1)
    secs = float(np.median(times))
    return {"value": round(tokens / secs, 2), "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "cpu_model": cpu_model(), "runs": runs, "seconds_median": round(secs, 3),
            "seconds_all": [round(t, 3) for t in times],
            "sample": f"first {tokens} of {w.N} tokens ({tokens / w.N:.1%}) of {w.name}: oracle routing (double "
                      f"logits, float32 selection) + per-expert loop form in double; median of {runs} runs; "
                      f"weight generation not timed"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="glm45_prefill_skewed", choices=synth.WORKLOAD_ORDER)
    ap.add_argument("--decode-steps", type=int, default=100)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=1024)
    ap.add_argument("--cpu-runs", type=int, default=3)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling rocprofv3 byte counters)")
    ap.add_argument("--profile-summary", metavar="DIR",
                    help="summarise rocprofv3 output under DIR for --workload (no GPU needed) and exit")
    ap.add_argument("--decode-sweep", action="store_true",
                    help="time --workload (a decode shape) at N = 1, 2, 4, ..., 256 tokens and print a table")
    ap.add_argument("--dense", choices=sorted(synth.DENSE_WORKLOADS),
                    help="time the dense SwiGLU FFN of this shape instead of the MoE layer and print one JSON line")
    args = ap.parse_args()
    if args.profile_summary:
        w = synth.WORKLOADS[args.workload]
        print(profile_summary(args.profile_summary, w.name, is_decode(w)), end="")
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_moe_layer_gate_amd  # noqa: F401  (fails loudly if libmoe.so is missing)

    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}))
        return

    if args.dense:
        print(json.dumps(dense_bench(synth.DENSE_WORKLOADS[args.dense], args.steps, args.warmup)), flush=True)
        return
    w = synth.WORKLOADS[args.workload]
    if args.decode_sweep:
        rows = decode_sweep(w, [1 << i for i in range(9)], args.decode_steps, args.warmup)
        keys = list(rows[0].keys())
        print(f"decode sweep, {w.name} (D={w.D}, E={w.E}, G={w.G}, TG={w.TG}, k={w.k}, d={w.d}, "
              f"n_shared={w.n_shared}), {args.decode_steps} steps per N\n")
        print("| " + " | ".join(keys) + " |")
        print("|" + "---|" * len(keys))
        for r in rows:
            print("| " + " | ".join(str(r[k]) for k in keys) + " |")
        return
    print(f"[bench] {w.name}: generating inputs", file=sys.stderr, flush=True)
    st = setup(w)
    r = time_forward(w, st, args.steps, args.warmup)
    m = measure(w, r)
    out = {
        "metric": METRIC,
        "value": round(w.N / (m["ms"] * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "N": w.N, "D": w.D, "E": w.E, "n_group": w.G, "topk_group": w.TG,
                   "k": w.k, "d_moe": w.d, "n_shared": w.n_shared, "alpha": w.alpha, "parallelism": "none"},
        "layer": m["layer"],
        "roofline": m["roofline"],
    }
    del st
    torch.cuda.empty_cache()

    if not args.no_decode:
        wd = synth.WORKLOADS["glm5_decode"]
        print(f"[bench] {wd.name}: generating inputs", file=sys.stderr, flush=True)
        sd = setup(wd)
        md = measure(wd, time_forward(wd, sd, args.decode_steps, args.warmup))
        out["decode"] = {"workload": wd.name, "tokens_per_s": round(wd.N / (md["ms"] * 1e-3), 1),
                         "ms_per_step": round(md["ms"], 4), "layer": md["layer"], "roofline": md["roofline"]}
        del sd
        torch.cuda.empty_cache()

    if not args.no_cpu:
        print(f"[bench] cpu baseline: oracle on {args.cpu_tokens} tokens", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_tokens, args.cpu_runs)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
