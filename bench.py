#!/usr/bin/env python3
"""Benchmark of one dropless top-k MoE expert layer, forward + backward, on
one MI355X.

A step is one pass of the whole layer over one batch of synthetic inputs
already resident in HBM: route -> dispatch -> grouped FFN forward ->
combine, then combine backward -> grouped FFN backward -> dispatch backward
-> router backward, all through the C ABI (libmoe_hip.so).

    python bench.py [--steps K] [--warmup W] [--workload NAME]

Prints one JSON line.  `value` is tokens per second of the whole layer
(forward + backward).  A few untimed steps with a HIP event after every
kernel give the per-kernel table and name the dominant kernel; inside the
timed region only that kernel's launches are bracketed by HIP events on the
library's stream, and their mean duration gives the `roofline` object.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.
`clock` is read by a pure-MFMA probe right after the timed steps.  For the
default (OLMoE-shaped, bf16) workload, the expert-count scan (E = 8, 32,
128), the bf16 and MXFP8 layers and one GPU's share of the trillion-scale
layer are also timed in the same run, one after the other and in the same
way ("companions"), for the E=128 / E=8 throughput ratio and the MXFP8
speed-up over bf16.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd+bwd tokens/s and TFLOP/s (% of MI355X bf16/MXFP8 MFMA peak)"
PEAK_TFLOPS = {"bf16": 2500.0, "mxfp8": 5000.0, "fp32": 157.3}
HBM_PEAK_GBS = 8000.0


def gemm_flops(name: str, wl) -> float:
    """Algorithmic FLOPs of one launch of a GEMM kernel: 2 * rows * (output
    width) * (contraction) with only the routed rows counted."""
    R, T, d, f, E = wl.R, wl.T, wl.d, wl.f, wl.E
    per_row = {
        "gemm_fwd_gateup_swiglu": 4.0 * d * f,      # Xs . [Wg|Wu]
        "gemm_fwd_down": 2.0 * f * d,               # A . Wd
        "gemm_dgrad_down_swiglu_bwd": 2.0 * d * f,  # dYs . Wd^T
        "gemm_dgrad_gateup": 4.0 * f * d,           # [dHg|dHu] . [Wg|Wu]^T
        "gemm_wgrad_gateup": 4.0 * d * f,           # Xs^T . [dHg|dHu]
        "gemm_wgrad_down": 2.0 * f * d,             # A^T . dYs
    }
    if name.startswith("gemm_mx_"):
        name = "gemm_" + name[len("gemm_mx_"):]
    if name in per_row:
        return per_row[name] * R
    if name in ("router_logits", "router_dx", "router_dwr", "gemm_router_logits",
                "gemm_router_dwr", "gemm_router_dx"):
        return 2.0 * T * d * E
    return 0.0


# ---------------------------------------------------------------------------
# measured HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE)
# ---------------------------------------------------------------------------
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "routing_grouped_gemm_amd", "csrc")

# rocprofv3 kernel symbol -> the library's launch names, in launch order
# within one step (the weight-gradient kernel runs twice per step)
_SYMBOLS = {
    "gemm_bf16_kernel<0>": ["gemm_fwd_gateup_swiglu"],
    "gemm_bf16_kernel<1>": ["gemm_fwd_down"],
    "gemm_bf16_kernel<2>": ["gemm_dgrad_down_swiglu_bwd"],
    "gemm_bf16_kernel<3>": ["gemm_dgrad_gateup"],
    "gemm_bf16_kernel<4>": ["gemm_wgrad_gateup", "gemm_wgrad_down"],
    "gemm8_kernel<4>": ["gemm_wgrad_gateup", "gemm_wgrad_down"],
    "gemm_bf16_kernel<5>": ["gemm_router_logits"],
    "gemm_bf16_kernel<7>": ["gemm_router_dx"],
    "gemm_bf16_kernel<12>": ["gemm_router_dwr"],
    "gemm_mx_kernel<8>": ["gemm_mx_fwd_gateup_swiglu"],
    "gemm_mx_kernel<9>": ["gemm_mx_fwd_down"],
    "gemm_mx_kernel<10>": ["gemm_mx_dgrad_down_swiglu_bwd"],
    "gemm_mx_kernel<11>": ["gemm_mx_dgrad_gateup"],
    "gemm_mx_kernel<14>": ["gemm_mx_wgrad_gateup", "gemm_mx_wgrad_down"],
    "gemm_mx_kernel<15>": ["gemm_mx_wgrad_gateup", "gemm_mx_wgrad_down"],
    "dispatch_scatter_kernel": ["dispatch_copy"],
    "router_logits_kernel": ["router_logits"],
    "router_dx_kernel": ["router_dx"],
    "router_dwr_kernel": ["router_dwr"],
    "mx_dispatch_kernel": ["mx_dispatch_quant"],
    "combine_kernel": ["combine"],
    "combine_bwd_kernel": ["combine_bwd"],
    "gather_sum_kernel": ["gather_sum"],
    "skinny_kernel<0>": ["skinny_fwd_gateup"],
    "skinny_kernel<1>": ["skinny_fwd_down"],
    "skinny_reduce_kernel<0>": ["skinny_reduce_gateup"],
    "skinny_reduce_kernel<1>": ["skinny_reduce_down"],
    "route_part_kernel": ["route_small_part"],
    "route_final_kernel": ["route_small_final"],
    "dispatch_small_kernel": ["dispatch_small"],
    "mx_quant_both_kernel": ["mx_quant_weights"],
    "combine_small_kernel": ["combine_small"],
}


def source_hash() -> str:
    """Digest of the HIP sources: measured traffic is reported only for the
    kernels it was measured on."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h"))):
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _counter_means(directory: str):
    """Mean counter value per launch name from a rocprofv3 --pmc csv directory."""
    import csv
    import glob
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    rows = []
    for path in files:
        with open(path) as fh:
            rows += list(csv.DictReader(fh))
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    seen = {}
    acc = {}
    for r in rows:
        name = r["Kernel_Name"].split("(")[0].replace("void ", "").replace("moe::mf::", "")
        name = name.replace("moe::sk::", "").replace("moe::mf8::", "").replace("moe::", "")
        sym = next((k for k in _SYMBOLS if name.startswith(k.split("<")[0]) and
                    (("<" not in k) or name.startswith(k))), name)
        n = seen.get(sym, 0)
        seen[sym] = n + 1
        names = _SYMBOLS.get(sym, [sym])
        launch = names[n % len(names)]
        acc.setdefault(launch, []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def write_traffic(workload_name, fetch_dir, write_dir, cal_fetch_dir, cal_write_dir) -> int:
    fetch, write = _counter_means(fetch_dir), _counter_means(write_dir)
    cf = _counter_means(cal_fetch_dir)["__amd_rocclr_copyBuffer"]
    cw = _counter_means(cal_write_dir)["__amd_rocclr_copyBuffer"]
    # the calibration copy moves exactly 1 GiB each way; counters are in KiB
    sf, sw = (1 << 30) / (cf * 1024.0), (1 << 30) / (cw * 1024.0)
    data = {}
    if os.path.exists(TRAFFIC_JSON):
        with open(TRAFFIC_JSON) as fh:
            data = json.load(fh)
    h = source_hash()
    if data.get("source_hash") != h:
        data = {"source_hash": h, "workloads": {}}
    data["workloads"][workload_name] = {
        "calibration": {"fetch_scale": round(sf, 4), "write_scale": round(sw, 4),
                        "copy_bytes": 1 << 30},
        "kernels": {k: {"fetch_bytes": int(fetch[k] * 1024 * sf),
                        "write_bytes": int(write.get(k, 0.0) * 1024 * sw)}
                    for k in sorted(fetch)},
    }
    os.makedirs(os.path.dirname(TRAFFIC_JSON), exist_ok=True)
    with open(TRAFFIC_JSON, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
    print(json.dumps({"traffic_json": TRAFFIC_JSON, "workload": workload_name,
                      "kernels": len(fetch), "source_hash": h}))
    return 0


def mfma_summary(workload_name: str, directory: str) -> int:
    """Per-kernel MFMA utilisation and clock from one rocprofv3 --pmc run.

    SQ_VALU_MFMA_BUSY_CYCLES counts 32 SIMD cycles per issued 32x32x16 bf16
    MFMA (64 per scaled fp8 32x32x64), so against 4 SIMDs x SQ_BUSY_CU_CYCLES
    (busy cycles summed over the CUs) it is the fraction of SIMD cycles the
    matrix cores were busy; the clock probe (pure MFMA work) reads 100% this
    way.  GRBM_GUI_ACTIVE sums the busy cycles of the 8 XCDs, so / 8 over the
    dispatch's duration is the clock it ran at."""
    import csv
    import glob
    from moe_synth import workload
    wl = workload(workload_name)
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    disp = {}
    for path in files:
        with open(path) as fh:
            for r in csv.DictReader(fh):
                d = disp.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"],
                                                            "ns": int(r["End_Timestamp"]) -
                                                            int(r["Start_Timestamp"])})
                d[r["Counter_Name"]] = float(r["Counter_Value"])
    seen, acc = {}, {}
    for i in sorted(disp):
        d = disp[i]
        name = d["name"].split("(")[0].replace("void ", "")
        for pre in ("moe::mf::", "moe::mf8::", "moe::sk::", "moe::"):
            name = name.replace(pre, "")
        sym = next((k for k in _SYMBOLS if name.startswith(k.split("<")[0]) and
                    (("<" not in k) or name.startswith(k))), name)
        if "clock_probe" in d["name"]:
            # the probe's short warm-up launch (it loads the code object) is left out
            if d["ns"] < 100_000:
                continue
            launch = "clock_probe (pure MFMA, every CU)"
        else:
            n = seen.get(sym, 0)
            seen[sym] = n + 1
            names = _SYMBOLS.get(sym, [sym])
            launch = names[n % len(names)]
        acc.setdefault(launch, []).append(d)
    w = workload_name
    comp = " --no-companions" if w == "olmoe_bf16" else ""
    print(f"# {w}: matrix-core utilisation and clock per kernel\n")
    print(f"Workload: T={wl.T}, d={wl.d}, E={wl.E}, f={wl.f}, k={wl.k}, {wl.prec}.  One MI355X.  "
          f"Source digest (`bench.py` `source_hash()`): `{source_hash()}`.\n")
    print("`SQ_VALU_MFMA_BUSY_CYCLES` counts 32 SIMD cycles per 32x32x16 bf16 MFMA (64 per "
          "scaled fp8 32x32x64); against 4 x `SQ_BUSY_CU_CYCLES` it is the fraction of SIMD "
          "cycles the matrix cores were busy (the clock probe, pure MFMA work on every CU, reads "
          "~100%).  `GRBM_GUI_ACTIVE` / 8 XCDs over a dispatch's duration is the clock it ran at "
          "(shown for dispatches of 100 µs or more).  TFLOP/s count routed rows only.\n")
    print("Commands (repository root; `export TMPDIR=/tmp` first; OUT is any scratch directory):\n")
    print("```")
    print(f"rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE -d "
          f"OUT/pmc_mfma_{w} -o run --output-format csv -- python3 bench.py --workload {w} "
          f"--steps 5 --warmup 2 --cpu-tokens 0{comp}")
    print(f"python3 bench.py --workload {w} --mfma-summary OUT/pmc_mfma_{w} > "
          f"profiles/{w}_mfma_counters.md")
    print("```\n")
    print("| kernel | launches | mean µs | clock MHz | MFMA busy (% of SIMD cycles) | "
          "algorithmic TFLOP/s | frac of 2.5 PF | frac of peak at its clock |")
    print("|---|---:|---:|---:|---:|---:|---:|---:|")
    order = sorted(acc, key=lambda k: -sum(x["ns"] for x in acc[k]))
    for k in order:
        ds = acc[k]
        need = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE")
        if not all(c in ds[0] for c in need):
            continue
        us = sum(x["ns"] for x in ds) / len(ds) / 1e3
        mhz = sum(x["GRBM_GUI_ACTIVE"] / 8.0 / (x["ns"] * 1e-3) for x in ds) / len(ds)
        busy = sum(x["SQ_VALU_MFMA_BUSY_CYCLES"] for x in ds) / \
            max(1.0, 4.0 * sum(x["SQ_BUSY_CU_CYCLES"] for x in ds))
        fl = gemm_flops(k, wl)
        peak = PEAK_TFLOPS["mxfp8" if k.startswith("gemm_mx_") else "bf16"]
        if k.startswith("clock_probe"):
            fl = None
        if fl:
            tf = fl / (us * 1e-6) / 1e12
            at_clk = f"{tf / (peak * mhz / 2400.0):.3f}" if us >= 100.0 else "-"
            cols = f"{tf:.0f} | {tf / peak:.3f} | {at_clk}"
        else:
            cols = "- | - | -"
        if busy == 0.0 and not fl and not k.startswith("clock_probe"):
            continue
        # the busy-cycle window of a dispatch shorter than ~0.1 ms does not
        # match its timestamps well enough for a clock
        clk = f"{mhz:.0f}" if us >= 100.0 else "-"
        print(f"| `{k}` | {len(ds)} | {us:.1f} | {clk} | {100.0 * busy:.1f} | {cols} |")
    return 0


SQ_PASSES = (
    "SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_BUSY_CU_CYCLES SQ_VALU_MFMA_BUSY_CYCLES "
    "SQ_WAIT_INST_LDS SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_VMEM",
    "SQ_VMEM_TA_CMD_FIFO_FULL SQ_VMEM_TA_ADDR_FIFO_FULL SQ_LDS_DATA_FIFO_FULL "
    "SQ_LDS_CMD_FIFO_FULL SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS SQ_INSTS_VMEM",
)


def sq_summary(workload_name: str, dirs) -> int:
    """Where the expert GEMMs' waves spend their cycles, from the two
    rocprofv3 --pmc passes of SQ_PASSES: per-wave stall fractions (the
    SQ_WAIT_*/SQ_ACTIVE_* counters are in wave quad-cycles against
    SQ_WAVE_CYCLES) and, per CU and clock cycle of the dispatch, how often the
    TA and LDS queues were full and the LDS busy."""
    import csv
    import glob
    acc, ns = {}, {}
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as fh:
                for r in csv.DictReader(fh):
                    name = _symbol_of(r["Kernel_Name"])
                    if not (name.startswith("gemm_bf16_kernel") or name.startswith("gemm8_kernel")):
                        continue
                    acc.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(
                        float(r["Counter_Value"]))
                    if r["Counter_Name"] == "SQ_INSTS_LDS":
                        ns.setdefault(name, []).append(
                            int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    w = workload_name
    comp = " --no-companions" if w == "olmoe_bf16" else ""
    print(f"# {w}: where the GEMM waves wait (SQ counters)\n")
    print(f"Source digest (`bench.py` `source_hash()`): `{source_hash()}`.  One MI355X.\n")
    print("Commands (repository root; `export TMPDIR=/tmp` first; OUT is any scratch directory):\n")
    print("```")
    for i, p in enumerate(SQ_PASSES):
        print(f"rocprofv3 --pmc {p} -d OUT/sq{i + 1}_{w} -o run --output-format csv -- python3 "
              f"bench.py --workload {w} --steps 3 --warmup 1 --cpu-tokens 0{comp}")
    print(f"python3 bench.py --workload {w} --sq-summary OUT/sq1_{w} OUT/sq2_{w} > "
          f"profiles/{w}_sq_counters.md")
    print("```\n")
    print("Per wave cycle: waiting on `s_waitcnt` or a barrier (WAIT_ANY), an instruction "
          "ready but not issued (WAIT_INST_ANY: mostly an MFMA waiting for the matrix core), "
          "issuing LDS and vector-memory instructions.  Per CU and cycle (the device-wide sums "
          "over 256 CUs times the dispatch's duration at 2.05 GHz): TA command/address queue full, "
          "LDS data queue full, LDS busy with indexed accesses, LDS bank-conflict stalls.\n")
    print("| kernel | µs | MFMA busy | WAIT_ANY | WAIT_INST_ANY | LDS issue | VMEM issue | "
          "TA cmd full | TA addr full | LDS data full | LDS busy | bank conflict |")
    print("|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|")
    for name in sorted(acc):
        m = {k: sum(v) / len(v) for k, v in acc[name].items()}
        if "SQ_WAVE_CYCLES" not in m or "SQ_INSTS_LDS" not in m:
            continue
        wc = 4.0 * m["SQ_WAVE_CYCLES"]
        dur = sum(ns[name]) / len(ns[name])
        cyc = 256.0 * dur * 2.05
        f = lambda k: 4.0 * m[k] / wc
        c = lambda k: m[k] / cyc
        busy = m["SQ_VALU_MFMA_BUSY_CYCLES"] / (4.0 * m["SQ_BUSY_CU_CYCLES"])
        launches = " + ".join(dict.fromkeys(_SYMBOLS.get(name, [name])))
        print(f"| `{name}` ({launches}) | {dur / 1e3:.0f} | {busy:.2f} | {f('SQ_WAIT_ANY'):.2f} | "
              f"{f('SQ_WAIT_INST_ANY'):.2f} | {f('SQ_ACTIVE_INST_LDS'):.2f} | "
              f"{f('SQ_ACTIVE_INST_VMEM'):.2f} | {c('SQ_VMEM_TA_CMD_FIFO_FULL'):.3f} | "
              f"{c('SQ_VMEM_TA_ADDR_FIFO_FULL'):.3f} | {c('SQ_LDS_DATA_FIFO_FULL'):.3f} | "
              f"{c('SQ_LDS_IDX_ACTIVE'):.3f} | {c('SQ_LDS_BANK_CONFLICT'):.3f} |")
    return 0


def _symbol_of(kernel_name: str) -> str:
    name = kernel_name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
    for pre in ("moe::mf::", "moe::mf8::", "moe::sk::", "moe::st::", "moe::"):
        name = name.replace(pre, "")
    return name


def profile_markdown(workload_name: str, kt_dir: str) -> int:
    """The committed per-workload profile summary: the rocprofv3 kernel trace
    of a bench run (kernel_stats.csv under kt_dir) and, while the sources are
    the ones they were taken on, the calibrated HBM bytes per launch of
    profiles/traffic.json; printed as markdown on stdout."""
    import csv
    import glob
    from moe_synth import workload
    wl = workload(workload_name)
    files = glob.glob(os.path.join(kt_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {kt_dir}")
    with open(files[0]) as fh:
        rows = list(csv.DictReader(fh))
    fwd_only = workload_name.startswith("olmoe_decode")
    w = workload_name
    # the default workload is traced with the bench's own step counts (50
    # timed after 10 warm-up), so that the trace's average of the priced
    # kernel compares with the per-launch time of the bench line
    steps = ("--steps 200 --warmup 20" if fwd_only else
             "--steps 50 --warmup 10" if w == "olmoe_bf16" else "--steps 20 --warmup 2")
    comp = "" if fwd_only or w != "olmoe_bf16" else " --no-companions"
    what = "the small-batch forward" if fwd_only else "one forward+backward step"
    routed = wl.T * wl.k
    print(f"# {w}: per-kernel profile of {what}\n")
    print(f"Workload: T={wl.T}, d={wl.d}, E={wl.E}, f={wl.f}, k={wl.k}, {wl.prec}, routing "
          f"{wl.routing} (R={routed} routed rows).  One MI355X.  Source digest of the kernels "
          f"profiled (`bench.py` `source_hash()`): `{source_hash()}`.\n")
    print("Commands (repository root; `export TMPDIR=/tmp` first; OUT is any scratch directory):\n")
    print("```")
    print(f"rocprofv3 --kernel-trace --stats -d OUT/kt_{w} -o run --output-format csv -- "
          f"python3 bench.py --workload {w} {steps} --cpu-tokens 0{comp}")
    if not fwd_only:
        for c, tag in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
            print(f"rocprofv3 --pmc {c} -d OUT/{tag}_{w} -o run --output-format csv -- python3 "
                  f"bench.py --workload {w} --steps 2 --warmup 1 --cpu-tokens 0{comp}")
        for c, tag in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
            print(f"rocprofv3 --pmc {c} -d OUT/cal_{tag} -o run --output-format csv -- python3 "
                  f"bench.py --calibrate-copy 1024")
        print(f"python3 bench.py --workload {w} --traffic OUT/fetch_{w} OUT/write_{w} "
              f"OUT/cal_fetch OUT/cal_write   # -> profiles/traffic.json")
    print(f"python3 bench.py --workload {w} --profile-md OUT/kt_{w} > profiles/{w}_layer_kernels.md")
    print("```\n")
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    print("## Kernel trace (`run_kernel_stats.csv`; the run's warm-up, per-kernel-event and "
          "timed steps together)\n")
    print("| kernel | launch name(s) | calls | average µs | share |")
    print("|---|---|---:|---:|---:|")
    avg_us = {}  # launch name (one name per kernel only) or kernel symbol -> average µs
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = _symbol_of(r["Name"])
        if name.startswith("__amd_rocclr") or "elementwise" in name or "at::" in name:
            continue
        sym = next((k for k in _SYMBOLS if name.startswith(k.split("<")[0]) and
                    (("<" not in k) or name.startswith(k))), None)
        launches = " + ".join(dict.fromkeys(_SYMBOLS[sym])) if sym else ""
        if name.startswith("clock_probe"):
            launches = "clock probe after the timed steps (not part of a step)"
        share = 100.0 * float(r["TotalDurationNs"]) / total
        print(f"| `{name}` | {launches} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
              f"{share:.2f}% |")
        avg_us[name] = float(r["AverageNs"]) / 1e3
        if sym and len(set(_SYMBOLS[sym])) == 1:
            avg_us[_SYMBOLS[sym][0]] = float(r["AverageNs"]) / 1e3
    print()
    try:
        with open(TRAFFIC_JSON) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        data = {}
    tw = data.get("workloads", {}).get(w) if data.get("source_hash") == source_hash() else None
    if tw:
        cal = tw["calibration"]
        print("## HBM traffic per launch (calibrated)\n")
        print(f"On a 1 GiB device-to-device copy FETCH_SIZE reports {1.0 / cal['fetch_scale']:.4f} "
              f"and WRITE_SIZE {1.0 / cal['write_scale']:.4f} of the true bytes, so every counter "
              f"below is multiplied by {cal['fetch_scale']:.4f} (fetch) and "
              f"{cal['write_scale']:.4f} (write).\n")
        print("The rate is the launch's bytes over its average duration in the trace above, "
              "where that kernel serves this launch alone (a kernel shared by two launches, "
              "such as the eight-wave weight-gradient GEMM, has no per-launch average), "
              f"against the {HBM_PEAK_GBS / 1000:.0f} TB/s HBM peak.\n")
        print("| launch | fetch MB | write MB | total MB | average µs | GB/s | frac of HBM peak |")
        print("|---|---:|---:|---:|---:|---:|---:|")
        ks = tw["kernels"]
        for k in sorted(ks, key=lambda k: -(ks[k]["fetch_bytes"] + ks[k]["write_bytes"])):
            f_, w_ = ks[k]["fetch_bytes"] / 1e6, ks[k]["write_bytes"] / 1e6
            if f_ + w_ < 1.0:
                continue
            us = avg_us.get(k)
            if us:
                gbs = (f_ + w_) * 1e6 / (us * 1e-6) / 1e9
                rate = f"{us:.1f} | {gbs:.0f} | {gbs / HBM_PEAK_GBS:.2f}"
            else:
                rate = "- | - | -"
            print(f"| `{k}` | {f_:.0f} | {w_:.0f} | {f_ + w_:.0f} | {rate} |")
        print()
    return 0


def measured_traffic(workload_name: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None when there is none or the sources changed since it was taken."""
    try:
        with open(TRAFFIC_JSON) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        return None
    if data.get("source_hash") != source_hash():
        return None
    k = data.get("workloads", {}).get(workload_name, {}).get("kernels", {}).get(kernel)
    if not k:
        return None
    return k["fetch_bytes"] + k["write_bytes"]


def cpu_baseline(wl, inp, tokens: int):
    """The CPU oracle, as it is, on the first `tokens` tokens (or rows)."""
    import numpy as np
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    S = min(tokens, wl.T)
    t0 = time.perf_counter()
    if wl.routing == "router":
        O.layer(inp["x"][:S], inp["Wr"], inp["Wg"], inp["Wu"], inp["Wd"], wl.k, inp["dY"][:S],
                wl.prec, mx_wgrad=wl.mx_wgrad)
    else:
        O.layer(inp["x"][:S], None, inp["Wg"], inp["Wu"], inp["Wd"], wl.k, inp["dY"][:S], wl.prec,
                topk_idx=inp["topk_idx"][:S], topk_w=inp["topk_w"][:S])
    dt = time.perf_counter() - t0
    return {"value": S / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"forward+backward of the first {S} of {wl.T} tokens with the full "
                      f"expert weights (numpy float64 oracle with {wl.prec} storage rounding)"}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="olmoe_bf16")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-tokens", type=int, default=2048,
                    help="tokens of the CPU-oracle sample (0 = skip the CPU baseline)")
    ap.add_argument("--kernels", action="store_true", help="per-kernel table on stderr")
    ap.add_argument("--no-companions", action="store_true",
                    help="skip the companion runs of the default workload (expert-count scan "
                         "ends and MXFP8, timed in the same run for the ratio keys)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (the "
                         "known-size reference for HBM byte counters) and exit")
    ap.add_argument("--mfma-summary", metavar="PMC_DIR",
                    help="only summarise a rocprofv3 --pmc run of SQ_VALU_MFMA_BUSY_CYCLES, "
                         "SQ_BUSY_CU_CYCLES and GRBM_GUI_ACTIVE (this workload, with the clock "
                         "probe) as a markdown table on stdout and exit")
    ap.add_argument("--sq-summary", nargs=2, metavar=("PASS1_DIR", "PASS2_DIR"),
                    help="only summarise the two rocprofv3 --pmc passes of SQ_PASSES (GEMM wave "
                         "stalls, queue-full and LDS counters) as markdown on stdout and exit")
    ap.add_argument("--profile-md", metavar="KT_DIR",
                    help="only print the markdown profile summary of this workload from a "
                         "rocprofv3 --kernel-trace --stats directory (and the committed traffic "
                         "counters) and exit")
    ap.add_argument("--traffic", nargs=4, metavar=("FETCH", "WRITE", "CAL_FETCH", "CAL_WRITE"),
                    help="only summarise four rocprofv3 --pmc output directories (FETCH_SIZE and "
                         "WRITE_SIZE of this workload, then of --calibrate-copy 1024) into "
                         + TRAFFIC_JSON + " and exit")
    args = ap.parse_args(argv)

    if args.traffic:
        return write_traffic(args.workload, *args.traffic)
    if args.mfma_summary:
        return mfma_summary(args.workload, args.mfma_summary)
    if args.profile_md:
        return profile_markdown(args.workload, args.profile_md)
    if args.sq_summary:
        return sq_summary(args.workload, args.sq_summary)

    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 3}))
        return 0

    if args.gpus != 1:
        print(f"bench.py: this layer runs on one GPU; --gpus {args.gpus} is not supported "
              "(expert-parallel exchange across GPUs is not built)", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import routing_grouped_gemm_amd as rgg
    from moe_synth import workload, make_inputs

    wl = workload(args.workload)
    inp = make_inputs(wl, seed=args.seed)
    dt = torch.float32 if wl.dtype == "fp32" else torch.bfloat16

    def dev(name):
        if dt == torch.bfloat16:
            return rgg.upload(inp[name + "_bits"], torch.bfloat16)
        return rgg.upload(inp[name])

    if wl.passes == "fwd":
        return bench_forward(args, wl, inp, dev)

    router = wl.routing == "router"
    x, dY = dev("x"), dev("dY")
    Wg, Wu, Wd = dev("Wg"), dev("Wu"), dev("Wd")
    Wr = dev("Wr") if router else None
    kw = {}
    if not router:
        kw = dict(topk_idx=rgg.upload(inp["topk_idx"]), topk_w=rgg.upload(inp["topk_w"]))
    layer = rgg.ExpertLayer(wl.T, wl.d, wl.E, wl.f, wl.k, dt, wl.prec, router=router,
                            mx_wgrad=wl.mx_wgrad)

    def step():
        layer.forward(x, Wr, Wg, Wu, Wd, **kw)
        layer.backward(dY)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Kernel table (untimed): an event after every kernel of a few steps
    # gives each kernel's share of a step, and names the dominant kernel.
    P = max(1, min(args.steps, 10))
    full = rgg.KernelTimer(capacity=P * 64)
    with full:
        for _ in range(P):
            step()
    kern = full.durations()
    if len(kern) >= full.capacity:
        raise RuntimeError("bench: the kernel table filled its event capacity (launches lost)")
    per = {}
    for name, dur in kern:
        c = per.setdefault(name, [0, 0.0])
        c[0] += 1
        c[1] += dur
    table = sorted(((n, c[0] / P, c[1] / P, c[1] / c[0]) for n, c in per.items()),
                   key=lambda r: -r[2])
    # expert FFN time: the expert GEMMs, and for MXFP8 also the quantizers
    gemm_ms = sum(r[2] for r in table if (r[0].startswith("gemm_") and "router" not in r[0])
                  or r[0].startswith("mx_"))
    # the kernel priced against its roofline: the expert GEMM with the most
    # time per step (the layer's cost is the GEMMs'); else the top kernel
    gemms = [r for r in table if r[0].startswith("gemm_") and "router" not in r[0]]
    dom_name = (gemms or table)[0][0]

    # Timed region: K steps; events only right before and after each launch
    # of the dominant kernel, so that the other kernels run back to back.
    K = args.steps
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    per_step = next(r[1] for r in table if r[0] == dom_name)
    timer = rgg.KernelTimer(capacity=int(K * (2 * per_step + 2)) + 16, only=dom_name)
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    w0 = time.perf_counter()
    with timer:
        t_start.record()
        for i in range(K):
            marks[i].record()
            step()
        marks[K].record()
        t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = t_start.elapsed_time(t_end) / K
    step_ms = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(K)])
    dom_runs = [dur for _, dur in timer.durations()]
    if not dom_runs or 2 * len(dom_runs) + 2 > timer.capacity:
        raise RuntimeError(f"bench: {len(dom_runs)} launches of {dom_name} timed "
                           f"(none, or the event capacity filled)")
    dom_launch_ms = float(np.mean(dom_runs))
    dom_flops = gemm_flops(dom_name, wl)
    peak = PEAK_TFLOPS[wl.prec]
    # a kernel is priced at the peak of its own operand type: the scaled fp8
    # GEMMs at the fp8 peak, the rest (bf16 weight gradients, router) at bf16
    dom_peak = PEAK_TFLOPS["mxfp8" if dom_name.startswith("gemm_mx_") else wl.dtype]
    if dom_flops > 0:
        ach = dom_flops / (dom_launch_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": dom_name, "achieved": round(ach, 2), "peak": dom_peak,
                "unit": "TFLOP/s", "frac": round(ach / dom_peak, 4),
                "traffic": measured_traffic(wl.name, dom_name),
                "per_launch_ms": round(dom_launch_ms, 4), "timed_launches": len(dom_runs),
                "algorithmic_flops_per_launch": dom_flops}
    else:
        roof = {"bound": "hbm", "kernel": dom_name, "achieved": None, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": None, "traffic": measured_traffic(wl.name, dom_name)}

    flops = wl.flops()
    tok_s = wl.T / (ms * 1e-3)
    tflops = flops / (ms * 1e-3) / 1e12
    ffn_tflops = wl.expert_flops() / (gemm_ms * 1e-3) / 1e12 if gemm_ms > 0 else None

    cpu = None
    if args.cpu_tokens > 0:
        cpu = cpu_baseline(wl, inp, args.cpu_tokens)

    # clock under MFMA load and the sustained dense MFMA rate, right after the
    # timed steps (a pure-MFMA probe on every CU)
    clk = rgg.probe_clock()

    companions = None
    if wl.name == "olmoe_bf16" and not args.no_companions:
        del layer, x, dY, Wg, Wu, Wd, Wr, kw, inp
        torch.cuda.empty_cache()
        companions = {n: time_workload(n, args.seed) for n in COMPANIONS}

    if args.kernels:
        print(f"{'kernel':32s} {'launches/step':>13s} {'ms/step':>9s} {'ms/launch':>10s}",
              file=sys.stderr)
        for n, c, tot, one in table:
            print(f"{n:32s} {c:13.0f} {tot:9.4f} {one:10.4f}", file=sys.stderr)

    out = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.prec,
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02^2) weights)",
        "config": {"workload": wl.name, "T": wl.T, "d_model": wl.d, "experts": wl.E,
                   "d_ff": wl.f, "top_k": wl.k, "routed_rows": wl.R, "routing": wl.routing,
                   "mx_weight_gradients": wl.mx_wgrad, "parallelism": "single GPU"},
        "tflops": round(tflops, 2),
        "pct_peak": round(100.0 * tflops / peak, 2),
        "ffn_gemm_tflops": None if ffn_tflops is None else round(ffn_tflops, 2),
        "ffn_gemm_pct_peak": None if ffn_tflops is None else round(100.0 * ffn_tflops / peak, 2),
        "wall_ms_per_step": round(wall * 1e3 / K, 4),
        "step_ms": {"median": round(float(np.median(step_ms)), 4),
                    "p10": round(float(np.percentile(step_ms, 10)), 4),
                    "p90": round(float(np.percentile(step_ms, 90)), 4)},
        "kernels_ms_per_step": {n: round(tot, 4) for n, _, tot, _ in table},
        "roofline": roof,
        "cpu_baseline": cpu,
        "clock": {"mhz_under_mfma_load": round(clk["clock_mhz"], 1),
                  "mhz_over_event_time": round(clk["event_clock_mhz"], 1),
                  "realtime_counter_mhz_over_event_time": round(clk["realtime_mhz"], 2),
                  "probe_mfma_tflops": round(clk["mfma_tflops"], 1),
                  "bf16_peak_at_measured_clock_tflops":
                      round(PEAK_TFLOPS["bf16"] * clk["clock_mhz"] / 2400.0, 1)},
    }
    if ffn_tflops is not None:
        out["ffn_gemm_pct_of_peak_at_measured_clock"] = round(
            100.0 * ffn_tflops / (peak * clk["clock_mhz"] / 2400.0), 2)
    if companions:
        out["companions"] = companions
        e8, e128 = companions["escan_e8_bf16"], companions["escan_e128_bf16"]
        out["expert_scan_tokens_ratio_e128_over_e8"] = round(e128["tokens_per_s"] /
                                                             e8["tokens_per_s"], 4)
        out["expert_scan_tokens_per_s"] = {
            str(companions[n]["config"]["experts"]): companions[n]["tokens_per_s"]
            for n in ("escan_e8_bf16", "escan_e32_bf16", "escan_e128_bf16")}
        out["mxfp8_speedup_over_bf16"] = round(companions["olmoe_bf16"]["ms_per_step"] /
                                               companions["olmoe_mxfp8"]["ms_per_step"], 4)
    print(json.dumps(out), flush=True)
    return 0


# Workloads timed beside the default one (same run, same box): both ends of
# the expert-count scan (16384 tokens, d 4096, f 1536, top-4; 8 and 128
# experts) and the OLMoE-shaped layer with MXFP8 expert GEMMs.
# the MXFP8 layer is compared with the bf16 layer timed the same way right
# before it (same step count, no per-kernel events in either)
COMPANIONS = ("escan_e8_bf16", "escan_e32_bf16", "escan_e128_bf16", "olmoe_bf16", "olmoe_mxfp8",
              "share1t_bf16")


def time_workload(name: str, seed: int, steps: int = 20, warmup: int = 5):
    """ms per forward+backward step of a workload (events around the steps,
    nothing else timed), with its inputs resident on the GPU."""
    import numpy as np
    import torch
    import routing_grouped_gemm_amd as rgg
    from moe_synth import workload, make_inputs
    wl = workload(name)
    inp = make_inputs(wl, seed=seed)
    up = lambda n: rgg.upload(inp[n + "_bits"], torch.bfloat16)
    router = wl.routing == "router"
    x, dY, Wg, Wu, Wd = up("x"), up("dY"), up("Wg"), up("Wu"), up("Wd")
    Wr = up("Wr") if router else None
    kw = {} if router else dict(topk_idx=rgg.upload(inp["topk_idx"]),
                                topk_w=rgg.upload(inp["topk_w"]))
    del inp
    layer = rgg.ExpertLayer(wl.T, wl.d, wl.E, wl.f, wl.k, torch.bfloat16, wl.prec, router=router,
                            mx_wgrad=wl.mx_wgrad)

    def step():
        layer.forward(x, Wr, Wg, Wu, Wd, **kw)
        layer.backward(dY)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    for i in range(steps):
        marks[i].record()
        step()
    marks[steps].record()
    torch.cuda.synchronize()
    per = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(steps)])
    ms = float(marks[0].elapsed_time(marks[steps])) / steps
    out = {"ms_per_step": round(ms, 4), "tokens_per_s": round(wl.T / (ms * 1e-3), 1),
           "tflops": round(wl.flops() / (ms * 1e-3) / 1e12, 2), "steps": steps,
           "warmup": warmup, "step_ms_median": round(float(np.median(per)), 4),
           "config": {"T": wl.T, "d_model": wl.d, "experts": wl.E, "d_ff": wl.f, "top_k": wl.k,
                      "precision": wl.prec}}
    del layer, x, dY, Wg, Wu, Wd, Wr, kw
    torch.cuda.empty_cache()
    return out


def fwd_gemm_bytes(name: str, wl, active: int) -> float:
    """Algorithmic HBM bytes of one forward expert GEMM launch on a small
    batch: the weights of the experts that received rows, read once, plus
    the activations read and written once (bf16)."""
    R, d, f = wl.R, wl.d, wl.f
    if name in ("gemm_fwd_gateup_swiglu", "skinny_fwd_gateup"):
        return 2.0 * (active * 2 * d * f + R * d + 3 * R * f)
    if name in ("gemm_fwd_down", "skinny_fwd_down"):
        return 2.0 * (active * f * d + R * f + R * d)
    return 0.0


def bench_forward(args, wl, inp, dev) -> int:
    """Inference-shaped workload: latency of one layer forward on a small
    batch (route -> dispatch -> grouped FFN forward -> combine), launched
    eagerly and replayed from a HIP graph captured once."""
    import numpy as np
    import torch
    import routing_grouped_gemm_amd as rgg

    x = dev("x")
    Wg, Wu, Wd, Wr = dev("Wg"), dev("Wu"), dev("Wd"), dev("Wr")
    dt = torch.float32 if wl.dtype == "fp32" else torch.bfloat16
    layer = rgg.ExpertLayer(wl.T, wl.d, wl.E, wl.f, wl.k, dt, wl.prec, router=True)
    K = args.steps

    def fwd():
        layer.forward(x, Wr, Wg, Wu, Wd)

    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    y_eager = layer.y.clone()
    active = int((layer.counts > 0).sum().item())

    # eager launches, with per-kernel events
    timer = rgg.KernelTimer(capacity=K * 16)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    with timer:
        for i in range(K):
            marks[i].record()
            fwd()
        marks[K].record()
    torch.cuda.synchronize()
    eager_ms = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(K)])
    kern = timer.durations()
    if len(kern) >= timer.capacity:
        raise RuntimeError("bench: the kernel table filled its event capacity (launches lost)")

    # one capture, K replays
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fwd()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(layer.y, y_eager))
    gmarks = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    w0 = time.perf_counter()
    for i in range(K):
        gmarks[i].record()
        graph.replay()
    gmarks[K].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    graph_ms = np.array([gmarks[i].elapsed_time(gmarks[i + 1]) for i in range(K)])

    per = {}
    for name, dur in kern:
        c = per.setdefault(name, [0, 0.0])
        c[0] += 1
        c[1] += dur
    table = sorted(((n, c[0] / K, c[1] / K, c[1] / c[0]) for n, c in per.items()),
                   key=lambda r: -r[2])
    dom_name = table[0][0]
    # the dominant kernel alone, bracketed by events, over K eager forwards
    only = rgg.KernelTimer(capacity=K * 8, only=dom_name)
    with only:
        for i in range(K):
            fwd()
    dom_runs = [dur for _, dur in only.durations()]
    if not dom_runs or 2 * len(dom_runs) + 2 > only.capacity:
        raise RuntimeError(f"bench: {len(dom_runs)} launches of {dom_name} timed "
                           f"(none, or the event capacity filled)")
    dom_launch_ms = float(np.mean(dom_runs))
    nbytes = fwd_gemm_bytes(dom_name, wl, active)
    if nbytes > 0:
        ach = nbytes / (dom_launch_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": dom_name, "achieved": round(ach, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(wl.name, dom_name),
                "per_launch_ms": round(dom_launch_ms, 4), "timed_launches": len(dom_runs),
                "algorithmic_bytes_per_launch": nbytes}
    else:
        roof = {"bound": "hbm", "kernel": dom_name, "achieved": None, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": None, "traffic": None}

    cpu = None
    if args.cpu_tokens > 0:
        from oracle import moe_oracle as O
        cores = len(os.sched_getaffinity(0))
        t0 = time.perf_counter()
        O.layer(inp["x"], inp["Wr"], inp["Wg"], inp["Wu"], inp["Wd"], wl.k, None, wl.prec)
        sec = time.perf_counter() - t0
        cpu = {"value": round(sec * 1e6, 1), "unit": "us", "cores": int(cores), "kind": "oracle",
               "sample": f"forward of all {wl.T} token(s) (numpy float64 oracle with "
                         f"{wl.prec} storage rounding)"}

    if args.kernels:
        for n, c, tot, one in table:
            print(f"{n:32s} {c:13.0f} {tot:9.4f} {one:10.4f}", file=sys.stderr)

    lat_us = float(np.median(graph_ms)) * 1e3
    out = {
        "metric": "MoE layer forward latency on a small batch (HIP graph replay)",
        "value": round(lat_us, 2),
        "unit": "us",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(lat_us / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.prec,
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02^2) weights)",
        "config": {"workload": wl.name, "T": wl.T, "d_model": wl.d, "experts": wl.E,
                   "d_ff": wl.f, "top_k": wl.k, "routed_rows": wl.R, "passes": "forward",
                   "active_experts": active, "parallelism": "single GPU"},
        "tokens_per_s": round(wl.T / (lat_us * 1e-6), 1),
        "graph_us": {"median": round(lat_us, 2),
                     "p10": round(float(np.percentile(graph_ms, 10)) * 1e3, 2),
                     "p90": round(float(np.percentile(graph_ms, 90)) * 1e3, 2)},
        "eager_us": {"median": round(float(np.median(eager_ms)) * 1e3, 2),
                     "p10": round(float(np.percentile(eager_ms, 10)) * 1e3, 2),
                     "p90": round(float(np.percentile(eager_ms, 90)) * 1e3, 2)},
        "graph_output_equals_eager": same,
        "wall_us_per_replay": round(wall * 1e6 / K, 2),
        "kernels_us_per_forward": {n: round(tot * 1e3, 2) for n, _, tot, _ in table},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
