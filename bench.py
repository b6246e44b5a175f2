"""Benchmark: fine-grained FP8 e4m3 GEMM throughput on one MI355X.

One step = one pass of the hot path over the dense NT sweep workload: the 15
shapes M in {64, 128, 4096} x (N, K) in {(2112, 7168), (24576, 1536),
(7168, 16384), (4096, 7168), (7168, 2048)}, bf16 out, inputs N(0,1) quantised
with 1x128 (A) and 128x128 (B) fp32 scales, all resident in HBM before the
timed region.  value = total algorithmic FLOP of a step (sum of 2*M*N*K) over
the measured time, in TFLOP/s.

Also reported on the same JSON line:
  roofline     -- the dominant launch of the step (largest share of time),
                  timed live with HIP events on the launch stream, against the
                  MFMA (fp8 dense 5.0 PFLOP/s) or HBM (8 TB/s) roof, whichever
                  bounds its arithmetic intensity;
  cpu_baseline -- the fp64 CPU oracle on a bounded sample of that shape's rows;
  detail       -- per-shape times, the three grouped MoE workloads
                  (contiguous, masked, K-grouped) timed the same way, the
                  FP8 casting kernels on bf16 operands of those shapes, and
                  the power-of-two (packed UE8M0) scale variant of the dense
                  sweep and the contiguous and masked workloads, and the NN /
                  TN / TT layouts and the M-grouped contiguous NN form, and the
                  FP8 MQA logits kernel on a 64-head causal prefill.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-detail]
                       [--no-cpu] [--json-out PATH]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0     # MI355X dense FP8 MFMA (published)
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E (published)
MACHINE_BALANCE = PEAK_FP8_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)   # FLOP per byte

# The rocprofv3 runs behind the profiles/ summaries (repository root, one GPU).
GROUPED_PROFILE_COMMANDS = [
    "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_grouped -o run -- "
    "python3 bench.py --steps 3 --warmup 1 --no-cpu --json-out gpurun_out/bench_grouped.json",
    "python3 bench.py --summarize-grouped gpurun_out/prof_grouped gpurun_out/bench_grouped.json "
    "profiles/grouped_moe__contiguous_masked_kgrouped.md",
]

PROFILE_COMMANDS = [
    "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_trace -o run -- "
    "python3 bench.py --no-detail --no-cpu --json-out gpurun_out/bench_prof.json",
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/prof_fetch -o run -- "
    "python3 bench.py --steps 1 --warmup 0 --no-detail --no-cpu --copy-calibration",
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/prof_write -o run -- "
    "python3 bench.py --steps 1 --warmup 0 --no-detail --no-cpu --copy-calibration",
    "python3 bench.py --summarize-profiles gpurun_out/prof_trace gpurun_out/prof_fetch "
    "gpurun_out/prof_write gpurun_out/bench_prof.json profiles/<kernel>__dense_sweep.md",
]


def dense_bytes(M, N, K, d_bytes=2):
    return M * K + N * K + 4 * (K // 128) * M + 4 * ((N + 127) // 128) * (K // 128) + d_bytes * M * N


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 100 timed sweeps after 300 untimed ones by default (about 0.45 s of GPU
    # time): the GPU leaves its idle power state and its clocks settle only
    # under sustained load, and on some machines that takes longer than a few
    # tens of sweeps (one machine, alternating runs: 30 warmup + 20 timed steps
    # 1591-1608 TFLOP/s, 300 + 100 steps 1722-1723)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--no-detail", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 1 GiB device copy before the GEMMs (a kernel of known "
                         "traffic, to scale hardware byte counters)")
    ap.add_argument("--summarize-profiles", nargs=5, metavar=("TRACE_DIR", "FETCH_DIR",
                                                              "WRITE_DIR", "BENCH_JSON", "OUT_MD"),
                    help="write a profiles/ summary from rocprofv3 CSV output and exit")
    ap.add_argument("--summarize-cast", nargs=3, metavar=("TRACE_DIR", "BENCH_JSON", "OUT_MD"),
                    help="write the profiles/ summary of the casting kernels")
    ap.add_argument("--summarize-grouped", nargs=3, metavar=("TRACE_DIR", "BENCH_JSON", "OUT_MD"),
                    help="write the profiles/ summary of the grouped-workload kernel trace and exit")
    args = ap.parse_args()

    if args.summarize_profiles:
        summarize_profiles(*args.summarize_profiles, commands=PROFILE_COMMANDS)
        return
    if args.summarize_cast:
        summarize_cast(*args.summarize_cast)
        return
    if args.summarize_grouped:
        summarize_grouped(*args.summarize_grouped)
        return

    if args.gpus != 1:
        print(f"bench.py: one GPU only; --gpus {args.gpus} is not supported (the kernels run on "
              "one GPU's shard; the multi-GPU exchange is not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch
    import fp8_fine_grained_e4m3_amd as dg
    from tests import gen

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    dg.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    # ---- inputs (host generation, then resident in HBM) ---------------------------
    t0 = time.time()
    shapes = list(gen.DENSE_SWEEP)
    ops = []
    for (M, N, K) in shapes:
        x = gen.gen_dense(M, N, K, seed=0)
        a, sa, b, sb = up(x.a), up(x.sfa), up(x.b), up(x.sfb)
        d = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        ops.append(dict(shape=(M, N, K), args=((a, sa), (b, sb), d), flop=2.0 * M * N * K,
                        bytes=dense_bytes(M, N, K),
                        kernel=dg.kernel_config_name(dg.FORM_DENSE, M, N, K)))
        del x
    gen_s = time.time() - t0
    print(f"[bench] generated dense sweep in {gen_s:.1f}s", file=sys.stderr, flush=True)

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(events=None, only=None):
        for i, op in enumerate(ops):
            rec = events is not None and (only is None or op["kernel"] == only)
            if rec:
                events[i][0].record(stream)
            dg.fp8_gemm_nt(*op["args"])
            if rec:
                events[i][1].record(stream)

    def new_events(n):
        return [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in ops] for _ in range(n)]

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- per-launch pass (untimed): an event pair around every launch ------------
    # gives the per-shape detail and picks the dominant kernel: the kernel
    # instance (tile configuration) with the largest share of the step's time.
    # Several shapes may share one instance.
    probe_steps = 3
    ev = new_events(probe_steps)
    for s_ in range(probe_steps):
        step(ev[s_])
    torch.cuda.synchronize()
    # median over the sweeps: the first launches after the warmup's synchronize
    # can run on clocks that have not yet come back up
    avg_ms = np.median([[ev[s_][i][0].elapsed_time(ev[s_][i][1]) for i in range(len(ops))]
                        for s_ in range(probe_steps)], axis=0)
    groups = {}
    for i, op in enumerate(ops):
        groups.setdefault(op["kernel"], []).append(i)
    dom_name = max(groups, key=lambda k: sum(avg_ms[i] for i in groups[k]))
    idx = groups[dom_name]

    # ---- timed region: exactly K steps ---------------------------------------------
    # Event pairs only around the dominant instance's launches (an event pair
    # around every launch adds several microseconds per launch to the step).
    ev = new_events(args.steps)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s_ in range(args.steps):
        step(ev[s_], only=dom_name)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    dom_ms = np.array([[ev[s_][i][0].elapsed_time(ev[s_][i][1]) for i in idx]
                       for s_ in range(args.steps)])
    flop_step = sum(op["flop"] for op in ops)
    value = flop_step * args.steps / elapsed / 1e12
    ms_per_step = elapsed * 1e3 / args.steps

    # Per-launch figures of the dominant instance: averages over its launches
    # in the timed region -- the same average a kernel-trace profile reports
    # for that kernel name.
    launch_ms = float(dom_ms.mean())
    launch_flop = float(np.mean([ops[i]["flop"] for i in idx]))
    launch_bytes = float(np.mean([ops[i]["bytes"] for i in idx]))
    intensity = launch_flop / launch_bytes
    if intensity >= MACHINE_BALANCE:
        achieved = launch_flop / (launch_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=PEAK_FP8_TFLOPS,
                    unit="TFLOP/s", frac=round(achieved / PEAK_FP8_TFLOPS, 4), traffic=None)
    else:
        achieved = launch_bytes / (launch_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(achieved / PEAK_HBM_GBS, 4), traffic=None)
    roof["traffic"] = measured_traffic(dom_name)
    roof["kernel"] = dom_name
    roof["launches_per_step"] = len(idx)
    roof["shapes"] = ["x".join(map(str, ops[i]["shape"])) for i in idx]
    roof["avg_launch_us"] = round(launch_ms * 1e3, 2)
    roof["alg_flop_per_launch"] = launch_flop
    roof["alg_bytes_per_launch"] = launch_bytes
    M, N, K = ops[max(idx, key=lambda i: avg_ms[i])]["shape"]

    per_shape = []   # from the per-launch pass
    for op, t in zip(ops, avg_ms):
        m, n, k = op["shape"]
        per_shape.append(dict(M=m, N=n, K=k, kernel=op["kernel"], us=round(t * 1e3, 2),
                              tflops=round(op["flop"] / (t * 1e-3) / 1e12, 1),
                              gbs=round(op["bytes"] / (t * 1e-3) / 1e9, 1)))
    print(f"[bench] step {ms_per_step:.3f} ms, {value:.1f} TFLOP/s", file=sys.stderr, flush=True)

    # ---- grouped workloads (detail, timed the same way) ------------------------------
    grouped, cast, ue8m0, layouts, mqa = {}, {}, {}, {}, {}
    if not args.no_detail:
        del ops
        torch.cuda.empty_cache()
        grouped = bench_grouped(dg, gen, up, dev, stream, args)
        cast = bench_cast(dg, dev, stream, args)
        ue8m0 = bench_ue8m0(dg, gen, up, dev, stream, args)
        layouts = bench_layouts(dg, gen, up, dev, stream, args)
        mqa = bench_mqa(dg, gen, up, dev, stream, args)

    # ---- CPU baseline: the oracle on a bounded sample ----------------------------------
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(gen, (M, N, K), args.cpu_seconds)

    result = {
        "metric": "FP8 GEMM TFLOPS + % of MI355X FP8 MFMA peak (dense NT, grouped MoE)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": "dense FP8 NT GEMM sweep: 15 shapes, M in {64,128,4096} x "
                               "(N,K) in {(2112,7168),(24576,1536),(7168,16384),(4096,7168),"
                               "(7168,2048)}, bf16 out, 1x128 / 128x128 fp32 scales, seed 0",
                   "frac_of_fp8_peak": round(value / PEAK_FP8_TFLOPS, 4)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "detail": {"dense": per_shape, "grouped": grouped, "cast": cast, "ue8m0": ue8m0,
                   "layouts": layouts, "mqa_logits": mqa},
    }
    line = json.dumps(result)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


# ------------------------------------------------------------------------------
# rocprofv3 summaries (profiles/) and the measured-traffic lookup
# ------------------------------------------------------------------------------

KERNEL_SOURCES = {
    "nt": ["fp8_fine_grained_e4m3_amd/csrc/nt_kernel.hip",
           "fp8_fine_grained_e4m3_amd/csrc/tile_common.h",
           "fp8_fine_grained_e4m3_amd/csrc/dg_internal.h"],
    "tn": ["fp8_fine_grained_e4m3_amd/csrc/tn_kernel.hip",
           "fp8_fine_grained_e4m3_amd/csrc/tile_common.h",
           "fp8_fine_grained_e4m3_amd/csrc/dg_internal.h"],
    "cast": ["fp8_fine_grained_e4m3_amd/csrc/cast_kernel.hip",
             "fp8_fine_grained_e4m3_amd/csrc/dg_internal.h"],
}


def source_hash(family: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(config_name: str):
    """HBM-side bytes per launch recorded in profiles/ for this kernel instance,
    or None when there is no record or the kernel sources changed since."""
    import glob
    import re
    fam = config_name.split("_")[0]
    for path in glob.glob(os.path.join(ROOT, "profiles", f"{config_name}__*.md")):
        text = open(path).read()
        m = re.search(r"traffic_bytes_per_launch:\s*([0-9.]+)", text)
        h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
        if m and h and fam in KERNEL_SOURCES and h.group(1) == source_hash(fam):
            return float(m.group(1))
    return None


def instance_matcher(name):
    """Predicate on demangled kernel names selecting the template instance
    behind a config name such as nt_dense_bf16_256x256 or
    tn_kgrouped_f32_256x256; also returns a readable tag."""
    parts = name.split("_")
    kind, form, out, tile = parts[0], parts[1], parts[2], parts[-1]
    ue8m0 = "ue8m0" in parts
    bm, bn = tile.split("x")
    if kind == "tn":
        tag = f"TnCfg<{bm}, {bn},"
        return (lambda k: "tn_fp8_kernel" in k and tag in k), tag + " ...>"
    form_id = {"dense": 0, "contiguous": 1, "masked": 2}[form]
    tail = (f", {form_id}, {'true' if out == 'f32' else 'false'}, "
            f"{'true' if ue8m0 else 'false'}>")
    tag = f"NtCfg<{bm}, {bn},"
    return (lambda k: "nt_fp8_kernel" in k and tag in k and tail in k), tag + " ...>" + tail


def summarize_profiles(trace_dir, fetch_dir, write_dir, bench_json, out_path, commands):
    """Write the profiles/ summary of one kernel instance from rocprofv3 CSVs."""
    import csv
    res = json.load(open(bench_json))
    roof = res["roofline"]
    name = roof["kernel"]
    stats = list(csv.DictReader(open(os.path.join(trace_dir, "run_kernel_stats.csv"))))

    def counters(d, counter):
        rows = list(csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))))
        return [(r["Kernel_Name"], float(r["Counter_Value"]), int(r["Grid_Size"])) for r in rows
                if r["Counter_Name"] == counter]

    fetch = counters(fetch_dir, "FETCH_SIZE")
    write = counters(write_dir, "WRITE_SIZE")
    copy_bytes = float(1 << 30)
    fetch_copy = max(v for k, v, g in fetch if "copyBuffer" in k) * 1024.0
    write_copy = max(v for k, v, g in write if "copyBuffer" in k) * 1024.0
    f_scale, w_scale = copy_bytes / fetch_copy, copy_bytes / write_copy
    match, tag = instance_matcher(name)
    f_k = [v for k, v, g in fetch if match(k)]
    w_k = [v for k, v, g in write if match(k)]
    fetch_b = float(np.mean(f_k)) * 1024.0 * f_scale
    write_b = float(np.mean(w_k)) * 1024.0 * w_scale
    lines = [f"# {name} -- dense FP8 NT sweep (M=4096 shapes), rocprofv3", "",
             "Commands (run from the repository root on one MI355X):", ""]
    lines += [f"    {c}" for c in commands]
    lines += ["", "## Kernel trace (--kernel-trace --stats)", "",
              "| kernel | calls | avg us | total ms | % |", "|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| `{r['Name'][:80]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.1f} |")
    avg_us = [float(r["AverageNs"]) / 1e3 for r in stats if match(r["Name"])][0]
    lines += ["", f"Dominant instance `{tag}` = `{name}`: rocprofv3 average {avg_us:.2f} us per "
              f"launch; bench.py's HIP-event average over its timed region {roof['avg_launch_us']} us.",
              f"Launches of this instance per step: {roof['launches_per_step']} "
              f"({', '.join(roof['shapes'])}).",
              f"Algorithmic work per launch (mean over those shapes): "
              f"{roof['alg_flop_per_launch'] / 1e9:.2f} GFLOP, {roof['alg_bytes_per_launch'] / 1e6:.2f} MB.",
              "", "## Traffic (--pmc FETCH_SIZE, then --pmc WRITE_SIZE)", "",
              f"Calibration: a 1 GiB device copy (`__amd_rocclr_copyBuffer`) reads FETCH_SIZE "
              f"{fetch_copy / 1024:.0f} KiB and WRITE_SIZE {write_copy / 1024:.0f} KiB, so the "
              f"scale factors are {f_scale:.4f} (fetch) and {w_scale:.4f} (write).",
              "", "| dispatch of this instance | FETCH_SIZE KiB | WRITE_SIZE KiB |", "|---|---|---|"]
    for i, (fv, wv) in enumerate(zip(f_k, w_k)):
        lines.append(f"| {i} | {fv:.1f} | {wv:.1f} |")
    lines += ["", f"Scaled per launch: fetch {fetch_b / 1e6:.1f} MB + write {write_b / 1e6:.1f} MB "
              f"= {(fetch_b + write_b) / 1e6:.1f} MB, {(fetch_b + write_b) / roof['alg_bytes_per_launch']:.2f}x "
              f"the algorithmic bytes.",
              "", "Machine-readable:", "",
              f"    traffic_bytes_per_launch: {fetch_b + write_b:.0f}",
              f"    kernel_source_sha256_16: {source_hash(name.split('_')[0])}",
              f"    bench_value_tflops: {res['value']}", ""]
    with open(out_path, "w") as f:
        f.write("\n".join(lines))
    print(out_path)


DETAIL_SUMMARIES = {
    # file -> (title, kernel-name filter, bench detail key, template-argument note)
    "grouped_moe__contiguous_masked_kgrouped.md": (
        "Grouped MoE workloads (contiguous, masked, K-grouped), fp32 scales",
        lambda k: ("nt_fp8_kernel" in k and (", 1, false, false>" in k or ", 2, false, false>" in k))
        or ("tn_fp8_kernel" in k and "false, false, true, false, false>" in k),
        "grouped",
        "`nt_fp8_kernel<Cfg, FORM, OUT_F32, UE8M0>`: FORM 1 = contiguous, 2 = masked. "
        "`tn_fp8_kernel<Cfg, A_MK, B_NK, OUT_F32, GROUPED_M, UE8M0>` with "
        "`false, false, true, false, false` = the K-grouped form."),
    "ue8m0__dense_sweep_contiguous_masked_kgrouped.md": (
        "Packed UE8M0 scales (block-scaled MFMA): dense sweep, contiguous, masked, K-grouped",
        lambda k: ("nt_fp8_kernel" in k and "true>(dg::NtArgs" in k)
        or ("tn_fp8_kernel" in k and "false, false, true, false, true>" in k)
        or "pack_ue8m0" in k,
        "ue8m0",
        "Last template argument `true` = UE8M0 instance."),
    "mn_major_layouts__nn_tn_tt_4096x4096x7168_and_nn_contiguous.md": (
        "NN / TN / TT layouts and the M-grouped contiguous NN form (MN-major kernel)",
        lambda k: "tn_fp8_kernel" in k and not ("false, false, true, false" in k),
        "layouts",
        "`tn_fp8_kernel<Cfg, A_MK, B_NK, OUT_F32, GROUPED_M, UE8M0>`: A_MK = A stored [M, K], "
        "B_NK = B stored [N, K], GROUPED_M = contiguous NN."),
    "mqa_logits__causal_prefill_4096x4096_h64.md": (
        "FP8 MQA logits, 64 heads, causal 4096 x 4096 and 8 packed sequences of 512",
        lambda k: "mqa_logits_kernel" in k,
        "mqa_logits",
        "`mqa_logits_kernel<H>`, H = heads."),
}


def summarize_grouped(trace_dir, bench_json, out_path):
    """profiles/ summaries of the bench detail workloads: for each kernel
    family, the rocprofv3 per-kernel averages next to bench.py's own HIP-event
    timings of the same run.  out_path names the grouped-MoE file; the other
    families are written beside it."""
    import csv
    res = json.load(open(bench_json))
    stats = list(csv.DictReader(open(os.path.join(trace_dir, "run_kernel_stats.csv"))))
    out_dir = os.path.dirname(out_path) or "."
    for fname, (title, match, key, note) in DETAIL_SUMMARIES.items():
        detail = res["detail"].get(key, {})
        lines = [f"# {title} -- rocprofv3 kernel trace", "",
                 "Commands (run from the repository root on one MI355X):", ""]
        lines += [f"    {c}" for c in GROUPED_PROFILE_COMMANDS]
        lines += ["", "One bench.py run times the dense sweep and then every detail workload; the",
                  "rows below are this family's kernels from that run's trace.", "", note, "",
                  "## Kernel trace (--kernel-trace --stats)", "",
                  "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
        for r in stats:
            if match(r["Name"]):
                lines.append(f"| `{r['Name'][:110]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                             f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
        lines += ["", "## bench.py HIP-event timings (same run)", "",
                  "| workload | us | TFLOP/s | fraction of roof |", "|---|---|---|---|"]
        items = list(detail.items()) if isinstance(detail, dict) else []
        for name, v in items:
            if name == "dense" and isinstance(v, list):
                for dd in v:
                    lines.append(f"| dense {dd['M']}x{dd['N']}x{dd['K']} | {dd['us']} | {dd['tflops']} | |")
                continue
            if not isinstance(v, dict):
                lines.append(f"| {name} | {v} | | |")
                continue
            frac = v.get("frac_mfma", v.get("frac_hbm", ""))
            roof = "MFMA" if "frac_mfma" in v else ("HBM" if "frac_hbm" in v else "")
            lines.append(f"| {name} | {v.get('us')} | {v.get('tflops')} | {frac} {roof} |")
        lines += ["", f"    kernel_source_sha256_16: nt {source_hash('nt')}, tn {source_hash('tn')}, "
                      f"cast {source_hash('cast')}", ""]
        path = os.path.join(out_dir, fname)
        with open(path, "w") as f:
            f.write("\n".join(lines))
        print(path)


def bench_grouped(dg, gen, up, dev, stream, args):
    import torch
    out = {}
    reps = max(3, min(args.steps, 10))

    def timed(fn, n):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        fn()
        torch.cuda.synchronize()
        for e0, e1 in evs:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return float(np.median([e0.elapsed_time(e1) for e0, e1 in evs]))

    # contiguous (MoE forward)
    x = gen.gen_contiguous(seed=0)
    a, sa, b, sb, mi = up(x.a), up(x.sfa), up(x.b), up(x.sfb), up(x.m_indices)
    d = torch.empty(x.M_tot, x.N, dtype=torch.bfloat16, device=dev)
    ms = timed(lambda: dg.m_grouped_fp8_gemm_nt_contiguous((a, sa), (b, sb), d, mi), reps)
    valid = int(x.counts.sum())
    flop = 2.0 * valid * x.N * x.K
    byts = x.a.nbytes + x.sfa.nbytes + x.b.nbytes + x.sfb.nbytes + x.m_indices.nbytes + 2 * x.M_tot * x.N
    out["contiguous_32x4096x4096"] = dict(us=round(ms * 1e3, 1), tflops=round(flop / ms / 1e9, 1),
                                         frac_mfma=round(flop / ms / 1e9 / PEAK_FP8_TFLOPS, 4),
                                         gbs=round(byts / ms / 1e6, 1))
    del a, sa, b, sb, mi, d, x
    torch.cuda.empty_cache()

    # masked (MoE decode)
    x = gen.gen_masked(seed=0)
    a, sa, b, sb, mm = up(x.a), up(x.sfa), up(x.b), up(x.sfb), up(x.masked_m)
    d = torch.empty(x.G, x.M_max, x.N, dtype=torch.bfloat16, device=dev)
    ms = timed(lambda: dg.m_grouped_fp8_gemm_nt_masked((a, sa), (b, sb), d, mm), reps)
    valid = int(x.masked_m.sum())
    live = int((x.masked_m > 0).sum())
    flop = 2.0 * valid * x.N * x.K
    byts = (valid * x.K + valid * 4 * (x.K // 128) + live * x.N * x.K
            + live * 4 * ((x.N + 127) // 128) * (x.K // 128) + 2 * valid * x.N + 4 * x.G)
    out["masked_32x256x4096x2048"] = dict(us=round(ms * 1e3, 1), tflops=round(flop / ms / 1e9, 1),
                                         gbs=round(byts / ms / 1e6, 1),
                                         frac_hbm=round(byts / ms / 1e6 / PEAK_HBM_GBS, 4))
    del a, sa, b, sb, mm, d, x
    torch.cuda.empty_cache()

    # K-grouped TN (MoE weight gradient)
    x = gen.gen_k_grouped(seed=0)
    a, sa, b, sb, c = up(x.a), up(x.sfa), up(x.b), up(x.sfb), up(x.c)
    d = torch.empty(x.G, x.M, x.N, dtype=torch.float32, device=dev)
    ks = x.k_sizes
    ms = timed(lambda: dg.k_grouped_fp8_gemm_tn_contiguous((a, sa), (b, sb), d, ks, c=c), reps)
    flop = 2.0 * x.M * x.N * x.K_tot
    byts = x.a.nbytes + x.sfa.nbytes + x.b.nbytes + x.sfb.nbytes + 2 * 4 * x.G * x.M * x.N
    out["k_grouped_32x2048x4096"] = dict(us=round(ms * 1e3, 1), tflops=round(flop / ms / 1e9, 1),
                                        gbs=round(byts / ms / 1e6, 1),
                                        frac_hbm=round(byts / ms / 1e6 / PEAK_HBM_GBS, 4))
    del a, sa, b, sb, c, d, x
    torch.cuda.empty_cache()
    return out


def median_ms(stream, fn, n):
    """Median HIP-event time of n launches of fn on `stream` (after one warm-up)."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    fn()
    torch.cuda.synchronize()
    for e0, e1 in evs:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return float(np.median([e0.elapsed_time(e1) for e0, e1 in evs]))


def bench_ue8m0(dg, gen, up, dev, stream, args):
    """The same workloads with power-of-two scales packed as UE8M0 words (the
    MFMA applies the scales; no separate promotion): the dense sweep shape by
    shape, and the contiguous, masked and K-grouped MoE workloads."""
    import torch
    reps = max(3, min(args.steps, 10))
    # the dense sweep, timed like the fp32 sweep: whole-sweep steps without
    # events, and per-shape medians from sweeps with an event pair per launch
    ops = []
    for (M, N, K) in gen.DENSE_SWEEP:
        x = gen.gen_dense_ue8m0(M, N, K, seed=0)
        ops.append(((M, N, K), (up(x.a), up(x.sfa)), (up(x.b), up(x.sfb)),
                    torch.empty(M, N, dtype=torch.bfloat16, device=dev)))
        del x

    def sweep(evs=None):
        for i, (_, a, b, d) in enumerate(ops):
            if evs is not None:
                evs[i][0].record(stream)
            dg.fp8_gemm_nt(a, b, d)
            if evs is not None:
                evs[i][1].record(stream)

    for _ in range(3):
        sweep()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        sweep()
    torch.cuda.synchronize()
    step_ms = (time.perf_counter() - t0) * 1e3 / reps
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in ops] for _ in range(3)]
    for e in evs:
        sweep(e)
    torch.cuda.synchronize()
    per = np.median([[e[i][0].elapsed_time(e[i][1]) for i in range(len(ops))] for e in evs], axis=0)
    dense, f_sum = [], 0.0
    for ((M, N, K), _, _, _), ms in zip(ops, per):
        flop = 2.0 * M * N * K
        byts = M * K + N * K + 4 * ((K // 128 + 3) // 4) * (M + N) + 2 * M * N
        dense.append(dict(M=M, N=N, K=K, us=round(ms * 1e3, 2), tflops=round(flop / ms / 1e9, 1),
                          gbs=round(byts / ms / 1e6, 1)))
        f_sum += flop
    out = {"dense": dense, "dense_sweep_step_ms": round(step_ms, 4),
           "dense_sweep_tflops": round(f_sum / step_ms / 1e9, 1)}
    del ops
    torch.cuda.empty_cache()

    x = gen.gen_contiguous(seed=0, pow2=True)
    wa, wb = gen.to_ue8m0(x.sfa, x.sfb, x.N)
    a, sa, b, sb, mi = up(x.a), up(wa), up(x.b), up(wb), up(x.m_indices)
    d = torch.empty(x.M_tot, x.N, dtype=torch.bfloat16, device=dev)
    ms = median_ms(stream, lambda: dg.m_grouped_fp8_gemm_nt_contiguous((a, sa), (b, sb), d, mi),
                   reps)
    flop = 2.0 * int(x.counts.sum()) * x.N * x.K
    out["contiguous_32x4096x4096"] = dict(us=round(ms * 1e3, 1), tflops=round(flop / ms / 1e9, 1),
                                         frac_mfma=round(flop / ms / 1e9 / PEAK_FP8_TFLOPS, 4))
    del a, sa, b, sb, mi, d, x, wa, wb
    torch.cuda.empty_cache()

    x = gen.gen_masked(seed=0, pow2=True)
    wa, wb = gen.to_ue8m0(x.sfa, x.sfb, x.N)
    a, sa, b, sb, mm = up(x.a), up(wa), up(x.b), up(wb), up(x.masked_m)
    d = torch.empty(x.G, x.M_max, x.N, dtype=torch.bfloat16, device=dev)
    ms = median_ms(stream, lambda: dg.m_grouped_fp8_gemm_nt_masked((a, sa), (b, sb), d, mm), reps)
    valid = int(x.masked_m.sum())
    live = int((x.masked_m > 0).sum())
    k4 = (x.K // 128 + 3) // 4
    byts = (valid * x.K + valid * 4 * k4 + live * x.N * x.K + live * 4 * k4 * x.N
            + 2 * valid * x.N + 4 * x.G)
    out["masked_32x256x4096x2048"] = dict(us=round(ms * 1e3, 1),
                                         tflops=round(2.0 * valid * x.N * x.K / ms / 1e9, 1),
                                         gbs=round(byts / ms / 1e6, 1),
                                         frac_hbm=round(byts / ms / 1e6 / PEAK_HBM_GBS, 4))
    del a, sa, b, sb, mm, d, x, wa, wb
    torch.cuda.empty_cache()

    x = gen.gen_k_grouped(seed=0, pow2=True)
    wa, wb = gen.k_grouped_ue8m0_words(x.sfa, x.k_sizes), gen.k_grouped_ue8m0_words(x.sfb, x.k_sizes)
    a, sa, b, sb, c = up(x.a), up(wa), up(x.b), up(wb), up(x.c)
    d = torch.empty(x.G, x.M, x.N, dtype=torch.float32, device=dev)
    ks = x.k_sizes
    ms = median_ms(stream, lambda: dg.k_grouped_fp8_gemm_tn_contiguous((a, sa), (b, sb), d, ks, c=c),
                   reps)
    flop = 2.0 * x.M * x.N * x.K_tot
    byts = x.a.nbytes + wa.nbytes + x.b.nbytes + wb.nbytes + 2 * 4 * x.G * x.M * x.N
    out["k_grouped_32x2048x4096"] = dict(us=round(ms * 1e3, 1), tflops=round(flop / ms / 1e9, 1),
                                        gbs=round(byts / ms / 1e6, 1),
                                        frac_hbm=round(byts / ms / 1e6 / PEAK_HBM_GBS, 4))
    del a, sa, b, sb, c, d, x, wa, wb
    torch.cuda.empty_cache()
    return out


def bench_layouts(dg, gen, up, dev, stream, args):
    """The NN, TN and TT layouts on the 4096 x 4096 x 7168 shape of the dense
    sweep (per-row scales on both operands), and the M-grouped contiguous NN
    form on the contiguous MoE workload (32 experts, N = K = 4096)."""
    import torch
    reps = max(3, min(args.steps, 10))
    out = {}
    M, N, K = 4096, 4096, 7168
    fns = {"nn": dg.fp8_gemm_nn, "tn": dg.fp8_gemm_tn, "tt": dg.fp8_gemm_tt}
    for layout, fn in fns.items():
        x = gen.gen_layout(layout, M, N, K, seed=0)
        a, sa, b, sb = up(x.a), up(x.sfa), up(x.b), up(x.sfb)
        d = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        ms = median_ms(stream, lambda: fn((a, sa), (b, sb), d), reps)
        flop = 2.0 * M * N * K
        out[f"{layout}_{M}x{N}x{K}"] = dict(
            kernel=dg.kernel_config_name({"nn": dg.FORM_NN, "tn": dg.FORM_TN, "tt": dg.FORM_TT}[layout],
                                         M, N, K),
            us=round(ms * 1e3, 1), tflops=round(flop / ms / 1e9, 1),
            frac_mfma=round(flop / ms / 1e9 / PEAK_FP8_TFLOPS, 4))
        del x, a, sa, b, sb, d
    torch.cuda.empty_cache()
    x = gen.gen_nn_contiguous(seed=0)
    a, sa, b, sb, mi = up(x.a), up(x.sfa), up(x.b), up(x.sfb), up(x.m_indices)
    d = torch.empty(x.M_tot, x.N, dtype=torch.bfloat16, device=dev)
    ms = median_ms(stream, lambda: dg.m_grouped_fp8_gemm_nn_contiguous((a, sa), (b, sb), d, mi),
                   reps)
    flop = 2.0 * int(x.counts.sum()) * x.N * x.K
    out["nn_contiguous_32x4096x4096"] = dict(us=round(ms * 1e3, 1), tflops=round(flop / ms / 1e9, 1),
                                             frac_mfma=round(flop / ms / 1e9 / PEAK_FP8_TFLOPS, 4))
    del a, sa, b, sb, mi, d, x
    torch.cuda.empty_cache()
    return out


def bench_mqa(dg, gen, up, dev, stream, args):
    """FP8 MQA logits: 64 heads, head_dim 128, one causal sequence of 4096
    queries over 4096 kv tokens (and 8 packed sequences of 512), -inf cleaning.
    Algorithmic FLOP = 2 * H * D per in-range (query, token) pair; bytes =
    q + kv + kv scales + weights + ranges + the fp32 logits written."""
    import torch
    reps = max(3, min(args.steps, 10))
    out = {}
    for name, lens in (("causal_4096x4096_h64", None), ("packed_8x512_h64", [512] * 8)):
        x = gen.gen_mqa(4096, 4096, H=64, seed=0, seq_lens=lens)
        q, kv, sf, w, ks, ke = up(x.q), up(x.kv), up(x.kv_sf), up(x.weights), up(x.ks), up(x.ke)
        o = torch.empty(x.S, x.S_kv, dtype=torch.float32, device=dev)
        ms = median_ms(stream, lambda: dg.fp8_mqa_logits(q, (kv, sf), w, ks, ke, True, out=o), reps)
        pairs = int(np.clip(x.ke, 0, x.S_kv).astype(np.int64).sum()
                    - np.clip(x.ks, 0, x.S_kv).astype(np.int64).sum())
        flop = 2.0 * x.H * x.D * pairs
        byts = x.q.nbytes + x.kv.nbytes + x.kv_sf.nbytes + x.weights.nbytes + 8 * x.S + 4 * x.S * x.S_kv
        out[name] = dict(us=round(ms * 1e3, 1), tflops=round(flop / ms / 1e9, 1),
                         frac_mfma=round(flop / ms / 1e9 / PEAK_FP8_TFLOPS, 4),
                         gbs=round(byts / ms / 1e6, 1), pairs=pairs)
        del x, q, kv, sf, w, ks, ke, o
    torch.cuda.empty_cache()
    return out


# FP8 casting workloads: the operands of the GEMM workloads above, unquantised
# (bf16), cast by the casting kernels.  name -> (per_block, shape)
CAST_WORKLOADS = {
    "per_token_4096x7168": (False, (4096, 7168)),          # dense M = 4096 A operand
    "per_token_51200x4096": (False, (51200, 4096)),        # contiguous MoE A operand
    "per_token_32x256x2048": (False, (32, 256, 2048)),     # masked MoE A operand
    "per_block_7168x16384": (True, (7168, 16384)),         # dense B operand
    "per_block_32x4096x4096": (True, (32, 4096, 4096)),    # MoE expert weights
}


def cast_bytes(per_block, shape):
    """Algorithmic HBM bytes: bf16 in, e4m3 out, fp32 scales out."""
    n = int(np.prod(shape))
    K = shape[-1]
    rows = int(np.prod(shape[:-1]))
    if per_block:
        G = shape[0] if len(shape) == 3 else 1
        n_sf = G * ((shape[-2] + 127) // 128) * (K // 128)
    else:
        n_sf = rows * (K // 128)
    return 2 * n + n + 4 * n_sf


def bench_cast(dg, dev, stream, args):
    """HIP-event times of the casting kernels on bf16 operands of the GEMM
    workloads' shapes (inputs resident in HBM), against the HBM roof."""
    import torch
    out = {}
    reps = max(3, min(args.steps, 10))
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    for name, (per_block, shape) in CAST_WORKLOADS.items():
        x = torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        fn = dg.per_block_cast_to_fp8 if per_block else dg.per_token_cast_to_fp8
        codes, sf = fn(x)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for e0, e1 in evs:
            e0.record(stream)
            fn(x, out=(codes, sf))
            e1.record(stream)
        torch.cuda.synchronize()
        ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in evs]))
        byts = cast_bytes(per_block, shape)
        out[name] = dict(us=round(ms * 1e3, 1), gbs=round(byts / ms / 1e6, 1),
                         frac_hbm=round(byts / ms / 1e6 / PEAK_HBM_GBS, 4), bytes=byts)
        del x, codes, sf
        torch.cuda.empty_cache()
    return out


def summarize_cast(trace_dir, bench_json, out_path):
    """profiles/ summary of the casting kernels: rocprofv3 per-kernel averages
    next to bench.py's HIP-event timings of the same run."""
    import csv
    res = json.load(open(bench_json))
    cast = res["detail"]["cast"]
    stats = [r for r in csv.DictReader(open(os.path.join(trace_dir, "run_kernel_stats.csv")))
             if "cast_kernel" in r["Name"]]
    lines = ["# FP8 casting kernels (per token 1x128, per block 128x128) -- rocprofv3 kernel trace",
             "", "Commands (run from the repository root on one MI355X):", ""]
    lines += [f"    {c}" for c in GROUPED_PROFILE_COMMANDS[:1]]
    lines += [f"    python3 bench.py --summarize-cast gpurun_out/prof_grouped "
              f"gpurun_out/bench_grouped.json {os.path.relpath(out_path, ROOT)}"]
    lines += ["", "Template arguments: input type (`unsigned short` = bf16 bits), rows per wave,",
              "per-block flag (true = 128 x 128 weights).", "",
              "## Kernel trace (--kernel-trace --stats)", "",
              "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    lines += ["", "## bench.py HIP-event timings (same run; bf16 in, e4m3 + fp32 scales out)", "",
              "| workload | us | algorithmic MB | GB/s | fraction of HBM roof (8 TB/s) |",
              "|---|---|---|---|---|"]
    for name, v in cast.items():
        lines.append(f"| {name} | {v['us']} | {v['bytes'] / 1e6:.1f} | {v['gbs']} | {v['frac_hbm']} |")
    lines += ["", f"    kernel_source_sha256_16: cast {source_hash('cast')}", ""]
    with open(out_path, "w") as f:
        f.write("\n".join(lines))
    print(out_path)


def cpu_baseline(gen, shape, target_s):
    """The fp64 oracle (as it stands) on sampled rows of the dominant shape."""
    import oracle
    M, N, K = shape
    x = gen.gen_dense(M, N, K, seed=0)
    threads = oracle.num_threads()
    rows = np.arange(min(M, threads), dtype=np.int64)
    t0 = time.perf_counter()
    oracle.gemm_nt(x.a, x.sfa, x.b, x.sfb, rows=rows)
    t = time.perf_counter() - t0
    n = int(min(M, max(len(rows), len(rows) * target_s / max(t, 1e-3))))
    n = max(threads, (n // threads) * threads) if n >= threads else n
    rows = np.arange(n, dtype=np.int64)
    t0 = time.perf_counter()
    oracle.gemm_nt(x.a, x.sfa, x.b, x.sfb, rows=rows)
    t = time.perf_counter() - t0
    flop = 2.0 * n * N * K
    return {"value": round(flop / t / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{n} of {M} rows of the dense {M}x{N}x{K} shape (all {N} columns), "
                      f"{t:.1f} s, fp64 exact block sums"}


if __name__ == "__main__":
    main()
