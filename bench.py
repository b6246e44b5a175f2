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
  detail       -- per-shape times (each launch after a 512 MiB write that
                  flushes L2 and the Infinity Cache, median / min / p90 over
                  --reps repetitions), the C1 shape, the three grouped MoE workloads
                  (contiguous, masked, K-grouped) timed the same way, the
                  FP8 casting kernels on bf16 operands of those shapes, and
                  the power-of-two (packed UE8M0) scale variant of the dense
                  sweep and the contiguous and masked workloads, and the NN /
                  TN / TT layouts and the M-grouped contiguous NN form, and the
                  FP8 MQA logits kernel on a 64-head causal prefill.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--reps R] [--no-detail]
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
# the same peak from the chip's units at its peak engine clock:
# 256 CUs x 8192 FP8 FLOP per clock x 2.4 GHz
PEAK_FP8_TFLOPS_CLOCK = 256 * 8192 * 2.4e9 / 1e12
FLUSH_BYTES = 512 << 20      # written before every detail repetition (L2 + 256 MB Infinity Cache)
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E (published)
MACHINE_BALANCE = PEAK_FP8_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)   # FLOP per byte

# The rocprofv3 runs behind the profiles/ summaries (repository root, one GPU):
# a kernel trace, FETCH_SIZE and WRITE_SIZE passes (HBM-side bytes, scaled
# by a 1 GiB device copy of known traffic), and an MFMA pass (MFMA busy
# cycles per SIMD, GPU-active cycles for the clock, FP8 MFMA op counts).
# Each counter pass is a run of its own.
MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_F8 "
                 "SQ_INSTS_VALU_MFMA_MOPS_F6F4")


PROF_OUT = "rocprof_out"   # where the profiling runs write (not versioned)


def _profile_commands(tag, trace_args, pmc_args, summarize):
    pre = "rocprofv3 {} --output-format csv -d " + PROF_OUT + "/prof_{}_{} -o run -- python3 bench.py "
    return [pre.format("--kernel-trace --stats", tag, "trace") + trace_args
            + f" --json-out {PROF_OUT}/bench_{tag}.json",
            pre.format("--pmc FETCH_SIZE", tag, "fetch") + pmc_args + " --copy-calibration",
            pre.format("--pmc WRITE_SIZE", tag, "write") + pmc_args + " --copy-calibration",
            pre.format("--pmc " + MFMA_COUNTERS, tag, "mfma") + pmc_args,
            f"python3 bench.py {summarize} {PROF_OUT}/prof_{tag} {PROF_OUT}/bench_{tag}.json profiles"]


# dense sweep: the roofline's dominant instance and the decode-size instances
PROFILE_COMMANDS = _profile_commands(
    "dense", "--no-detail --no-cpu", "--steps 2 --warmup 2 --reps 1 --no-detail --no-cpu",
    "--summarize-dense")
# every detail workload (C1, grouped MoE, casting, UE8M0, layouts, MQA logits)
DETAIL_PROFILE_COMMANDS = _profile_commands(
    "detail", "--steps 3 --warmup 1 --reps 10 --no-cpu", "--steps 1 --warmup 0 --reps 1 --no-cpu",
    "--summarize-detail")


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
    ap.add_argument("--reps", type=int, default=30,
                    help="timed repetitions per detail workload (median / min / p90)")
    ap.add_argument("--no-detail", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 1 GiB device copy before the GEMMs (a kernel of known "
                         "traffic, to scale hardware byte counters)")
    ap.add_argument("--summarize-dense", nargs=3, metavar=("PROF_PREFIX", "BENCH_JSON", "OUT_DIR"),
                    help="write the dense-sweep profiles/ summaries from rocprofv3 CSV output")
    ap.add_argument("--summarize-detail", nargs=3, metavar=("PROF_PREFIX", "BENCH_JSON", "OUT_DIR"),
                    help="write the detail-workload profiles/ summaries from rocprofv3 CSV output")
    args = ap.parse_args()

    if args.summarize_dense:
        summarize_set(*args.summarize_dense, families=DENSE_FAMILIES, commands=PROFILE_COMMANDS)
        return
    if args.summarize_detail:
        summarize_set(*args.summarize_detail, families=DETAIL_FAMILIES,
                      commands=DETAIL_PROFILE_COMMANDS)
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
    # one caller-owned split-K workspace serves every shape: calls on one
    # stream run in order and each leaves the counters zero for the next
    ws_bytes = max(dg.get_fp8_gemm_nt_workspace_bytes(*s_) for s_ in shapes)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
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

    def launch(op):
        dg.fp8_gemm_nt(*op["args"], workspace=ws)

    def step(events=None, only=None):
        # with `only`, one event pair spans each run of consecutive launches
        # of that instance (its start before the run's first launch, its end
        # after the last); otherwise one pair per launch
        for i, op in enumerate(ops):
            mine = events is not None and (only is None or op["kernel"] == only)
            first = mine and (only is None or i == 0 or ops[i - 1]["kernel"] != only)
            last = mine and (only is None or i + 1 == len(ops) or ops[i + 1]["kernel"] != only)
            if first:
                events[i][0].record(stream)
            launch(op)
            if last:
                events[i][1].record(stream)

    def new_events(n):
        return [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in ops] for _ in range(n)]

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- per-shape detail (untimed by the step clock) -------------------------------
    # Each shape alone, --reps times, every repetition after a 512 MiB write
    # that evicts its operands from L2 and the Infinity Cache (outside the
    # event pair): median, min and p90.  It also picks the dominant kernel:
    # the instance (tile configuration) with the largest share of the sweep's
    # median time.  Several shapes may share one instance.
    timer = Timer(stream, args.reps)
    per_stats = [timer.measure(lambda op=op: launch(op)) for op in ops]
    avg_ms = np.array([st["median_us"] for st in per_stats]) * 1e-3
    groups = {}
    for i, op in enumerate(ops):
        groups.setdefault(op["kernel"], []).append(i)
    dom_name = max(groups, key=lambda k: sum(avg_ms[i] for i in groups[k]))
    idx = groups[dom_name]

    # ---- timed region: exactly K steps ---------------------------------------------
    # Event pairs only around the dominant instance's launches, one pair per
    # run of consecutive launches of it (an event pair around every launch
    # adds several microseconds per launch to the step and to the launch).
    runs = []
    for i in idx:
        if runs and runs[-1][-1] == i - 1:
            runs[-1].append(i)
        else:
            runs.append([i])
    ev = new_events(args.steps)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s_ in range(args.steps):
        step(ev[s_], only=dom_name)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    # per step: the runs' spans in ms, and their launch counts
    dom_span = np.array([[ev[s_][r[0]][0].elapsed_time(ev[s_][r[-1]][1]) for r in runs]
                         for s_ in range(args.steps)])
    flop_step = sum(op["flop"] for op in ops)
    value = flop_step * args.steps / elapsed / 1e12
    ms_per_step = elapsed * 1e3 / args.steps

    # Per-launch figures of the dominant instance: averages over its launches
    # in the timed region -- the same average a kernel-trace profile reports
    # for that kernel name.
    launch_ms = float(dom_span.sum() / (args.steps * len(idx)))
    launch_flop = float(np.mean([ops[i]["flop"] for i in idx]))
    launch_bytes = float(np.mean([ops[i]["bytes"] for i in idx]))
    intensity = launch_flop / launch_bytes
    if intensity >= MACHINE_BALANCE:
        achieved = launch_flop / (launch_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=PEAK_FP8_TFLOPS,
                    unit="TFLOP/s", frac=round(achieved / PEAK_FP8_TFLOPS, 4), traffic=None,
                    frac_of_clock_peak=round(achieved / PEAK_FP8_TFLOPS_CLOCK, 4))
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

    per_shape = []   # from the per-shape pass (flushed, --reps repetitions)
    for op, st in zip(ops, per_stats):
        m, n, k = op["shape"]
        t = st["median_us"] * 1e-3
        row = dict(M=m, N=n, K=k, kernel=op["kernel"], us=st["median_us"],
                   us_min=st["min_us"], us_p90=st["p90_us"],
                   tflops=round(op["flop"] / (t * 1e-3) / 1e12, 1),
                   gbs=round(op["bytes"] / (t * 1e-3) / 1e9, 1))
        if op["flop"] / op["bytes"] >= MACHINE_BALANCE:
            row["frac_mfma"] = round(op["flop"] / (t * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4)
        else:
            row["frac_hbm"] = round(op["bytes"] / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        per_shape.append(row)
    print(f"[bench] step {ms_per_step:.3f} ms, {value:.1f} TFLOP/s", file=sys.stderr, flush=True)

    # ---- grouped workloads (detail, timed the same way) ------------------------------
    grouped, cast, ue8m0, layouts, mqa, c1 = {}, {}, {}, {}, {}, {}
    if not args.no_detail:
        del ops
        torch.cuda.empty_cache()
        c1 = bench_c1(dg, gen, up, dev, timer)
        grouped = bench_grouped(dg, gen, up, dev, timer)
        cast = bench_cast(dg, dev, timer)
        ue8m0 = bench_ue8m0(dg, gen, up, dev, timer)
        layouts = bench_layouts(dg, gen, up, dev, timer)
        mqa = bench_mqa(dg, gen, up, dev, timer)

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
        "detail": {"timing": f"HIP events around each launch on its stream; a {FLUSH_BYTES >> 20} MiB "
                             f"write before every repetition, outside the events; median, min and "
                             f"p90 of {args.reps} repetitions after one untimed launch",
                   "dense": per_shape, "c1": c1, "grouped": grouped, "cast": cast, "ue8m0": ue8m0,
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
    "mqa": ["fp8_fine_grained_e4m3_amd/csrc/mqa_kernel.hip",
            "fp8_fine_grained_e4m3_amd/csrc/tile_common.h",
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
        h = re.search(r"kernel_source_sha256_16:\s*(.+)", text)
        if not (m and h and fam in KERNEL_SOURCES):
            continue
        # "nt <hash>, tn <hash>, ..." or, for a one-family summary, the bare hash
        hashes = dict(re.findall(r"(nt|tn|cast|mqa)\s+([0-9a-f]{16})", h.group(1)))
        recorded = hashes.get(fam, h.group(1).strip())
        if recorded == source_hash(fam):
            return float(m.group(1))
    return None


def _read_csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _counter_rows(prefix, kind):
    """{dispatch id: {"kernel", "ns", counter: value}} of one counter pass."""
    out = {}
    for r in _read_csv(os.path.join(f"{prefix}_{kind}", "run_counter_collection.csv")):
        d = out.setdefault(int(r["Dispatch_Id"]), {
            "kernel": r["Kernel_Name"],
            "ns": float(r["End_Timestamp"]) - float(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def _num_xcc(prefix):
    try:
        for r in _read_csv(os.path.join(f"{prefix}_mfma", "run_agent_info.csv")):
            if r.get("Agent_Type", r.get("Type", "")).upper().endswith("GPU") or "gfx" in str(r):
                for key in ("Num_Xcc", "Num_XCC", "num_xcc"):
                    if key in r and r[key]:
                        return int(float(r[key]))
    except (OSError, KeyError, ValueError):
        pass
    return 8


CLOCK_MIN_NS = 50_000   # dispatches shorter than this report no clock


def instance_stats(prefix):
    """Per kernel name: trace average (us, calls), scaled HBM fetch / write
    bytes per dispatch, MFMA busy %, shader clock and counted MFMA FLOP per
    dispatch, from the four runs of one profile set."""
    stats = {r["Name"]: r for r in _read_csv(os.path.join(f"{prefix}_trace", "run_kernel_stats.csv"))}
    fetch, write, mfma = (_counter_rows(prefix, k) for k in ("fetch", "write", "mfma"))
    copy = float(1 << 30)
    f_scale = copy / (max(d["FETCH_SIZE"] for d in fetch.values() if "copyBuffer" in d["kernel"]) * 1024)
    w_scale = copy / (max(d["WRITE_SIZE"] for d in write.values() if "copyBuffer" in d["kernel"]) * 1024)
    xcc = _num_xcc(prefix)
    out = {}
    for name, st in stats.items():
        e = dict(calls=int(st["Calls"]), avg_us=float(st["AverageNs"]) / 1e3,
                 min_us=float(st["MinNs"]) / 1e3, max_us=float(st["MaxNs"]) / 1e3)
        fv = [d["FETCH_SIZE"] * 1024 * f_scale for d in fetch.values() if d["kernel"] == name]
        wv = [d["WRITE_SIZE"] * 1024 * w_scale for d in write.values() if d["kernel"] == name]
        if fv and wv:
            e.update(fetch_b=float(np.mean(fv)), write_b=float(np.mean(wv)), n_pmc=len(fv))
        mv = [d for d in mfma.values() if d["kernel"] == name and d.get("GRBM_GUI_ACTIVE", 0) > 0]
        if mv:
            grbm = np.array([d["GRBM_GUI_ACTIVE"] for d in mv]) / xcc      # cycles per XCC
            busy = np.array([d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for d in mv])
            mops = np.array([d.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0)
                             + d.get("SQ_INSTS_VALU_MFMA_MOPS_F6F4", 0.0) for d in mv])
            ns = np.array([d["ns"] for d in mv])
            e.update(mfma_busy_pct=float(np.mean(busy / (grbm * 1024.0) * 100.0)),
                     mfma_flop=float(np.mean(mops * 512.0)))
            # GRBM_GUI_ACTIVE also counts the GPU-active cycles around a
            # dispatch (launch, counter setup), which dominate a short one:
            # its cycles / duration is a clock only for long dispatches
            if np.mean(ns) >= CLOCK_MIN_NS:
                e.update(clock_ghz=float(np.mean(grbm / ns)))
        out[name] = e
    return out, dict(fetch_scale=f_scale, write_scale=w_scale, xcc=xcc)


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


def _nt(form, ue8m0="false", tile=None):
    tail = f", {form}, false, {ue8m0}>"
    return lambda k: "nt_fp8_kernel" in k and tail in k and (tile is None or f"NtCfg<{tile}," in k)


def _tn(args):
    return lambda k: "tn_fp8_kernel" in k and args in k


# A family: one profiles/ file.  `match` picks its kernels; `workloads` map a
# bench detail record to the single kernel instance that runs it (for the
# bytes-per-algorithmic-byte ratio); `traffic_for` marks the dominant dense
# instance, whose file carries the traffic figure bench.py reports.
DENSE_FAMILIES = [
    dict(file="{dominant}__dense_sweep.md", dominant=True,
         title="Dominant instance of the dense FP8 NT sweep (the five M = 4096 shapes)",
         note="`nt_fp8_kernel<Cfg, FORM, OUT_F32, UE8M0>`, FORM 0 = dense."),
    dict(file="nt_dense_decode__m64_m128_shapes.md",
         title="Decode-size dense instances (the ten M = 64 / 128 shapes of the sweep)",
         match=lambda k: (_nt(0, tile="64, 64")(k) or _nt(0, tile="64, 256")(k)
                          or _nt(0, tile="128, 64")(k) or _nt(0, tile="128, 256")(k)),
         note="`NtCfg<64, 256, ...>` and `NtCfg<128, 256, ...>` run M x 7168 x 16384 (N * K >= "
              "64 Mi), `NtCfg<64, 64, ...>` and `NtCfg<128, 64, ...>` the other M = 64 and M = 128 "
              "shapes; K is split over workgroups (caller-owned workspace)."),
]
DETAIL_FAMILIES = [
    dict(file="grouped_moe__contiguous_masked_kgrouped.md",
         title="Grouped MoE workloads (contiguous, masked, K-grouped), fp32 scales",
         match=lambda k: _nt(1)(k) or _nt(2)(k) or _tn("false, false, true, false, false>")(k),
         workloads=[("grouped.contiguous_32x4096x4096", _nt(1)),
                    ("grouped.masked_32x256x4096x2048", _nt(2)),
                    ("grouped.k_grouped_32x2048x4096", _tn("false, false, true, false, false>"))],
         note="`nt_fp8_kernel<Cfg, FORM, OUT_F32, UE8M0>`: FORM 1 = contiguous, 2 = masked. "
              "`tn_fp8_kernel<Cfg, A_MK, B_NK, OUT_F32, GROUPED_M, UE8M0>` with "
              "`false, false, true, false, false` = the K-grouped form."),
    dict(file="ue8m0__dense_sweep_contiguous_masked_kgrouped.md",
         title="Packed UE8M0 scales (block-scaled MFMA): dense sweep, contiguous, masked, K-grouped",
         match=lambda k: ("nt_fp8_kernel" in k and "true>(dg::NtArgs" in k)
         or _tn("false, false, true, false, true>")(k) or "pack_ue8m0" in k,
         workloads=[("ue8m0.contiguous_32x4096x4096", _nt(1, "true")),
                    ("ue8m0.masked_32x256x4096x2048", _nt(2, "true")),
                    ("ue8m0.k_grouped_32x2048x4096", _tn("false, false, true, false, true>"))],
         note="Last template argument `true` = UE8M0 instance."),
    dict(file="mn_major_layouts__nn_tn_tt_4096x4096x7168_and_nn_contiguous.md",
         title="NN / TN / TT layouts and the M-grouped contiguous NN form (MN-major kernel)",
         match=lambda k: "tn_fp8_kernel" in k and "false, false, true, false" not in k,
         workloads=[("layouts.nn_4096x4096x7168", _tn("true, false, false, false, false>")),
                    ("layouts.tn_4096x4096x7168", _tn("false, false, false, false, false>")),
                    ("layouts.tt_4096x4096x7168", _tn("false, true, false, false, false>")),
                    ("layouts.nn_contiguous_32x4096x4096", _tn("true, false, false, true, false>"))],
         note="`tn_fp8_kernel<Cfg, A_MK, B_NK, OUT_F32, GROUPED_M, UE8M0>`: A_MK = A stored [M, K], "
              "B_NK = B stored [N, K], GROUPED_M = contiguous NN."),
    dict(file="mqa_logits__causal_prefill_4096x4096_h64.md",
         title="FP8 MQA logits, 64 heads, causal 4096 x 4096 and 8 packed sequences of 512",
         match=lambda k: "mqa_logits_kernel" in k,
         note="`mqa_logits_kernel<H>`, H = heads; both workloads run the same instance."),
    dict(file="fp8_cast__per_token_per_block.md",
         title="FP8 casting kernels (per token 1 x 128, per block 128 x 128)",
         match=lambda k: "cast_kernel" in k,
         note="Template arguments: input type (`unsigned short` = bf16 bits), rows per wave, "
              "per-block flag (true = 128 x 128 weights)."),
]


def _detail(res, path):
    v = res.get("detail", {})
    for p in path.split("."):
        v = v.get(p, {}) if isinstance(v, dict) else {}
    return v


def summarize_set(prefix, bench_json, out_dir, families, commands):
    """Write the profiles/ summaries of one profile set (kernel trace plus the
    three counter passes), one file per family."""
    res = json.load(open(bench_json))
    inst, cal = instance_stats(prefix)
    roof = res["roofline"]
    for fam in families:
        if fam.get("dominant"):
            name = roof["kernel"]
            match, tag = instance_matcher(name)
            fname = fam["file"].format(dominant=name)
        else:
            match, fname = fam["match"], fam["file"]
        rows = {k: v for k, v in inst.items() if match(k)}
        lines = [f"# {fam['title']} -- rocprofv3", "",
                 "Commands (run from the repository root on one MI355X):", ""]
        lines += [f"    {c}" for c in commands]
        lines += ["", fam["note"], "",
                  "Counters: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what they read "
                  f"for a 1 GiB device copy (`__amd_rocclr_copyBuffer`): fetch x{cal['fetch_scale']:.4f}, "
                  f"write x{cal['write_scale']:.4f}.  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / "
                  f"(GRBM_GUI_ACTIVE per XCC x 1024 SIMDs); clock = GRBM_GUI_ACTIVE per XCC / dispatch "
                  f"time ({cal['xcc']} XCCs); MFMA FLOP = (SQ_INSTS_VALU_MFMA_MOPS_F8 + _F6F4) x 512.  "
                  "Counter passes serialise dispatches, so their clock is that of isolated launches; "
                  "dispatches shorter than 50 us report none (the active cycles around the dispatch "
                  "dominate them), and their MFMA busy % is a lower bound for the same reason.",
                  "", "## Per kernel instance", "",
                  "| kernel | calls (trace) | trace avg us | min | max | HBM fetch MB / dispatch | "
                  "HBM write MB / dispatch | MFMA busy % | clock GHz | MFMA GFLOP / dispatch |",
                  "|---|---|---|---|---|---|---|---|---|---|"]
        for k, e in sorted(rows.items(), key=lambda kv: -kv[1]["avg_us"] * kv[1]["calls"]):
            f = lambda key, sc=1e-6, fmt="{:.1f}": fmt.format(e[key] * sc) if key in e else "-"
            lines.append(f"| `{k[:110]}` | {e['calls']} | {e['avg_us']:.2f} | {e['min_us']:.2f} | "
                         f"{e['max_us']:.2f} | {f('fetch_b')} | {f('write_b')} | "
                         f"{f('mfma_busy_pct', 1.0)} | {f('clock_ghz', 1.0, '{:.2f}')} | "
                         f"{f('mfma_flop', 1e-9, '{:.2f}')} |")
        machine = []
        if fam.get("dominant"):
            e = [v for k, v in rows.items()]
            e = e[0] if e else {}
            lines += ["", f"Dominant instance `{tag}` = `{name}`: {roof['launches_per_step']} launches per "
                          f"step ({', '.join(roof['shapes'])}); rocprofv3 trace average "
                          f"{e.get('avg_us', float('nan')):.2f} us per launch, bench.py's HIP-event "
                          f"average over its timed region {roof['avg_launch_us']} us.",
                      f"Algorithmic work per launch (mean over those shapes): "
                      f"{roof['alg_flop_per_launch'] / 1e9:.2f} GFLOP, "
                      f"{roof['alg_bytes_per_launch'] / 1e6:.2f} MB."]
            if "fetch_b" in e:
                tot = e["fetch_b"] + e["write_b"]
                lines.append(f"HBM traffic per launch: fetch {e['fetch_b'] / 1e6:.1f} MB + write "
                             f"{e['write_b'] / 1e6:.1f} MB = {tot / 1e6:.1f} MB, "
                             f"{tot / roof['alg_bytes_per_launch']:.2f}x the algorithmic bytes.")
                machine.append(f"    traffic_bytes_per_launch: {tot:.0f}")
            if "mfma_flop" in e:
                lines.append(f"MFMA FLOP counted per launch {e['mfma_flop'] / 1e9:.2f} G against "
                             f"{roof['alg_flop_per_launch'] / 1e9:.2f} G algorithmic; MFMA busy "
                             f"{e['mfma_busy_pct']:.1f}%"
                             + (f" at {e['clock_ghz']:.2f} GHz." if "clock_ghz" in e else "."))
        if fam.get("workloads"):
            lines += ["", "## Workloads run by one instance each (bench.py, same trace run)", "",
                      "| workload | bench median us | min | p90 | trace avg us | alg MB | "
                      "HBM MB (fetch + write) | HBM / alg | alg GFLOP | MFMA GFLOP counted | "
                      "MFMA busy % | frac of roof |", "|---|---|---|---|---|---|---|---|---|---|---|---|"]
            for label, pred in fam["workloads"]:
                d = _detail(res, label)
                hit = [v for k, v in rows.items() if pred(k)]
                if not d or len(hit) != 1:
                    continue
                e = hit[0]
                hbm = e.get("fetch_b", float("nan")) + e.get("write_b", float("nan"))
                frac = d.get("frac_mfma", d.get("frac_hbm"))
                roofname = "MFMA" if "frac_mfma" in d else "HBM"
                lines.append(
                    f"| {label} | {d.get('us')} | {d.get('us_min')} | {d.get('us_p90')} | "
                    f"{e['avg_us']:.2f} | {d.get('alg_bytes', 0) / 1e6:.1f} | {hbm / 1e6:.1f} | "
                    f"{hbm / max(d.get('alg_bytes', 1), 1):.2f} | {d.get('alg_flop', 0) / 1e9:.1f} | "
                    f"{e.get('mfma_flop', float('nan')) / 1e9:.1f} | "
                    f"{e.get('mfma_busy_pct', float('nan')):.1f} | {frac} {roofname} |")
        lines += ["", "Machine-readable:", ""] + machine
        fams = ("nt", "tn", "cast", "mqa")
        lines += ["    kernel_source_sha256_16: " + ", ".join(f"{f} {source_hash(f)}" for f in fams),
                  f"    bench_value_tflops: {res['value']}", ""]
        path = os.path.join(out_dir, fname)
        with open(path, "w") as fh:
            fh.write("\n".join(lines))
        print(path)


class Timer:
    """Detail timing: an event pair around each launch on `stream`, and before
    every repetition (outside the pair) a FLUSH_BYTES write that evicts the
    operands from the L2 caches and the 256 MB Infinity Cache, so every
    repetition reads its operands from HBM.  One untimed launch first."""

    def __init__(self, stream, reps):
        import torch
        self.stream = stream
        self.reps = max(1, int(reps))
        self.flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=stream.device)
        self.fill = 0.0

    def measure(self, fn):
        import torch
        fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(self.reps)]
        with torch.cuda.stream(self.stream):
            for e0, e1 in evs:
                self.fill += 1.0
                self.flush.fill_(self.fill)
                e0.record(self.stream)
                fn()
                e1.record(self.stream)
        torch.cuda.synchronize()
        t = np.array([e0.elapsed_time(e1) for e0, e1 in evs]) * 1e3
        return dict(median_us=round(float(np.median(t)), 2), min_us=round(float(t.min()), 2),
                    p90_us=round(float(np.percentile(t, 90)), 2), reps=self.reps)


def entry(st, flop, byts, roof, **extra):
    """One detail record: times, TFLOP/s, GB/s and the fraction of the binding
    roof (MFMA: fp8 dense peak; HBM: 8 TB/s) at the median time."""
    t = st["median_us"] * 1e-6
    out = dict(us=st["median_us"], us_min=st["min_us"], us_p90=st["p90_us"], reps=st["reps"],
               tflops=round(flop / t / 1e12, 1), gbs=round(byts / t / 1e9, 1),
               alg_flop=flop, alg_bytes=byts)
    if roof == "mfma":
        out["frac_mfma"] = round(flop / t / 1e12 / PEAK_FP8_TFLOPS, 4)
    else:
        out["frac_hbm"] = round(byts / t / 1e9 / PEAK_HBM_GBS, 4)
    out.update(extra)
    return out


def bench_c1(dg, gen, up, dev, timer):
    """The smallest configuration, dense 128 x 256 x 512 (bound by launch
    latency; reported, no roofline target)."""
    print("[bench] detail: c1", file=sys.stderr, flush=True)
    import torch
    M, N, K = 128, 256, 512
    x = gen.gen_dense(M, N, K, seed=0)
    a, sa, b, sb = up(x.a), up(x.sfa), up(x.b), up(x.sfb)
    d = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    ws = dg.make_fp8_gemm_nt_workspace(M, N, K, dev)
    st = timer.measure(lambda: dg.fp8_gemm_nt((a, sa), (b, sb), d, workspace=ws))
    return {"dense_128x256x512": entry(st, 2.0 * M * N * K, dense_bytes(M, N, K), "hbm",
                                       kernel=dg.kernel_config_name(dg.FORM_DENSE, M, N, K))}


def bench_grouped(dg, gen, up, dev, timer):
    print("[bench] detail: grouped", file=sys.stderr, flush=True)
    import torch
    out = {}

    # contiguous (MoE forward)
    x = gen.gen_contiguous(seed=0)
    a, sa, b, sb, mi = up(x.a), up(x.sfa), up(x.b), up(x.sfb), up(x.m_indices)
    d = torch.empty(x.M_tot, x.N, dtype=torch.bfloat16, device=dev)
    st = timer.measure(lambda: dg.m_grouped_fp8_gemm_nt_contiguous((a, sa), (b, sb), d, mi))
    valid = int(x.counts.sum())
    flop = 2.0 * valid * x.N * x.K
    byts = x.a.nbytes + x.sfa.nbytes + x.b.nbytes + x.sfb.nbytes + x.m_indices.nbytes + 2 * x.M_tot * x.N
    out["contiguous_32x4096x4096"] = entry(st, flop, byts, "mfma")
    del a, sa, b, sb, mi, d, x
    torch.cuda.empty_cache()

    # masked (MoE decode)
    x = gen.gen_masked(seed=0)
    a, sa, b, sb, mm = up(x.a), up(x.sfa), up(x.b), up(x.sfb), up(x.masked_m)
    d = torch.empty(x.G, x.M_max, x.N, dtype=torch.bfloat16, device=dev)
    st = timer.measure(lambda: dg.m_grouped_fp8_gemm_nt_masked((a, sa), (b, sb), d, mm))
    valid = int(x.masked_m.sum())
    live = int((x.masked_m > 0).sum())
    flop = 2.0 * valid * x.N * x.K
    byts = (valid * x.K + valid * 4 * (x.K // 128) + live * x.N * x.K
            + live * 4 * ((x.N + 127) // 128) * (x.K // 128) + 2 * valid * x.N + 4 * x.G)
    out["masked_32x256x4096x2048"] = entry(st, flop, byts, "hbm")
    del a, sa, b, sb, mm, d, x
    torch.cuda.empty_cache()

    # K-grouped TN (MoE weight gradient)
    x = gen.gen_k_grouped(seed=0)
    a, sa, b, sb, c = up(x.a), up(x.sfa), up(x.b), up(x.sfb), up(x.c)
    d = torch.empty(x.G, x.M, x.N, dtype=torch.float32, device=dev)
    ks = x.k_sizes
    st = timer.measure(lambda: dg.k_grouped_fp8_gemm_tn_contiguous((a, sa), (b, sb), d, ks, c=c))
    flop = 2.0 * x.M * x.N * x.K_tot
    byts = x.a.nbytes + x.sfa.nbytes + x.b.nbytes + x.sfb.nbytes + 2 * 4 * x.G * x.M * x.N
    out["k_grouped_32x2048x4096"] = entry(st, flop, byts, "hbm")
    del a, sa, b, sb, c, d, x
    torch.cuda.empty_cache()
    return out


def bench_ue8m0(dg, gen, up, dev, timer):
    """The same workloads with power-of-two scales packed as UE8M0 words (the
    MFMA applies the scales; no separate promotion): the dense sweep shape by
    shape, and the contiguous, masked and K-grouped MoE workloads."""
    print("[bench] detail: ue8m0", file=sys.stderr, flush=True)
    import torch
    ops = []
    for (M, N, K) in gen.DENSE_SWEEP:
        x = gen.gen_dense_ue8m0(M, N, K, seed=0)
        ops.append(((M, N, K), (up(x.a), up(x.sfa)), (up(x.b), up(x.sfb)),
                    torch.empty(M, N, dtype=torch.bfloat16, device=dev)))
        del x
    ws_bytes = max(dg.get_fp8_gemm_nt_workspace_bytes(*o[0]) for o in ops)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    dense = []
    for (M, N, K), a, b, d in ops:
        st = timer.measure(lambda: dg.fp8_gemm_nt(a, b, d, workspace=ws))
        flop = 2.0 * M * N * K
        byts = M * K + N * K + 4 * ((K // 128 + 3) // 4) * (M + N) + 2 * M * N
        dense.append(dict(M=M, N=N, K=K, **entry(st, flop, byts,
                                                 "mfma" if flop / byts >= MACHINE_BALANCE else "hbm")))
    out = {"dense": dense}
    del ops
    torch.cuda.empty_cache()

    x = gen.gen_contiguous(seed=0, pow2=True)
    wa, wb = gen.to_ue8m0(x.sfa, x.sfb, x.N)
    a, sa, b, sb, mi = up(x.a), up(wa), up(x.b), up(wb), up(x.m_indices)
    d = torch.empty(x.M_tot, x.N, dtype=torch.bfloat16, device=dev)
    st = timer.measure(lambda: dg.m_grouped_fp8_gemm_nt_contiguous((a, sa), (b, sb), d, mi))
    flop = 2.0 * int(x.counts.sum()) * x.N * x.K
    byts = x.a.nbytes + wa.nbytes + x.b.nbytes + wb.nbytes + x.m_indices.nbytes + 2 * x.M_tot * x.N
    out["contiguous_32x4096x4096"] = entry(st, flop, byts, "mfma")
    del a, sa, b, sb, mi, d, x, wa, wb
    torch.cuda.empty_cache()

    x = gen.gen_masked(seed=0, pow2=True)
    wa, wb = gen.to_ue8m0(x.sfa, x.sfb, x.N)
    a, sa, b, sb, mm = up(x.a), up(wa), up(x.b), up(wb), up(x.masked_m)
    d = torch.empty(x.G, x.M_max, x.N, dtype=torch.bfloat16, device=dev)
    st = timer.measure(lambda: dg.m_grouped_fp8_gemm_nt_masked((a, sa), (b, sb), d, mm))
    valid = int(x.masked_m.sum())
    live = int((x.masked_m > 0).sum())
    k4 = (x.K // 128 + 3) // 4
    byts = (valid * x.K + valid * 4 * k4 + live * x.N * x.K + live * 4 * k4 * x.N
            + 2 * valid * x.N + 4 * x.G)
    out["masked_32x256x4096x2048"] = entry(st, 2.0 * valid * x.N * x.K, byts, "hbm")
    del a, sa, b, sb, mm, d, x, wa, wb
    torch.cuda.empty_cache()

    x = gen.gen_k_grouped(seed=0, pow2=True)
    wa, wb = gen.k_grouped_ue8m0_words(x.sfa, x.k_sizes), gen.k_grouped_ue8m0_words(x.sfb, x.k_sizes)
    a, sa, b, sb, c = up(x.a), up(wa), up(x.b), up(wb), up(x.c)
    d = torch.empty(x.G, x.M, x.N, dtype=torch.float32, device=dev)
    ks = x.k_sizes
    st = timer.measure(lambda: dg.k_grouped_fp8_gemm_tn_contiguous((a, sa), (b, sb), d, ks, c=c))
    flop = 2.0 * x.M * x.N * x.K_tot
    byts = x.a.nbytes + wa.nbytes + x.b.nbytes + wb.nbytes + 2 * 4 * x.G * x.M * x.N
    out["k_grouped_32x2048x4096"] = entry(st, flop, byts, "hbm")
    del a, sa, b, sb, c, d, x, wa, wb
    torch.cuda.empty_cache()
    return out


def bench_layouts(dg, gen, up, dev, timer):
    """The NN, TN and TT layouts on the 4096 x 4096 x 7168 shape of the dense
    sweep (per-row scales on both operands), and the M-grouped contiguous NN
    form on the contiguous MoE workload (32 experts, N = K = 4096)."""
    print("[bench] detail: layouts", file=sys.stderr, flush=True)
    import torch
    out = {}
    M, N, K = 4096, 4096, 7168
    fns = {"nn": dg.fp8_gemm_nn, "tn": dg.fp8_gemm_tn, "tt": dg.fp8_gemm_tt}
    for layout, fn in fns.items():
        x = gen.gen_layout(layout, M, N, K, seed=0)
        a, sa, b, sb = up(x.a), up(x.sfa), up(x.b), up(x.sfb)
        d = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        st = timer.measure(lambda: fn((a, sa), (b, sb), d))
        byts = x.a.nbytes + x.sfa.nbytes + x.b.nbytes + x.sfb.nbytes + 2 * M * N
        out[f"{layout}_{M}x{N}x{K}"] = entry(
            st, 2.0 * M * N * K, byts, "mfma",
            kernel=dg.kernel_config_name({"nn": dg.FORM_NN, "tn": dg.FORM_TN, "tt": dg.FORM_TT}[layout],
                                         M, N, K))
        del x, a, sa, b, sb, d
    torch.cuda.empty_cache()
    x = gen.gen_nn_contiguous(seed=0)
    a, sa, b, sb, mi = up(x.a), up(x.sfa), up(x.b), up(x.sfb), up(x.m_indices)
    d = torch.empty(x.M_tot, x.N, dtype=torch.bfloat16, device=dev)
    st = timer.measure(lambda: dg.m_grouped_fp8_gemm_nn_contiguous((a, sa), (b, sb), d, mi))
    flop = 2.0 * int(x.counts.sum()) * x.N * x.K
    byts = x.a.nbytes + x.sfa.nbytes + x.b.nbytes + x.sfb.nbytes + x.m_indices.nbytes + 2 * x.M_tot * x.N
    out["nn_contiguous_32x4096x4096"] = entry(st, flop, byts, "mfma")
    del a, sa, b, sb, mi, d, x
    torch.cuda.empty_cache()
    return out


def bench_mqa(dg, gen, up, dev, timer):
    """FP8 MQA logits: 64 heads, head_dim 128, one causal sequence of 4096
    queries over 4096 kv tokens (and 8 packed sequences of 512), -inf cleaning.
    Algorithmic FLOP = 2 * H * D per in-range (query, token) pair; bytes =
    q + kv + kv scales + weights + ranges + the fp32 logits written."""
    print("[bench] detail: mqa", file=sys.stderr, flush=True)
    import torch
    out = {}
    for name, lens in (("causal_4096x4096_h64", None), ("packed_8x512_h64", [512] * 8)):
        x = gen.gen_mqa(4096, 4096, H=64, seed=0, seq_lens=lens)
        q, kv, sf, w, ks, ke = up(x.q), up(x.kv), up(x.kv_sf), up(x.weights), up(x.ks), up(x.ke)
        o = torch.empty(x.S, x.S_kv, dtype=torch.float32, device=dev)
        st = timer.measure(lambda: dg.fp8_mqa_logits(q, (kv, sf), w, ks, ke, True, out=o))
        pairs = int(np.clip(x.ke, 0, x.S_kv).astype(np.int64).sum()
                    - np.clip(x.ks, 0, x.S_kv).astype(np.int64).sum())
        flop = 2.0 * x.H * x.D * pairs
        byts = x.q.nbytes + x.kv.nbytes + x.kv_sf.nbytes + x.weights.nbytes + 8 * x.S + 4 * x.S * x.S_kv
        out[name] = entry(st, flop, byts, "mfma", pairs=pairs)
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


def bench_cast(dg, dev, timer):
    """HIP-event times of the casting kernels on bf16 operands of the GEMM
    workloads' shapes (inputs resident in HBM), against the HBM roof."""
    print("[bench] detail: cast", file=sys.stderr, flush=True)
    import torch
    out = {}
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    for name, (per_block, shape) in CAST_WORKLOADS.items():
        x = torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        fn = dg.per_block_cast_to_fp8 if per_block else dg.per_token_cast_to_fp8
        codes, sf = fn(x)
        st = timer.measure(lambda: fn(x, out=(codes, sf)))
        byts = cast_bytes(per_block, shape)
        out[name] = entry(st, 0.0, byts, "hbm", bytes=byts)
        del x, codes, sf
        torch.cuda.empty_cache()
    return out


def cpu_model() -> str:
    """The host CPU's model name (lscpu), for the CPU-baseline record."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    return "unknown"


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
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{n} of {M} rows of the dense {M}x{N}x{K} shape (all {N} columns), "
                      f"{t:.1f} s, fp64 exact block sums"}


if __name__ == "__main__":
    main()
