"""Benchmark of the MoE-layer megakernel on one MI355X.

A step is one forward of the whole layer (router, top-k, histogram/scan, grouping, both
GroupGEMMs, combine) over one batch of synthetic inputs already resident in HBM.  The
headline workload (`value`) is the Mixtral-shaped decode layer (B=32, d=4096, f=14336,
E=8, k=2).  The same JSON line lists every other configuration under `workloads`: the
prefill-sized layer (B=4096, MFMA roofline) and the DeepSeek-shaped skewed layer on both
schedules, the six batches of the dynamic-shape sweep on one plan, and the tiny layer.
Each carries the kernel time, its roofline fraction (HBM bytes of the activated experts
per launch, or GroupGEMM flops, over the measured launch time), the HBM traffic from the
committed rocprofv3 counter summary when it was taken on the current kernel source, and
for B <= 64 the launch time after evicting the Infinity Cache.  The CPU oracle is timed
on a bounded sample of the headline workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="mixtral_decode")
    ap.add_argument("--batch", type=int, default=0, help="batch size (default: the configuration's first)")
    ap.add_argument("--sched", default="dynamic", choices=["static", "dynamic"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--policy", default="by_rows", choices=["by_rows", "narrow_only", "batch_rule", "grouped_gate_up"],
                    help="tile policy of the headline run (the library's own choice by default; the others are "
                    "A/B comparisons)")
    ap.add_argument("--no-prefetch", action="store_true", help="turn off the weight prefetch during routing")
    ap.add_argument("--cpu-sample", type=int, default=0, help="tokens of the oracle sample (default: auto)")
    ap.add_argument("--trace", action="store_true", help="after timing, run one traced forward and print "
                    "per-task-kind timings to stderr")
    ap.add_argument("--copy-kernel", action="store_true",
                    help="after timing, run one 1 GiB device copy (reference for the HBM byte counters)")
    ap.add_argument("--flush", choices=["read", "write"], default=None,
                    help="also time launches each preceded by a 1 GiB read (or write) of a scratch buffer, "
                    "which evicts the Infinity Cache; reported under 'cold' (a write also leaves its dirty "
                    "lines to be written back during the next launch)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip measuring the box's achievable copy bandwidth and bf16 GEMM rate")
    ap.add_argument("--summarize", choices=["stats", "pmc", "mfma"], default=None,
                    help="write the profiles/ summary of rocprofv3 output under --prof-dir (no GPU use)")
    ap.add_argument("--prof-dir", default=None)
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache launches of a B <= 64 workload")
    ap.add_argument("--no-unfused", action="store_true",
                    help="skip the comparison with the same layer as one kernel per phase (plain and graph)")
    ap.add_argument("--workloads", default="all",
                    help="configurations timed beside the headline one: 'all', 'none', or a comma list of "
                    "config:sched[:policy] (e.g. prefill:static,sweep:dynamic,prefill:static:narrow_only)")
    return ap.parse_args()


def algorithmic(cfg, B, hist, with_bias):
    """Bytes the layer must move and GroupGEMM flops, from the actual routing."""
    active = int((hist > 0).sum())
    weights = 6 * cfg.d * cfg.f * active            # W1, W3, W2 bf16 of every activated expert
    other = 4 * cfg.d * cfg.E + 4 * B * cfg.d + (4 * cfg.E if with_bias else 0)  # Wr fp32, x and out bf16
    flops = 6 * B * cfg.k * cfg.d * cfg.f
    return weights + other, flops, active


def cpu_baseline(cfg, x, Wr, bias, weights, sample, min_seconds=10.0, max_reps=20):
    """The oracle as it stands, on a bounded sample of the same workload (repeated to ~10 s)."""
    import oracle

    cores = oracle.num_threads()
    B = x.shape[0]
    n = min(B, sample)
    toks = list(range(n))
    reps, t0 = 0, time.perf_counter()
    while True:
        r = oracle.routing(x[:n], Wr, bias, cfg.k)
        oracle.moe_tokens(x, toks, r["topk_idx"], r["topk_w"], weights, cfg.d, cfg.f)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or reps >= max_reps:
            break
    return {"value": reps * n / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} of {B} tokens of the same workload (router, top-k, grouping, fp64 SwiGLU experts, "
                      f"combine) x {reps} repetitions = {dt:.1f} s on {cores} OpenMP threads"}


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in ("megakernel.hip", "mk_common.h", "mk_device.h"):
        with open(os.path.join(ROOT, "moe_groupgemm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def profile_path(cfg_name, B, sched, kind):
    return os.path.join(ROOT, "profiles", f"megakernel_{cfg_name}_B{B}_{sched}_{kind}.txt")


def measured_traffic(cfg_name, B, sched):
    """HBM bytes per launch from the committed rocprofv3 byte-counter summary of this workload,
    or None when there is none or the kernel source changed since the counters were taken."""
    path = profile_path(cfg_name, B, sched, "pmc")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for ln in fh:
            if ": " in ln and not ln.startswith(" "):
                key, val = ln.split(": ", 1)
                kv[key.strip()] = val.strip()
    if kv.get("kernel_source_sha256") != kernel_source_hash() or kv.get("sched") != sched:
        return None
    return float(kv["traffic_bytes_per_launch"])


# ------------------------------------------------------------------------------ profile summaries
# The committed summaries under profiles/ are written from rocprofv3 CSV output by
# `python3 bench.py --summarize stats|pmc|mfma --prof-dir DIR --config C --batch B --sched S`,
# where DIR holds the output of the rocprofv3 commands each summary quotes (run from the
# repository root on the GPU machine; <repo> stands for that root).

def _prof_cmd(args, what):
    run = (f"python3 <repo>/bench.py --config {args.config} --batch {args.batch} --sched {args.sched} "
           f"--no-cpu-baseline --no-peaks --no-unfused --no-cold --workloads none")
    d = f"<repo>/gpurun_out/prof_{args.config}_B{args.batch}_{args.sched}"
    if what == "stats":
        return (f"cd /tmp && export TMPDIR=/tmp && timeout -k 10 300 rocprofv3 --kernel-trace --stats -d {d}/stats "
                f"-o p --output-format csv -- {run} --steps 20 --warmup 3")
    if what == "mfma":
        return (f"cd /tmp && export TMPDIR=/tmp && timeout -s KILL 150 rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES "
                f"SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE -d {d}/mfma -o p --output-format csv "
                f"-- {run} --steps 3 --warmup 1")
    return (f"cd /tmp && export TMPDIR=/tmp && timeout -s KILL 150 rocprofv3 --pmc {what} -d {d}/{what.lower()} "
            f"-o p --output-format csv -- {run} --steps 3 --warmup 1 --copy-kernel")


def _csv_rows(directory, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _per_dispatch(rows, kernel, counter, largest=False):
    """Mean over the dispatches of `kernel` of the summed value of `counter` (or the largest
    dispatch's value: the 1 GiB calibration copy among the smaller input uploads)."""
    per = {}
    for r in rows:
        if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter:
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        return None, 0
    if largest:
        return max(per.values()), 1
    return sum(per.values()) / len(per), len(per)


def summarize(args):
    name = f"megakernel_{args.config}_B{args.batch}_{args.sched}"
    lines = [f"# rocprofv3 {args.summarize}: {name}", "", "commands (from the repository root):"]
    kern = "moe_megakernel"
    if args.summarize == "stats":
        lines.append("  " + _prof_cmd(args, "stats"))
        rows = _csv_rows(os.path.join(args.prof_dir, "stats"), "kernel_stats.csv")
        lines += ["", '"Name","Calls","AverageNs","MinNs","MaxNs"']
        avg = None
        for r in rows:
            lines.append(f'"{r["Name"]}",{r["Calls"]},{float(r["AverageNs"]):.1f},{r["MinNs"]},{r["MaxNs"]}')
            if kern in r["Name"]:
                avg = float(r["AverageNs"]) / 1e3
        lines += ["", f"megakernel_avg_us: {avg:.2f}"]
    elif args.summarize == "pmc":
        lines += ["  " + _prof_cmd(args, "FETCH_SIZE"), "  " + _prof_cmd(args, "WRITE_SIZE"),
                  "  (--copy-kernel adds one 1 GiB device-to-device copy whose counter readings calibrate the scale)"]
        fr = _csv_rows(os.path.join(args.prof_dir, "fetch_size"), "counter_collection.csv")
        wr = _csv_rows(os.path.join(args.prof_dir, "write_size"), "counter_collection.csv")
        f_kib, nf = _per_dispatch(fr, kern, "FETCH_SIZE")
        w_kib, nw = _per_dispatch(wr, kern, "WRITE_SIZE")
        cf, _ = _per_dispatch(fr, "copyBuffer", "FETCH_SIZE", largest=True)
        cw, _ = _per_dispatch(wr, "copyBuffer", "WRITE_SIZE", largest=True)
        # the 1 GiB copy reads and writes 1 GiB: the counters' KiB readings for it give the scales
        fs, ws = (1 << 20) / cf, (1 << 20) / cw
        traffic = (f_kib * fs + w_kib * ws) * 1024
        lines += ["", f"megakernel FETCH_SIZE KiB per dispatch (mean of {nf}): {f_kib:.3f}",
                  f"megakernel WRITE_SIZE KiB per dispatch (mean of {nw}): {w_kib:.3f}",
                  f"1 GiB copy FETCH_SIZE KiB: {cf:.3f}  -> fetch scale {fs:.5f}",
                  f"1 GiB copy WRITE_SIZE KiB: {cw:.3f}  -> write scale {ws:.5f}",
                  f"read bytes per launch: {f_kib * fs * 1024:.0f}", f"written bytes per launch: {w_kib * ws * 1024:.0f}",
                  f"sched: {args.sched}", f"traffic_bytes_per_launch: {traffic:.0f}",
                  f"kernel_source_sha256: {kernel_source_hash()}"]
    else:
        lines.append("  " + _prof_cmd(args, "mfma"))
        rows = _csv_rows(os.path.join(args.prof_dir, "mfma"), "counter_collection.csv")
        vals = {c: _per_dispatch(rows, kern, c) for c in ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                                                           "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE")}
        busy, mops, gui = (vals[c][0] for c in ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                                                "GRBM_GUI_ACTIVE"))
        lines += ["", f"per dispatch of the megakernel (mean of {vals['GRBM_GUI_ACTIVE'][1]}; summed over XCDs and SIMDs):"]
        lines += [f"  {c:30s} {v[0]:.0f}" for c, v in vals.items()]
        # GRBM_GUI_ACTIVE sums the 8 XCDs' busy cycles; 1024 SIMDs issue MFMAs
        durs = {}
        for r in rows:
            if kern in r["Kernel_Name"]:
                durs[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        dur = sum(durs.values()) / len(durs)
        lines += [f"  dispatch duration under the profiler: {dur:.1f} us (mean)",
                  f"  clock while the kernel runs: {gui / 8 / dur / 1e3:.2f} GHz (GUI-active cycles per XCD / duration)",
                  f"  MFMA busy fraction (busy cycles / (GUI-active cycles per XCD x 1024 SIMDs)): "
                  f"{busy / (gui / 8 * 1024):.3f}",
                  f"  issued bf16 MFMA work: {mops * 512 / 1e9:.1f} GFLOP (MOPS x 512)",
                  f"kernel_source_sha256: {kernel_source_hash()}"]
    out = profile_path(args.config, args.batch, args.sched, args.summarize)
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(out)


def copy_calibration(nbytes=1 << 30):
    """One plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1.0)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    return nbytes


def achievable_peaks(dev, reps=10):
    """What this machine reaches on plain library work: a 1 GiB device-to-device copy (bytes read
    plus written per second) and an 8192^3 bf16 matrix product (hipBLASLt through torch)."""
    import torch
    n = 1 << 30
    a = torch.ones(n // 2, dtype=torch.bfloat16, device=dev)
    b = torch.empty_like(a)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    copy_gbs = 2.0 * n * reps / (s.elapsed_time(e) / 1e3) / 1e9
    del a, b
    m = 8192
    x = torch.randn(m, m, dtype=torch.bfloat16, device=dev)
    y = torch.randn(m, m, dtype=torch.bfloat16, device=dev)
    z = torch.empty(m, m, dtype=torch.bfloat16, device=dev)
    for _ in range(2):
        torch.mm(x, y, out=z)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        torch.mm(x, y, out=z)
    e.record()
    torch.cuda.synchronize()
    gemm_tflops = 2.0 * m ** 3 * reps / (s.elapsed_time(e) / 1e3) / 1e12
    del x, y, z
    torch.cuda.empty_cache()
    return copy_gbs, gemm_tflops


def trace_report(layer, x, out, B):
    """One forward with per-task timestamps; per-kind summary on stderr (microseconds)."""
    import numpy as np
    import torch

    import moe_groupgemm_amd as mk

    flags0 = getattr(layer, "debug_flags", 0)
    view = mk.moe_mk_trace_view(layer.plan, B, layer.ws)
    view.zero_()  # records left from earlier traced forwards would look like tasks of this one
    mk.moe_mk_plan_set_debug(layer.plan, 0, flags0 | mk.MOE_MK_DEBUG_TRACE)
    layer(x, out)
    torch.cuda.synchronize()
    mk.moe_mk_plan_set_debug(layer.plan, 0, flags0)
    tr = view.cpu().numpy()
    tr = tr[tr[:, 1] != 0]  # tasks that ran (padding positions of the static layout leave no record)
    kind = (tr[:, 0] >> 32) & 0xFF
    wg = tr[:, 0] >> 40
    t0 = tr[:, 1].min()
    us = lambda v: v / 100.0  # 100 MHz ticks -> microseconds
    print(f"# trace: {len(tr)} tasks, {len(set(wg.tolist()))} workgroups, span {us(tr[:, 3].max() - t0):.1f} us",
          file=sys.stderr)
    for kd, name in enumerate(mk.TASK_KINDS):
        m = kind == kd
        if not m.any():
            continue
        wait = tr[m, 2] - tr[m, 1]
        body = tr[m, 4] - tr[m, 2]
        tail = tr[m, 3] - tr[m, 4]
        print(f"#  {name:8s} n={int(m.sum()):6d} start {us(tr[m, 1].min() - t0):7.1f} ready {us(tr[m, 2].min() - t0):7.1f} "
              f"end {us(tr[m, 3].max() - t0):7.1f} | wait {us(wait.mean()):6.2f} (max {us(wait.max()):6.1f}) | "
              f"body {us(body.mean()):7.2f} (max {us(body.max()):6.1f}) | notify {us(tail.mean()):5.2f}",
              file=sys.stderr)
    fused = (kind == 1) & (tr[:, 6] != 0)
    for r in tr[fused]:  # top-k task that also scans and groups (one routing tile)
        print(f"#  top-k tail: scan {us(r[6] - r[4]):.2f} us, grouping and pushes {us(r[7] - r[6]):.2f}, "
              f"notify {us(r[3] - r[7]):.2f}", file=sys.stderr)
    first = np.array([tr[wg == w, 1].min() for w in sorted(set(wg.tolist()))]) - t0
    print(f"#  first task of a workgroup obtained at: median {us(np.median(first)):.1f} us, "
          f"90th percentile {us(np.percentile(first, 90)):.1f}, max {us(first.max()):.1f}", file=sys.stderr)
    xcc = tr[:, 5]
    print(f"#  XCD of a task equals its workgroup index mod 8 for {100.0 * np.mean(xcc == wg % 8):.1f}% of tasks",
          file=sys.stderr)
    gaps = []  # time between a workgroup finishing one task and obtaining the next
    for w in set(wg.tolist()):
        r = tr[wg == w]
        r = r[np.argsort(r[:, 1])]
        if len(r) > 1:
            gaps.append(r[1:, 1] - r[:-1, 3])
    if gaps:
        gaps = np.concatenate(gaps)
        print(f"#  between tasks: mean {us(gaps.mean()):.2f} us, max {us(gaps.max()):.1f} us", file=sys.stderr)


def time_launches(layer, tx, out, stream, steps):
    """Per-launch kernel times (ms) from HIP events recorded on the launch stream."""
    import torch
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        layer(tx, out)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [s.elapsed_time(e) for s, e in zip(starts, ends)], wall


def time_cold(layer, tx, out, stream, reps, flush, dev):
    """Launch times (ms) each after evicting the Infinity Cache by a 1 GiB read (or write)."""
    import torch
    scratch = torch.ones((1 << 30) // 4, dtype=torch.float32, device=dev)
    sink = torch.empty(1, dtype=torch.float32, device=dev)
    ms = []
    for i in range(reps):
        if flush == "write":
            scratch.fill_(float(i))
        else:
            torch.sum(scratch, dim=0, keepdim=True, out=sink)
        s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        layer(tx, out)
        e0.record(stream)
        torch.cuda.synchronize()
        ms.append(s0.elapsed_time(e0))
    del scratch, sink
    return ms


def roofline(cfg_name, B, sched, alg_bytes, flops, kern_ms, policy="by_rows"):
    """Roofline of the launch: MFMA for prefill-sized batches (B >= 2048), else HBM.  The
    counter traffic comes from the profiles of the library's own tile choice ('by_rows'), so
    it is null for the comparison policies."""
    gbs = alg_bytes / (kern_ms / 1e3) / 1e9
    tflops = flops / (kern_ms / 1e3) / 1e12
    traffic = measured_traffic(cfg_name, B, sched) if policy == "by_rows" else None
    if B >= 2048:
        return {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": tflops / PEAK_BF16_TFLOPS, "traffic": traffic}
    return {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
            "traffic": traffic}


# MOE_MK_DEBUG_* flags; 'grouped_gate_up' keeps the gate/up tiles on grouped rows where the library
# would run them over all tokens from the start of the forward (forward_info "all_token_gate_up")
TILE_POLICIES = {"by_rows": 0, "narrow_only": 8, "batch_rule": 16, "grouped_gate_up": 32}


def measure_workload(cfg_name, sched_name, steps, warmup, dev, batches=None, cold_reps=10, policy="by_rows"):
    """Time the layer of one configuration (each of its batches on one plan and workspace).
    policy: the row-tile shape of each expert chosen from its row count ('by_rows', the
    library's default), narrow for every expert ('narrow_only'), or chosen from the batch size alone
    ('batch_rule': every expert wide when B*k >= 128*E) for comparison."""
    import numpy as np
    import torch

    import moe_groupgemm_amd as mk
    from moe_inputs import CONFIGS, device_weights, make_x, to_torch_bf16

    cfg = CONFIGS[cfg_name]
    batches = batches or cfg.batches
    sched = mk.MOE_MK_SCHED_STATIC if sched_name == "static" else mk.MOE_MK_SCHED_DYNAMIC
    print(f"# workload {cfg_name} {sched_name} {policy} B={list(batches)}", file=sys.stderr, flush=True)
    tWr, tb, t1, t3, t2 = device_weights(cfg, device=dev)
    tx_all = to_torch_bf16(make_x(cfg, max(batches))).to(dev)
    layer = mk.MoELayer(cfg.E, cfg.k, cfg.d, cfg.f, tWr, t1, t3, t2, router_bias=tb, sched=sched,
                        max_batch=max(batches), device=dev)
    mk.moe_mk_plan_set_debug(layer.plan, 0, TILE_POLICIES[policy])
    stream = torch.cuda.current_stream(dev)
    res = []
    for B in batches:
        tx = tx_all[:B]
        out = torch.empty((B, cfg.d), dtype=torch.bfloat16, device=dev)
        for _ in range(warmup):
            layer(tx, out)
        torch.cuda.synchronize()
        if layer.error():
            raise RuntimeError(f"device error word {layer.error()} ({cfg_name} B={B} {sched_name})")
        hist = layer.routing(B)["hist"].cpu().numpy()
        alg_bytes, flops, active = algorithmic(cfg, B, hist, tb is not None)
        ms, _ = time_launches(layer, tx, out, stream, steps)
        if layer.error():
            raise RuntimeError(f"device error word {layer.error()} ({cfg_name} B={B} {sched_name})")
        kern_ms = float(np.mean(ms))
        ctl = layer.routing(B)["ctl"].cpu().numpy()
        e = {"workload": cfg.note, "config": cfg_name, "B": B, "sched": sched_name, "tile_policy": policy,
             "row_tiles": int(ctl[mk.CTL["mt_total"]]), "wide_row_tiles": int(ctl[mk.CTL["mw"]]),
             "all_token_gate_up": bool(mk.moe_mk_forward_info(layer.plan, B, "all_token_gate_up"))
             and not TILE_POLICIES[policy] & mk.MOE_MK_DEBUG_GROUPED_GATE_UP,
             "active_experts": active,
             "kernel_ms": kern_ms, "kernel_ms_min": float(np.min(ms)), "tokens_per_s": B / (kern_ms / 1e3),
             "roofline": roofline(cfg_name, B, sched_name, alg_bytes, flops, kern_ms, policy),
             "hbm_frac": alg_bytes / (kern_ms / 1e3) / 1e9 / PEAK_HBM_GBS,
             "mfma_frac": flops / (kern_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
             "algorithmic_bytes": alg_bytes, "gemm_flops": flops}
        if B <= 64 and cold_reps:
            cms = float(np.median(time_cold(layer, tx, out, stream, cold_reps, "read", dev)))
            e["cold"] = {"flush": "read", "kernel_ms_median": cms,
                         "hbm_frac": alg_bytes / (cms / 1e3) / 1e9 / PEAK_HBM_GBS}
        res.append(e)
        print(f"#   B={B}: {kern_ms * 1e3:.1f} us, {e['roofline']['bound']} {e['roofline']['frac']:.3f}",
              file=sys.stderr, flush=True)
    layer.close()
    del layer, tWr, tb, t1, t3, t2, tx_all
    torch.cuda.empty_cache()
    return res


def unfused_comparison(cfg_name, steps, warmup, dev, batches=None):
    """The megakernel (both schedules) beside the same layer as seven kernels, one per phase,
    launched plainly and replayed from a HIP graph; and the warm-up each approach needs per
    batch size (a graph must be captured and instantiated for every B; the megakernel needs
    nothing).  Kernel-side times come from HIP events around each forward on its stream."""
    import numpy as np
    import torch

    import moe_groupgemm_amd as mk
    from moe_inputs import CONFIGS, device_weights, make_x, to_torch_bf16

    cfg = CONFIGS[cfg_name]
    batches = batches or cfg.batches
    print(f"# unfused comparison {cfg_name} B={list(batches)}", file=sys.stderr, flush=True)
    tWr, tb, t1, t3, t2 = device_weights(cfg, device=dev)
    tx_all = to_torch_bf16(make_x(cfg, max(batches))).to(dev)
    layers = {name: mk.MoELayer(cfg.E, cfg.k, cfg.d, cfg.f, tWr, t1, t3, t2, router_bias=tb, sched=sc,
                                max_batch=max(batches), device=dev)
              for name, sc in (("static", mk.MOE_MK_SCHED_STATIC), ("dynamic", mk.MOE_MK_SCHED_DYNAMIC))}
    stream = torch.cuda.current_stream(dev)

    def timed(fn, n):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3

    res = []
    for B in batches:
        tx = tx_all[:B]
        out = torch.empty((B, cfg.d), dtype=torch.bfloat16, device=dev)
        lay = layers["dynamic"]
        for _ in range(warmup):
            layers["static"](tx, out)
            lay(tx, out)
            lay.forward_unfused(tx, out)
        torch.cuda.synchronize()
        e = {"config": cfg_name, "B": B,
             "megakernel_static_us": timed(lambda: layers["static"](tx, out), steps),
             "megakernel_dynamic_us": timed(lambda: lay(tx, out), steps),
             "unfused_us": timed(lambda: lay.forward_unfused(tx, out), steps)}
        # warm-up of the graph approach at this B: capture and instantiate, then the first replay
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            lay.forward_unfused(tx, out)
        t1c = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        e["unfused_graph_capture_ms"] = (t1c - t0) * 1e3
        e["unfused_graph_first_replay_ms"] = (time.perf_counter() - t1c) * 1e3
        e["unfused_graph_us"] = timed(g.replay, steps)
        del g
        # the megakernel at a batch size it has not run yet needs no capture: its first call
        # is an ordinary launch (wall time to completion, host included)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        layers["static"](tx, out)
        torch.cuda.synchronize()
        e["megakernel_call_ms"] = (time.perf_counter() - t0) * 1e3
        if lay.error() or layers["static"].error():
            raise RuntimeError(f"device error in the unfused comparison ({cfg_name} B={B})")
        res.append(e)
        print(f"#   B={B}: megakernel {e['megakernel_static_us']:.1f} / {e['megakernel_dynamic_us']:.1f} us, "
              f"unfused {e['unfused_us']:.1f} us, graph {e['unfused_graph_us']:.1f} us "
              f"(capture {e['unfused_graph_capture_ms']:.2f} ms)", file=sys.stderr, flush=True)
    for lay in layers.values():
        lay.close()
    del layers, tWr, tb, t1, t3, t2, tx_all
    torch.cuda.empty_cache()
    return res


# configurations listed beside the headline line (configuration, schedule[, tile policy]);
# the skewed and prefill-sized layers also run with each fixed row-tile shape, beside the
# per-expert choice
WORKLOADS = [("prefill", "static"), ("prefill", "dynamic"), ("prefill", "static", "narrow_only"),
             ("prefill", "static", "batch_rule"), ("deepseek_zipf", "static"), ("deepseek_zipf", "dynamic"),
             ("deepseek_zipf", "dynamic", "narrow_only"), ("deepseek_zipf", "dynamic", "batch_rule"),
             ("sweep", "static"), ("sweep", "dynamic"), ("tiny", "static"), ("tiny", "dynamic"),
             ("tiny", "static", "grouped_gate_up"), ("mixtral_decode", "static"),
             ("mixtral_decode", "dynamic", "grouped_gate_up")]


def main():
    args = parse()
    if args.summarize:
        from moe_inputs import CONFIGS
        args.batch = args.batch or CONFIGS[args.config].B
        summarize(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the layer runs on one "
              f"MI355X, with no sharding across GPUs)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import moe_groupgemm_amd as mk
    from moe_inputs import CONFIGS, all_expert_weights, make_bias, make_wr, make_x, to_torch_bf16

    cfg = CONFIGS[args.config]
    B = args.batch or cfg.B
    sched = mk.MOE_MK_SCHED_STATIC if args.sched == "static" else mk.MOE_MK_SCHED_DYNAMIC
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"# generating {cfg.name} inputs", file=sys.stderr, flush=True)
    Wr, bias = make_wr(cfg), make_bias(cfg)
    W1, W3, W2 = all_expert_weights(cfg)
    tWr = torch.from_numpy(Wr).to(dev)
    tb = None if bias is None else torch.from_numpy(bias).to(dev)
    t1, t3, t2 = (to_torch_bf16(a).to(dev) for a in (W1, W3, W2))
    x = make_x(cfg, B)
    tx = to_torch_bf16(x).to(dev)
    layer = mk.MoELayer(cfg.E, cfg.k, cfg.d, cfg.f, tWr, t1, t3, t2, router_bias=tb, sched=sched,
                        max_batch=B, device=dev)
    out = torch.empty((B, cfg.d), dtype=torch.bfloat16, device=dev)
    base_flags = (mk.MOE_MK_DEBUG_NO_PREFETCH if args.no_prefetch else 0) | TILE_POLICIES[args.policy]
    mk.moe_mk_plan_set_debug(layer.plan, 0, base_flags)
    layer.debug_flags = base_flags
    stream = torch.cuda.current_stream(dev)
    print(f"# warmup {args.warmup}, steps {args.steps}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        layer(tx, out)
    torch.cuda.synchronize()
    if layer.error():
        raise RuntimeError(f"device error word {layer.error()}")
    hist = layer.routing(B)["hist"].cpu().numpy()
    alg_bytes, flops, active = algorithmic(cfg, B, hist, tb is not None)
    per_launch_ms, wall = time_launches(layer, tx, out, stream, args.steps)
    if layer.error():
        raise RuntimeError(f"device error word {layer.error()}")
    kern_ms = float(np.mean(per_launch_ms))
    ms_per_step = wall * 1e3 / args.steps
    tokens_per_s = B / (ms_per_step / 1e3)
    gbs = alg_bytes / (kern_ms / 1e3) / 1e9
    tflops = flops / (kern_ms / 1e3) / 1e12
    line = {
        "metric": "MoE-layer tokens/s + achieved HBM TB/s (B<=64) / MFMA TFLOP/s (B>=2048) vs peak",
        "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.note, "B": B, "d": cfg.d, "f": cfg.f, "E": cfg.E, "k": cfg.k,
                   "sched": args.sched, "active_experts": active,
                   "all_token_gate_up": bool(mk.moe_mk_forward_info(layer.plan, B, "all_token_gate_up"))
                   and not base_flags & mk.MOE_MK_DEBUG_GROUPED_GATE_UP},
        "roofline": roofline(cfg.name, B, args.sched, alg_bytes, flops, kern_ms, args.policy),
        "kernel_ms": kern_ms, "kernel_ms_min": float(np.min(per_launch_ms)),
        "hbm_tbs": gbs / 1e3, "hbm_frac": gbs / PEAK_HBM_GBS,
        "mfma_tflops": tflops, "mfma_frac": tflops / PEAK_BF16_TFLOPS,
        "algorithmic_bytes": alg_bytes, "gemm_flops": flops,
        "grid": mk.moe_mk_plan_info(layer.plan, "grid"),
        "cpu_baseline": None,
    }
    if args.trace:  # first, while nothing else has run on the device since the timed launches
        trace_report(layer, tx, out, B)
    if args.flush or (B <= 64 and not args.no_cold):
        cold_ms = time_cold(layer, tx, out, stream, min(args.steps, 10), args.flush or "read", dev)
        cms = float(np.median(cold_ms))
        line["cold"] = {"flush": args.flush or "read", "kernel_ms_median": cms,
                        "kernel_ms_min": float(np.min(cold_ms)),
                        "hbm_frac": alg_bytes / (cms / 1e3) / 1e9 / PEAK_HBM_GBS,
                        "mfma_frac": flops / (cms / 1e3) / 1e12 / PEAK_BF16_TFLOPS}
    layer.close()
    del layer, t1, t3, t2
    torch.cuda.empty_cache()
    if args.workloads != "none":
        wanted = WORKLOADS if args.workloads == "all" else \
            [tuple(w.split(":")) for w in args.workloads.split(",")]
        line["workloads"] = []
        for w in wanted:
            line["workloads"].extend(measure_workload(w[0], w[1], args.steps, args.warmup, dev,
                                                      policy=w[2] if len(w) > 2 else "by_rows"))
    if not args.no_unfused:
        line["unfused"] = []
        for name in ("tiny", "sweep", "mixtral_decode", "prefill"):
            line["unfused"].extend(unfused_comparison(name, args.steps, args.warmup, dev))
    if not args.no_peaks:
        copy_gbs, gemm_tflops = achievable_peaks(dev)
        line["achievable"] = {"copy_gbs": copy_gbs, "bf16_gemm_tflops": gemm_tflops,
                              "hbm_frac_of_copy": gbs / copy_gbs, "mfma_frac_of_gemm": tflops / gemm_tflops}
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        sample = args.cpu_sample or max(1, min(B, int(2.0e10 / (6 * cfg.k * cfg.d * cfg.f))))
        line["cpu_baseline"] = cpu_baseline(cfg, x, Wr, bias, (W1, W3, W2), sample)
    if args.copy_kernel:
        line["copy_kernel_bytes"] = copy_calibration()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
