"""Benchmark of the MoE-layer megakernel on one MI355X.

A step is one forward of the whole layer (router, top-k, histogram/scan, grouping, both
GroupGEMMs, combine) over one batch of synthetic inputs already resident in HBM.  The
default workload is the Mixtral-shaped decode layer (B=32, d=4096, f=14336, E=8, k=2).
Prints one JSON line with tokens/s, the roofline of the kernel (HBM bytes or MFMA flops
of the activated experts per launch over the measured launch time) and the CPU oracle
timed on a bounded sample of the same workload.
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


def measured_traffic(cfg_name, B, sched):
    """HBM bytes per launch from the committed rocprofv3 byte-counter summary of this workload,
    or None when there is none or the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"megakernel_{cfg_name}_B{B}_pmc.txt")
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

    flags0 = layer.debug_flags if hasattr(layer, "debug_flags") else 0
    mk.moe_mk_plan_set_debug(layer.plan, 0, flags0 | mk.MOE_MK_DEBUG_TRACE)
    layer(x, out)
    torch.cuda.synchronize()
    mk.moe_mk_plan_set_debug(layer.plan, 0, flags0)
    ctl = layer.routing(B)["ctl"].cpu().numpy()
    tr = mk.moe_mk_trace_view(layer.plan, B, layer.ws).cpu().numpy()
    E, k, d, f = layer.E, layer.k, layer.d, layer.f
    info = lambda key: mk.moe_mk_plan_info(layer.plan, key)
    waves = info("threads") // 64
    tpw = 1 if B <= 512 else 8 if E % 4 == 0 and d % 128 == 0 and -(-B // 64) * -(-E // 16) >= 512 else 4
    reb = 4 if tpw == 1 and E % 4 == 0 and d % 512 == 0 and -(-B // waves) * -(-E // 16) < 64 else 16
    nR = -(-B // (waves * tpw)) * -(-E // reb)
    T = -(-B // 64)
    mt = int(ctl[mk.CTL["mt_total"]])
    a = B * k
    if a >= info("wide_min_rows") * E and d % info("wide_BN2") == 0 and f % info("wide_BN1") == 0:
        S, nb1, nb2 = 1, f // info("wide_BN1"), d // info("wide_BN2")
    else:
        nb1, nb2 = f // info("BN1"), d // info("BN2")
        S = 4 if (a <= 1024 and f >= 8192 and nb1 % 4 == 0) else 2 if (a <= 1024 and f >= 4096 and nb1 % 2 == 0) else 1
    # GroupGEMM blocks are padded to multiples of 8 task positions (empty tasks leave no record)
    r8 = lambda v: (v + 7) // 8 * 8
    total = r8(nR + 2 * T + 1) + S * (r8(mt * nb1 // S) + r8(mt * nb2)) + -(-B // (8 if B >= 1024 and k <= 8 else 1 if B <= 64 else 4)) * -(-d // (4 * info("threads")))
    tr = tr[:total]
    tr = tr[tr[:, 1] != 0]
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
          f"90th percentile {us(np.percentile(first, 90)):.1f}, max {us(first.max()):.1f} "
          f"(router tasks: {', '.join(f'{us(v - t0):.1f}' for v in sorted(tr[kind == 0, 1])[:8])})", file=sys.stderr)
    xcc = tr[:, 5]
    print(f"#  XCD of a task equals its workgroup index mod 8 for {100.0 * np.mean(xcc == wg % 8):.1f}% of tasks",
          file=sys.stderr)
    # time between a workgroup finishing one task and obtaining the next (queue / loop overhead)
    gaps = []
    for w in set(wg.tolist()):
        r = tr[wg == w]
        r = r[np.argsort(r[:, 1])]
        if len(r) > 1:
            gaps.append(r[1:, 1] - r[:-1, 3])
    if gaps:
        gaps = np.concatenate(gaps)
        print(f"#  between tasks: mean {us(gaps.mean()):.2f} us, max {us(gaps.max()):.1f} us", file=sys.stderr)
    del np


def main():
    args = parse()
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
    base_flags = mk.MOE_MK_DEBUG_NO_PREFETCH if args.no_prefetch else 0
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

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        layer(tx, out)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if layer.error():
        raise RuntimeError(f"device error word {layer.error()}")
    per_launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    kern_ms = float(np.mean(per_launch_ms))
    ms_per_step = wall * 1e3 / args.steps
    tokens_per_s = B / (ms_per_step / 1e3)
    gbs = alg_bytes / (kern_ms / 1e3) / 1e9
    tflops = flops / (kern_ms / 1e3) / 1e12
    prefill = B >= 2048
    if prefill:
        roof = {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": tflops / PEAK_BF16_TFLOPS, "traffic": measured_traffic(cfg.name, B, args.sched)}
    else:
        roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": gbs / PEAK_HBM_GBS, "traffic": measured_traffic(cfg.name, B, args.sched)}
    line = {
        "metric": "MoE-layer tokens/s + achieved HBM TB/s (B<=64) / MFMA TFLOP/s (B>=2048) vs peak",
        "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.note, "B": B, "d": cfg.d, "f": cfg.f, "E": cfg.E, "k": cfg.k,
                   "sched": args.sched, "active_experts": active},
        "roofline": roof,
        "kernel_ms": kern_ms, "kernel_ms_min": float(np.min(per_launch_ms)),
        "hbm_tbs": gbs / 1e3, "hbm_frac": gbs / PEAK_HBM_GBS,
        "mfma_tflops": tflops, "mfma_frac": tflops / PEAK_BF16_TFLOPS,
        "algorithmic_bytes": alg_bytes, "gemm_flops": flops,
        "grid": mk.moe_mk_plan_info(layer.plan, "grid"),
        "cpu_baseline": None,
    }
    if args.trace:  # first, while nothing else has run on the device since the timed launches
        trace_report(layer, tx, out, B)
    if args.flush:
        # the same launches, each after a 1 GiB read (or write) of a scratch buffer that evicts
        # the Infinity Cache, so the weights come from HBM even where the activated ones would
        # fit in the cache
        scratch = torch.ones((1 << 30) // 4, dtype=torch.float32, device=dev)
        sink = torch.empty(1, dtype=torch.float32, device=dev)
        cold_ms = []
        for i in range(min(args.steps, 10)):
            if args.flush == "write":
                scratch.fill_(float(i))
            else:
                torch.sum(scratch, dim=0, keepdim=True, out=sink)
            s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s0.record(stream)
            layer(tx, out)
            e0.record(stream)
            torch.cuda.synchronize()
            cold_ms.append(s0.elapsed_time(e0))
        del scratch, sink
        cms = float(np.median(cold_ms))
        line["cold"] = {"flush": args.flush, "kernel_ms_median": cms, "kernel_ms_min": float(np.min(cold_ms)),
                        "hbm_frac": alg_bytes / (cms / 1e3) / 1e9 / PEAK_HBM_GBS,
                        "mfma_frac": flops / (cms / 1e3) / 1e12 / PEAK_BF16_TFLOPS}
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
    layer.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
