#!/usr/bin/env python3
"""Benchmark of the hot path on one MI355X: prints ONE JSON line.

A step is one pass of the whole hot path over one batch of synthetic input:
one fp32 GEMM + bias + ReLU (M = N = K = 4096, uniform[-1,1), 2-stage ring,
default launch configuration) and one LDS-staged copy of 1 GiB of fp32
(64 KiB tiles, 2-stage ring). Inputs are generated on the host, copied to
HBM and resident before timing starts.

First an untimed settle phase: hot-path steps until --settle-ms (default
200) of wall time have passed, so that the GPU has left the low clocks of
its idle state before anything is timed (reported as `settle`). Then W
untimed warmup steps, then K timed steps. The GEMMs and the copies are
timed as two back-to-back regions, each bracketed by torch.cuda.synchronize()
(and HIP events on the launch stream for the per-launch kernel durations):
  value                = GEMM TFLOP/s over its timed region (2*M*N*K per launch)
  copy.value           = copy GB/s over its timed region (2 * bytes per launch)
  roofline             = the GEMM kernel against the fp32 MFMA peak
  copy_roofline        = the copy kernel against the HBM peak
  cpu_baseline         = the CPU oracle on a bounded sample of the same GEMM
                         (its rows also give `parity`)
  copy_cpu_baseline    = the copy oracle (a multi-threaded host memcpy of the
                         same 1 GiB), median of its calls
  copy.parity          = the timed copy configuration's output against its
                         source on the GPU and against the oracle's copy on
                         the host, byte for byte (outside the timed regions)
  homogeneous_baseline = the same GEMM, tile and ring depth on the kernel
                         without roles (every wave loads, barrier, computes)
  vendor_library       = the same GEMM through torch (relu_(addmm), hipBLASLt)
                         in the input dtype, for context; two launches, so
                         its figure includes a separate ReLU pass
  copy.plain_device_copy = torch's own device-to-device copy of the same
                         buffers
  copy.direct_baseline = this library's unstaged copy of the same buffers
                         (no LDS ring, no roles), the ablation of staging
  ring_depth_2         = for a workload whose ring depth is above 2 (bf16
                         8192^3: S = 4), the same GEMM through the default
                         configuration of a 2-slot ring, for context
Each comparison leg first runs --leg-settle-ms (default 100) of untimed
launches of its own kernel, then the warmup steps.
Options select other workloads (--workload 4: ragged fp32, --workload 5:
bf16 8192^3, --moe: a mixture-of-experts expert layer on the grouped GEMM,
--attention: attention forward)
or a launch configuration (--stages, --bm/--bn/--bk,
--producers, --consumers); --sweep prints one line per stage/producer point.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"fp32": 157.3, "bf16": 2516.6}  # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "gemm": ["warp_specialized_gemm_amd/csrc/gemm_bias_relu.hip", "warp_specialized_gemm_amd/csrc/ring.hpp",
             "warp_specialized_gemm_amd/csrc/tiles.hpp"],
    "copy": ["warp_specialized_gemm_amd/csrc/staged_copy.hip", "warp_specialized_gemm_amd/csrc/ring.hpp"],
    "attention": ["warp_specialized_gemm_amd/csrc/attention.hip", "warp_specialized_gemm_amd/csrc/ring.hpp",
                  "warp_specialized_gemm_amd/csrc/tiles.hpp"],
}


def source_hash(kind: str) -> str:
    """Hash of the kernel sources' code: line comments and blank lines do not count, so an edit
    to the prose alone keeps the measured traffic figures current."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(key: str, kind: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if still current."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f).get(key)
    except (OSError, ValueError):
        return None
    if not t or t.get("source_hash") != source_hash(kind):
        return None
    return t.get("bytes_per_launch")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def make_gemm_inputs(wid: int):
    import numpy as np
    import synth
    w = synth.WORKLOADS[wid]
    M, N, K = w["M"], w["N"], w["K"]
    if w["dtype"] == "fp32":
        A = synth.uniform_pm1(synth.seed_for(wid, "A"), M * K).reshape(M, K)
        B = synth.uniform_pm1(synth.seed_for(wid, "B"), K * N).reshape(K, N)
        bias = synth.uniform_pm1(synth.seed_for(wid, "bias"), N)
    else:
        A = synth.normal_bf16_bits(synth.seed_for(wid, "A"), M * K).reshape(M, K)
        B = synth.normal_bf16_bits(synth.seed_for(wid, "B"), K * N).reshape(K, N)
        bias = synth.normal_bf16_bits(synth.seed_for(wid, "bias"), N)
    return w, A, B, bias


def gemm_launcher(wsg, w, dA, dB, dbias, dC, stages, config):
    if w["dtype"] == "fp32" and config is None:
        return lambda: wsg.gemm_bias_relu(dA, dB, dbias, dC, stages=stages)
    if w["dtype"] == "bf16" and config is None:
        return lambda: wsg.gemm_bias_relu_bf16(dA, dB, dbias, dC, stages=stages)
    return lambda: wsg.gemm_bias_relu_ex(dA, dB, dbias, dC, stages=stages, config=config)


def time_region(torch, fn, steps: int):
    """Wall time of `steps` launches between two synchronizations, and the
    mean per-launch kernel time from HIP events on the launch stream."""
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [a.elapsed_time(b) / 1e3 for a, b in ev]
    LAST_MEDIAN[0] = sorted(per)[len(per) // 2]
    return wall, sum(per) / len(per), min(per)


LAST_MEDIAN = [0.0]  # median per-launch kernel time of the latest time_region call


def warm_leg(torch, fn, args) -> None:
    """Untimed launches of a comparison leg before it is timed: its own settle
    phase (--leg-settle-ms) and the warmup steps. A leg that follows another
    kernel needs more than a few launches: on MI355X hipBLASLt's bf16 GEMM
    read ~1170 TFLOP/s over its first 20 timed launches after 3 warmups and
    ~1310 over the next 20, and kernels after a host pause start at a lower
    clock."""
    settle(torch, fn, args.leg_settle_ms)
    for _ in range(args.warmup):
        fn()


def settle(torch, fn, min_ms: float) -> dict:
    """Untimed calls of fn, four at a time between synchronizations, until at
    least min_ms of wall time has passed with the GPU busy.

    An MI355X that has been idle (here: while the host drew the inputs) runs
    its first tens of milliseconds of work at lower clocks. Measured on one
    box with the default step: the GEMM kernel at 130.0 TFLOP/s after 3
    warmup steps against 133.3 after 30 and 133.4 after 100; bf16 8192^3 at
    968 against 1065 and 1067. Without this phase the first timed region
    (the specialized kernel) would run during that ramp while the regions
    timed after it (the baselines) ran warm."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    steps = 0
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        for _ in range(4):
            fn()
        steps += 4
        torch.cuda.synchronize()
    return {"steps": steps, "ms": round((time.perf_counter() - t0) * 1e3, 1)}


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or the platform's processor string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline_copy(src_host, budget_s: float):
    """The copy oracle (a multi-threaded host memcpy of the whole buffer) timed call by call
    until about budget_s; returns (GB/s of the median call, calls, seconds, threads, last output)."""
    import oracle
    threads = oracle.host_threads()
    times, out = [], None
    while not times or (sum(times) < budget_s and len(times) < 20):
        t0 = time.perf_counter()
        out = oracle.copy(src_host, threads=threads)
        times.append(time.perf_counter() - t0)
    med = sorted(times)[len(times) // 2]
    return 2.0 * src_host.nbytes / med / 1e9, len(times), sum(times), threads, out


def cpu_baseline_gemm(A, B, bias, budget_s: float):
    """The oracle on the first rows of the same GEMM, 16 rows at a time, until
    about budget_s of CPU work; returns (TFLOP/s, rows, seconds, threads, rows_out)."""
    import numpy as np
    import oracle
    M, K = A.shape
    N = B.shape[1]
    threads = oracle.host_threads()
    rows_done, spent, outs = 0, 0.0, []
    while rows_done < M and spent < budget_s:
        rows = np.arange(rows_done, min(M, rows_done + 16), dtype=np.int64)
        t0 = time.perf_counter()
        outs.append(oracle.gemm_bias_relu_rows(A, B, bias, rows, threads=threads))
        spent += time.perf_counter() - t0
        rows_done += rows.size
    flops = 2.0 * rows_done * N * K
    return flops / spent / 1e12, rows_done, spent, threads, np.concatenate(outs, axis=0)


def run(args):
    import numpy as np
    import torch

    import oracle
    import synth
    import warp_specialized_gemm_amd as wsg

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    w, A, B, bias = make_gemm_inputs(args.workload)
    M, N, K = w["M"], w["N"], w["K"]
    dtype = w["dtype"]
    stages = args.stages or w["stages"]
    config = None
    if any(v for v in (args.bm, args.bn, args.bk, args.producers, args.consumers, args.group_k, args.homogeneous,
                       args.flags)):
        config = dict(BM=args.bm or 0, BN=args.bn or 0, BK=args.bk or 0,
                      producer_waves=args.producers or 0, consumer_waves=args.consumers or 0,
                      group_k=args.group_k or 0,
                      flags=args.flags | (wsg.WSG_FLAG_HOMOGENEOUS if args.homogeneous else 0))
    resolved = wsg.resolve_config(wsg.WSG_FP32 if dtype == "fp32" else wsg.WSG_BF16, M, N, K, stages, config)
    log("gemm workload %d %s: %s stages=%d" % (args.workload, w["name"], resolved, stages))

    tdt = torch.float32 if dtype == "fp32" else torch.int16
    dA = torch.from_numpy(A.view(np.int16) if dtype != "fp32" else A).to(dev)
    dB = torch.from_numpy(B.view(np.int16) if dtype != "fp32" else B).to(dev)
    dbias = torch.from_numpy(bias.view(np.int16) if dtype != "fp32" else bias).to(dev)
    assert dA.dtype == tdt
    dC = torch.empty((M, N), dtype=torch.float32, device=dev)
    gemm = gemm_launcher(wsg, w, dA, dB, dbias, dC, stages, config)

    cw = synth.WORKLOADS[2]
    copy_src = None
    if not args.no_copy:
        nel = cw["bytes"] // 4
        copy_host = synth.uniform_pm1(synth.seed_for(2, "src"), nel)
        copy_src = torch.from_numpy(copy_host).to(dev)
        copy_dst = torch.empty_like(copy_src)
        copy_cfg = dict(copy_tile_bytes=args.copy_tile or cw["tile_bytes"], producer_waves=args.copy_producers,
                        copy_workgroups=args.copy_workgroups,
                        consumer_waves=args.copy_consumers, flags=0 if args.copy_cached else wsg.WSG_FLAG_NONTEMPORAL)
        copy_stages = args.copy_stages or cw["stages"]
        copy = lambda: wsg.staged_copy_ex(copy_src, copy_dst, stages=copy_stages, config=copy_cfg)  # noqa: E731

    def step():
        gemm()
        if copy_src is not None:
            copy()

    settled = settle(torch, step, args.settle_ms)
    log("settled after %d untimed steps (%.0f ms); warmup %d" % (settled["steps"], settled["ms"], args.warmup))
    for _ in range(args.warmup):
        step()
    wsg.check_device_status()

    log("timing %d steps" % args.steps)
    g_wall, g_kern, g_min = time_region(torch, gemm, args.steps)
    g_med = LAST_MEDIAN[0]
    wsg.check_device_status()
    flops = 2.0 * M * N * K
    gemm_tflops = flops * args.steps / g_wall / 1e12
    result = {
        "metric": "GEMM+bias+ReLU TFLOP/s (% MFMA peak); LDS-staged copy HBM GB/s",
        "value": round(gemm_tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": settled,
        "ms_per_step": None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if dtype == "fp32" else "bf16",
        "data": "synthetic",
        "config": {
            "workload": w["name"] + (" + " + cw["name"] if copy_src is not None else ""),
            "M": M, "N": N, "K": K, "stages": stages,
            "tile": [resolved["BM"], resolved["BN"], resolved["BK"]],
            "producer_waves": resolved["producer_waves"], "consumer_waves": resolved["consumer_waves"],
            "group_k": resolved["group_k"], "homogeneous": bool(resolved["flags"] & wsg.WSG_FLAG_HOMOGENEOUS),
            "stream_k": bool(resolved["flags"] & wsg.WSG_FLAG_STREAM_K),
            "input": "uniform[-1,1) splitmix64" if dtype == "fp32" else "N(0,1)*0.1 rounded to bf16",
            "seeds": {t: synth.seed_for(args.workload, t) for t in ("A", "B", "bias")},
        },
    }
    peak = PEAK_TFLOPS[dtype]
    achieved = flops / g_kern / 1e12
    traffic = measured_traffic("gemm_w%d_%s" % (args.workload, "x".join(str(resolved[k]) for k in
                                                                         ("BM", "BN", "BK"))), "gemm")
    result["roofline"] = {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                          "frac": round(achieved / peak, 4), "traffic": traffic,
                          "kernel_ms": round(g_kern * 1e3, 4), "kernel_ms_min": round(g_min * 1e3, 4),
                          "kernel_ms_median": round(g_med * 1e3, 4)}
    step_s = g_wall / args.steps

    if not args.homogeneous and not args.no_ablation:
        # the same GEMM on the kernel without roles: same tile, consumer waves,
        # fragments and ring depth; every wave loads, a barrier, every wave computes
        hcfg = dict(BM=resolved["BM"], BN=resolved["BN"], BK=resolved["BK"],
                    consumer_waves=resolved["consumer_waves"], group_k=resolved["group_k"],
                    flags=wsg.WSG_FLAG_HOMOGENEOUS)
        try:
            dC_h = torch.empty_like(dC)
            hgemm = lambda: wsg.gemm_bias_relu_ex(dA, dB, dbias, dC_h, stages=stages, config=hcfg)  # noqa: E731
            warm_leg(torch, hgemm, args)
            h_wall, h_kern, h_min = time_region(torch, hgemm, args.steps)
            wsg.check_device_status()
            h_ach = flops / h_kern / 1e12
            result["homogeneous_baseline"] = {
                "tile": [hcfg["BM"], hcfg["BN"], hcfg["BK"]], "waves": hcfg["consumer_waves"], "stages": stages,
                "value": round(flops * args.steps / h_wall / 1e12, 3), "unit": "TFLOP/s",
                "kernel_tflops": round(h_ach, 3), "frac": round(h_ach / peak, 4),
                "kernel_ms": round(h_kern * 1e3, 4),
                "specialized_speedup": round(h_kern / g_kern, 4),
                "bit_identical_to_specialized": bool(torch.equal(dC_h, dC)),
            }
            del dC_h
        except wsg.WsgError as e:
            result["homogeneous_baseline"] = {"error": str(e)}

    if result["config"]["stream_k"] and not args.no_ablation:
        # the same launch with one workgroup per tile (no stream-K tail), so the
        # tail's share of the gain over the homogeneous kernel shows
        ncfg = dict(BM=resolved["BM"], BN=resolved["BN"], BK=resolved["BK"],
                    producer_waves=resolved["producer_waves"], consumer_waves=resolved["consumer_waves"],
                    group_k=resolved["group_k"], flags=(args.flags | wsg.WSG_FLAG_NO_STREAM_K) & ~wsg.WSG_FLAG_STREAM_K)
        dC_n = torch.empty_like(dC)
        ngemm = lambda: wsg.gemm_bias_relu_ex(dA, dB, dbias, dC_n, stages=stages, config=ncfg)  # noqa: E731
        warm_leg(torch, ngemm, args)
        n_wall, n_kern, _ = time_region(torch, ngemm, args.steps)
        wsg.check_device_status()
        result["no_stream_k"] = {"kernel_tflops": round(flops / n_kern / 1e12, 3), "kernel_ms": round(n_kern * 1e3, 4),
                                 "stream_k_speedup": round(n_kern / g_kern, 4)}
        del dC_n

    explicit_tile = any((args.bm, args.bn, args.bk, args.producers, args.consumers, args.group_k, args.flags))
    if stages != 2 and not args.no_ablation and not args.homogeneous and not explicit_tile:
        # context for a workload whose ring depth is fixed above 2: the same GEMM
        # through the default configuration of a 2-slot ring (for bf16 256 x 256
        # tiles that allows k tiles of 64, which a 4-slot ring does not fit)
        d2 = wsg.resolve_config(wsg.WSG_FP32 if dtype == "fp32" else wsg.WSG_BF16, M, N, K, 2, None)
        dC_2 = torch.empty_like(dC)
        gemm2 = gemm_launcher(wsg, w, dA, dB, dbias, dC_2, 2, None)
        warm_leg(torch, gemm2, args)
        r_wall, r_kern, _ = time_region(torch, gemm2, args.steps)
        wsg.check_device_status()
        r_ach = flops / r_kern / 1e12
        result["ring_depth_2"] = {
            "stages": 2, "tile": [d2["BM"], d2["BN"], d2["BK"]], "producer_waves": d2["producer_waves"],
            "consumer_waves": d2["consumer_waves"], "kernel_tflops": round(r_ach, 3), "frac": round(r_ach / peak, 4),
            "kernel_ms": round(r_kern * 1e3, 4), "speedup_over_workload_stages": round(g_kern / r_kern, 4),
            "bit_identical": bool(torch.equal(dC_2, dC)),
        }
        del dC_2

    if not args.no_vendor:
        # the vendor library (hipBLASLt through torch) on the same operands, for
        # context: relu(addmm) in the input dtype, so its output is bf16 when the
        # inputs are (half the C bytes this library writes)
        tdt_v = torch.float32 if dtype == "fp32" else torch.bfloat16
        vA, vB, vb = dA.view(tdt_v), dB.view(tdt_v), dbias.view(tdt_v)
        prev_tf32 = torch.backends.cuda.matmul.allow_tf32
        torch.backends.cuda.matmul.allow_tf32 = False
        try:
            vendor = lambda: torch.relu_(torch.addmm(vb, vA, vB))  # noqa: E731
            warm_leg(torch, vendor, args)
            v_wall, v_kern, _ = time_region(torch, vendor, args.steps)
        finally:
            torch.backends.cuda.matmul.allow_tf32 = prev_tf32
        result["vendor_library"] = {
            "op": "torch.relu_(torch.addmm(bias, A, B)), %s in and out" % ("fp32" if dtype == "fp32" else "bf16"),
            "value": round(flops * args.steps / v_wall / 1e12, 3), "unit": "TFLOP/s",
            "launch_tflops": round(flops / v_kern / 1e12, 3),
            "ours_over_vendor": round(v_kern / g_kern, 4),
        }

    if copy_src is not None:
        c_wall, c_kern, c_min = time_region(torch, copy, args.steps)
        c_med = LAST_MEDIAN[0]
        wsg.check_device_status()
        nbytes = cw["bytes"]
        moved = 2.0 * nbytes
        result["copy"] = {"value": round(moved * args.steps / c_wall / 1e9, 1), "unit": "GB/s",
                          "bytes": nbytes, "tile_bytes": copy_cfg["copy_tile_bytes"], "stages": copy_stages,
                          "producer_waves": args.copy_producers or None, "consumer_waves": args.copy_consumers or None,
                          "workgroups": args.copy_workgroups or None,
                          "nontemporal": not args.copy_cached}
        c_ach = moved / c_kern / 1e9
        result["copy_roofline"] = {"bound": "hbm", "achieved": round(c_ach, 1), "peak": PEAK_HBM_GBS,
                                   "unit": "GB/s", "frac": round(c_ach / PEAK_HBM_GBS, 4),
                                   "traffic": measured_traffic("copy_1GiB_64KiB", "copy"),
                                   "kernel_ms": round(c_kern * 1e3, 4), "kernel_ms_min": round(c_min * 1e3, 4),
                                   "kernel_ms_median": round(c_med * 1e3, 4)}
        result["copy"]["seed"] = synth.seed_for(2, "src")
        step_s += c_wall / args.steps
        # torch's own device copy of the same buffers, timed the same way: what
        # a plain (unstaged) copy kernel reaches on this device
        plain = lambda: copy_dst.copy_(copy_src)  # noqa: E731
        warm_leg(torch, plain, args)
        _, p_kern, _ = time_region(torch, plain, args.steps)
        result["copy"]["plain_device_copy"] = {"value": round(moved / p_kern / 1e9, 1), "unit": "GB/s",
                                               "kind": "torch Tensor.copy_ on the device"}
        result["copy"]["staged_over_plain"] = round(p_kern / c_kern, 4)
        # the unstaged baseline of this library (no LDS ring, no roles: every lane moves 16-byte chunks
        # through registers in a grid-stride loop, 4 in flight), timed the same way
        direct_cfg = dict(flags=wsg.WSG_FLAG_DIRECT_COPY | (0 if args.copy_cached else wsg.WSG_FLAG_NONTEMPORAL))
        direct = lambda: wsg.staged_copy_ex(copy_src, copy_dst, stages=copy_stages, config=direct_cfg)  # noqa
        warm_leg(torch, direct, args)
        _, d_kern, _ = time_region(torch, direct, args.steps)
        wsg.check_device_status()
        result["copy"]["direct_baseline"] = {"value": round(moved / d_kern / 1e9, 1), "unit": "GB/s",
                                             "kind": "unstaged copy (WSG_FLAG_DIRECT_COPY), 256 workgroups x 4 "
                                                     "waves, 4 chunks of 16 bytes in flight per lane"}
        result["copy"]["staged_over_direct"] = round(d_kern / c_kern, 4)
        # parity of the timed launch configuration, outside the timed regions: dst is overwritten
        # with a sentinel first, so only the staged copy can make it equal to src again
        copy_dst.fill_(-7.0)
        copy()
        torch.cuda.synchronize()
        result["copy"]["parity"] = {"bytes_checked": nbytes, "kind": "bit-exact, on the GPU",
                                    "pass": bool(torch.equal(copy_dst.view(torch.int32),
                                                             copy_src.view(torch.int32)))}
    result["ms_per_step"] = round(step_s * 1e3, 4)

    if args.calibrate_copy and copy_src is not None:
        # a plain device copy of known size (torch's copy kernel), outside the
        # timed regions, for scaling the HBM traffic counters
        for _ in range(3):
            copy_dst.copy_(copy_src)
        torch.cuda.synchronize()

    if args.wait_stats:
        # one more launch of each kernel with the ring's wait counters on
        wsg.read_wait_stats()
        wsg.set_wait_stats(True)
        gemm()
        if copy_src is not None:
            copy()
        st = wsg.read_wait_stats()
        wsg.set_wait_stats(False)
        result["wait_stats"] = {k: dict(v, blocked_frac=round(v["blocked"] / v["waits"], 4) if v["waits"] else None)
                                for k, v in st.items() if v["waits"]}

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle, about %.0f s)" % args.cpu_budget)
        tf, rows, secs, threads, ref = cpu_baseline_gemm(A, B, bias, args.cpu_budget)
        result["cpu_baseline"] = {"value": round(tf, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                                  "sample": "first %d rows of the %dx%dx%d GEMM (%d x %d x %d), %.1f s"
                                            % (rows, M, N, K, rows, N, K, secs),
                                  "cpu_model": cpu_model()}
        got = dC[:rows].cpu().numpy()
        s = oracle.compare(got, ref)
        result["parity"] = {"rows_checked": rows, "max_abs": s["max_abs"], "rel_fro": s["rel_fro"],
                            "pass": bool(oracle.within_tolerance(s, dtype))}
        if copy_src is not None:
            log("copy cpu baseline (oracle memcpy of %d bytes)" % nbytes)
            gbs, calls, csecs, cthreads, host_ref = cpu_baseline_copy(copy_host, args.copy_cpu_budget)
            result["copy_cpu_baseline"] = {"value": round(gbs, 1), "unit": "GB/s", "cores": cthreads,
                                           "kind": "oracle",
                                           "sample": "the whole %d-byte copy, %d calls in %.1f s, median call"
                                                     % (nbytes, calls, csecs),
                                           "cpu_model": cpu_model()}
            # the staged copy's output (left in dst above) against the oracle's, byte for byte
            mism = oracle.first_mismatch(copy_dst.cpu().numpy(), host_ref)
            result["copy"]["parity"]["oracle_first_mismatch"] = mism
            result["copy"]["parity"]["pass"] = result["copy"]["parity"]["pass"] and mism == -1
    return result


def run_moe(args):
    """The mixture-of-experts expert layer on the grouped GEMM: one JSON line."""
    import numpy as np
    import torch
    import synth
    import warp_specialized_gemm_amd as wsg
    w = synth.MOE
    rows = [int(r) for r in synth.moe_group_rows(synth.seed_for(w["id"], "A") + 50, w["tokens"], w["experts"],
                                                    w["top_k"])]
    G, K, N, M = w["experts"], w["K"], w["N"], sum(rows)
    stages = args.stages or w["stages"]
    log("generating the expert layer: %d experts, rows %s, K %d, N %d" % (G, rows, K, N))
    A = synth.normal_bf16_bits(synth.seed_for(w["id"], "A"), M * K).reshape(M, K)
    B = synth.normal_bf16_bits(synth.seed_for(w["id"], "B"), G * K * N).reshape(G, K, N)
    bias = synth.normal_bf16_bits(synth.seed_for(w["id"], "bias"), G * N).reshape(G, N)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()  # noqa: E731
    dA, dB, dbias = dev(A), dev(B), dev(bias)
    dC = torch.empty((M, N), dtype=torch.float32, device="cuda")
    config = None
    if args.bm or args.bn or args.bk or args.producers or args.consumers or args.group_k or args.flags:
        config = dict(BM=args.bm, BN=args.bn, BK=args.bk, producer_waves=args.producers,
                      consumer_waves=args.consumers, group_k=args.group_k, flags=args.flags)
    resolved = wsg.resolve_config(wsg.WSG_BF16, M, N, K, stages, config)
    grouped = lambda: wsg.grouped_gemm_bias_relu_ex(dA, dB, dbias, rows, dC, stages=stages, config=config)  # noqa
    settled = settle(torch, grouped, args.settle_ms)
    for _ in range(args.warmup):
        grouped()
    wsg.check_device_status()
    flops = 2.0 * M * N * K
    g_wall, g_kern, g_min = time_region(torch, grouped, args.steps)
    wsg.check_device_status()
    # the same flops as one dense GEMM: every row through expert 0's weights
    dC_d = torch.empty_like(dC)
    dense = lambda: wsg.gemm_bias_relu_ex(dA, dB[0], dbias[0], dC_d, stages=stages, config=config)  # noqa: E731
    warm_leg(torch, dense, args)
    _, d_kern, _ = time_region(torch, dense, args.steps)
    wsg.check_device_status()
    del dC_d
    peak = PEAK_TFLOPS["bf16"]
    achieved = flops / g_kern / 1e12
    result = {
        "metric": "grouped GEMM+bias+ReLU TFLOP/s (% bf16 MFMA peak)",
        "value": round(flops * args.steps / g_wall / 1e12, 3), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "settle": settled,
        "ms_per_step": round(g_wall / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w["name"], "experts": G, "tokens": w["tokens"], "top_k": w["top_k"],
                   "group_rows": rows, "rows": M, "K": K, "N": N, "stages": stages,
                   "tile": [resolved["BM"], resolved["BN"], resolved["BK"]],
                   "producer_waves": resolved["producer_waves"], "consumer_waves": resolved["consumer_waves"],
                   "group_k": resolved["group_k"], "input": "N(0,1)*0.1 rounded to bf16; seeded top-2 routing"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic("grouped_moe_%s" % "x".join(str(resolved[k]) for k in
                                                                              ("BM", "BN", "BK")), "gemm"),
                     "kernel_ms": round(g_kern * 1e3, 4), "kernel_ms_min": round(g_min * 1e3, 4)},
        "dense_same_flops": {"kernel_ms": round(d_kern * 1e3, 4), "kernel_tflops": round(flops / d_kern / 1e12, 3),
                             "grouped_over_dense_time": round(g_kern / d_kern, 4)},
    }
    if not args.no_cpu_baseline:
        import oracle
        starts = np.concatenate([[0], np.cumsum(rows)])
        # 16 consecutive rows of one expert per oracle call, experts in turn
        want = [int(starts[e] + 16 * b + i) for b in range(4) for e in range(G) for i in range(16)
                if 16 * b + i < rows[e]]
        threads = oracle.host_threads()
        done, spent, outs = 0, 0.0, []
        while done < len(want) and spent < args.cpu_budget:
            part = want[done:done + 16]
            t0 = time.perf_counter()
            outs.append(oracle.grouped_gemm_bias_relu_rows(A, B, bias, rows, part, threads=threads))
            spent += time.perf_counter() - t0
            done += len(part)
        ref = np.concatenate(outs, axis=0)
        result["cpu_baseline"] = {"value": round(2.0 * done * N * K / spent / 1e12, 6), "unit": "TFLOP/s",
                                  "cores": threads, "kind": "oracle",
                                  "sample": "%d rows spread over the %d experts (%d x %d x %d per row), %.1f s"
                                            % (done, G, 1, N, K, spent)}
        s = oracle.compare(dC[want[:done]].cpu().numpy(), ref)
        result["parity"] = {"rows_checked": done, "max_abs": s["max_abs"], "rel_fro": s["rel_fro"],
                            "pass": bool(oracle.within_tolerance(s, "bf16"))}
    return result


def run_attention_bench(args):
    """Attention forward (the second consumer type): one JSON line, non-causal headline plus the causal run."""
    import math
    import numpy as np
    import torch
    import synth
    import warp_specialized_gemm_amd as wsg
    w = synth.ATTENTION
    Bn, H, S, D = w["batch"], w["heads"], w["S"], w["D"]
    stages = args.stages or w["stages"]
    n = Bn * H * S * D
    log("generating attention inputs %s" % ((Bn, H, S, D),))
    Q = synth.normal_bf16_bits(synth.seed_for(w["id"], "A"), n, scale=1.0).reshape(Bn, H, S, D)
    K = synth.normal_bf16_bits(synth.seed_for(w["id"], "B"), n, scale=1.0).reshape(Bn, H, S, D)
    V = synth.normal_bf16_bits(synth.seed_for(w["id"], "src"), n, scale=1.0).reshape(Bn, H, S, D)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()  # noqa: E731
    dQ, dK, dV = dev(Q), dev(K), dev(V)
    dO = torch.empty((Bn, H, S, D), dtype=torch.float32, device="cuda")
    # the library's default for head dimension 128: one producer and seven consumer waves
    producers = args.producers or 1
    consumers = args.consumers or (7 if producers == 1 and D == 128 else 4)
    config = dict(producer_waves=producers, consumer_waves=consumers)
    peak = PEAK_TFLOPS["bf16"]
    out = {}
    settled = settle(torch, lambda: wsg.attention_fwd(dQ, dK, dV, dO, causal=False, stages=stages, config=config),
                     args.settle_ms)
    for causal in (False, True):
        fn = lambda: wsg.attention_fwd(dQ, dK, dV, dO, causal=causal, stages=stages, config=config)  # noqa: E731
        for _ in range(args.warmup):
            fn()
        wsg.check_device_status()
        wall, kern, kmin = time_region(torch, fn, args.steps)
        wsg.check_device_status()
        pairs = S * (S + 1) // 2 if causal else S * S  # (query, key) pairs that count
        flops = 4.0 * Bn * H * pairs * D
        out[causal] = (flops, wall, kern, kmin)
    flops, wall, kern, kmin = out[False]
    result = {
        "metric": "attention forward TFLOP/s (% bf16 MFMA peak)",
        "value": round(flops * args.steps / wall / 1e12, 3), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "settle": settled,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w["name"], "batch": Bn, "heads": H, "Sq": S, "Skv": S, "D": D, "stages": stages,
                   "producer_waves": producers, "consumer_waves": consumers, "queries_per_workgroup": 32 * consumers,
                   "keys_per_slot": 64, "input": "N(0,1) rounded to bf16, scale 1/sqrt(D)"},
        "roofline": {"bound": "mfma", "achieved": round(flops / kern / 1e12, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(flops / kern / 1e12 / peak, 4),
                     "traffic": measured_traffic("attention_d128_noncausal", "attention"),
                     "kernel_ms": round(kern * 1e3, 4), "kernel_ms_min": round(kmin * 1e3, 4)},
    }
    cf, cw, ck, cm = out[True]
    result["causal"] = {"value": round(cf * args.steps / cw / 1e12, 3), "unit": "TFLOP/s",
                        "kernel_tflops": round(cf / ck / 1e12, 3), "frac": round(cf / ck / 1e12 / peak, 4),
                        "kernel_ms": round(ck * 1e3, 4), "flops": cf}
    if not args.no_cpu_baseline:
        import oracle
        import oracle.attention as att
        from threadpoolctl import threadpool_limits
        threads = oracle.host_threads()
        # the causal output is still in dO: rows of head (0, 0), 32 at a time, against the oracle
        got = dO[0, 0].cpu().numpy()
        done, spent, refs, rows_all = 0, 0.0, [], []
        with threadpool_limits(limits=threads):
            while done < S and spent < args.cpu_budget:
                rows = np.arange(done, min(S, done + 32))
                t0 = time.perf_counter()
                refs.append(att.attention_rows(Q, K, V, 1.0 / math.sqrt(D), True, 0, 0, rows))
                spent += time.perf_counter() - t0
                rows_all.append(rows)
                done += rows.size
        rows = np.concatenate(rows_all)
        pairs = int(np.sum(rows + 1))
        result["cpu_baseline"] = {"value": round(4.0 * pairs * D / spent / 1e12, 6), "unit": "TFLOP/s",
                                  "cores": threads, "kind": "oracle",
                                  "sample": "causal rows 0..%d of head (0, 0), %.1f s (numpy fp64, BLAS limited to "
                                            "%d threads)" % (done - 1, spent, threads)}
        s = oracle.compare(got[rows], np.concatenate(refs))
        result["parity"] = {"rows_checked": int(done), "max_abs": s["max_abs"], "rel_fro": s["rel_fro"],
                            "pass": bool(oracle.within_tolerance(s, "bf16"))}
    return result


def sweep(args):
    """Ring depth S in 2, 3, 4 x 1, 2 or 4 producer waves on the 4096^3 fp32
    GEMM (256x128 tiles, 4 consumer waves; each point takes the deepest k tile
    whose ring fits in LDS), then the kernel without roles at S = 1, 2, 3 on
    the same tiles. Points with no built kernel are printed with the error."""
    import copy as _copy
    out = []
    points = [(p, s, False) for p in (1, 2, 4) for s in (2, 3, 4)] + [(0, s, True) for s in (1, 2, 3)]
    for producers, stages, homogeneous in points:
        a = _copy.copy(args)
        a.stages, a.producers, a.no_copy, a.no_cpu_baseline = stages, producers, True, True
        a.homogeneous, a.no_ablation = homogeneous, True
        a.bm, a.bn, a.consumers = a.bm or 256, a.bn or 128, a.consumers or 4
        try:
            r = run(a)
            line = {"stages": stages, "producer_waves": producers, "homogeneous": homogeneous,
                    "tile": r["config"]["tile"], "consumer_waves": r["config"]["consumer_waves"],
                    "tflops": r["value"], "kernel_tflops": r["roofline"]["achieved"], "frac": r["roofline"]["frac"]}
        except Exception as e:  # an unsupported point is reported, not fatal
            line = {"stages": stages, "producer_waves": producers, "homogeneous": homogeneous, "error": str(e)}
        print(json.dumps(line), flush=True)
        out.append(line)
    return out


def main():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--leg-settle-ms", type=float, default=100.0,
                   help="untimed launches of each comparison leg before it is timed (ms)")
    p.add_argument("--settle-ms", type=float, default=200.0,
                   help="untimed hot-path steps for at least this long before the first warmup step")
    p.add_argument("--workload", type=int, default=3, choices=[1, 3, 4, 5])
    p.add_argument("--stages", type=int, default=0)
    p.add_argument("--bm", type=int, default=0)
    p.add_argument("--bn", type=int, default=0)
    p.add_argument("--bk", type=int, default=0)
    p.add_argument("--producers", type=int, default=0)
    p.add_argument("--consumers", type=int, default=0)
    p.add_argument("--group-k", type=int, default=0, help="consumer k per fragment group (16 or 32)")
    p.add_argument("--flags", type=int, default=0,
                   help="GEMM wsg_config.flags bits (1: register-staged producer)")
    p.add_argument("--no-copy", action="store_true")
    p.add_argument("--copy-tile", type=int, default=0, help="staged copy: bytes per ring slot")
    p.add_argument("--copy-stages", type=int, default=0)
    p.add_argument("--copy-producers", type=int, default=0)
    p.add_argument("--copy-consumers", type=int, default=0)
    p.add_argument("--copy-workgroups", type=int, default=0, help="staged copy: persistent grid size (0: default)")
    p.add_argument("--copy-cached", action="store_true",
                   help="staged copy: ordinary (cached) loads and stores instead of streaming ones")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    p.add_argument("--copy-cpu-budget", type=float, default=5.0,
                   help="seconds of copy-oracle calls for copy_cpu_baseline")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="after timing, run torch's plain 1 GiB device copy 3 times (for counter calibration)")
    p.add_argument("--homogeneous", action="store_true",
                   help="time the GEMM kernel without roles (every wave loads, barrier, computes) instead")
    p.add_argument("--no-ablation", action="store_true", help="skip the homogeneous_baseline measurement")
    p.add_argument("--no-vendor", action="store_true",
                   help="skip the vendor_library leg (the same GEMM through torch.addmm, for context)")
    p.add_argument("--sweep", action="store_true")
    p.add_argument("--attention", action="store_true",
                   help="attention forward (batch 4, 32 heads, 4096 x 4096, D 128) instead of the default step")
    p.add_argument("--moe", action="store_true",
                   help="the mixture-of-experts expert layer on the grouped GEMM instead of the default step")
    p.add_argument("--wait-stats", action="store_true",
                   help="after timing, count ring flag waits per role over one launch of each kernel")
    args = p.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (each GPU would run the same "
              "kernels on its own share of output tiles or bytes); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.sweep:
        sweep(args)
        return
    if args.moe:
        print(json.dumps(run_moe(args)), flush=True)
        return
    if args.attention:
        print(json.dumps(run_attention_bench(args)), flush=True)
        return
    print(json.dumps(run(args)), flush=True)


if __name__ == "__main__":
    main()
