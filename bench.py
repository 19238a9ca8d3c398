"""Benchmark: W4A16 GEMV / small-M GEMM achieved HBM bandwidth and microseconds per call.

Default workload: the FFN up/gate projection (K=5120, N=17408, group 128, symmetric zero
point) swept over M = 1, 2, 4, 8, 16 rows; one step is one call at each M. Inputs are seeded
synthetic tensors with the value distributions of an int4 GPTQ checkpoint and bf16
activations (no checkpoint is loaded). Every call reads a different copy of the weights
(consecutive calls included) from a rotating pool far larger than the 256 MB last-level cache,
so the weights stream from HBM as they do in decode, where each layer's weights are read once
per token.

Algorithmic bytes per call = qweight (K*N/2) + scales (2*K*N/g) + qzeros (K*N/(2g), if any)
+ activations (2*M*K) + outputs (4*M*N for fp32). Re-reads, padding and split-K scratch are
not counted.

Warm-up: W steps, then more until the device has been busy for 0.3 s (its clock ramps up over
the first tens of milliseconds of work). Timed regions (all on the library's stream, inputs
resident in HBM):
  1. K steps back to back -> `value` (whole-step throughput, wall clock between synchronizes);
  2. each row count's call alone, K launches back to back (rotating weight copies) between one
     HIP event pair -> `per_m` us_per_call (device time per call); the row count with the most
     device time is the dominant call, whose algorithmic bytes / us_per_call is
     `roofline.achieved`;
  3. context only: the K steps again with an event pair around every launch (per_m
     us_lone_event_pair, which includes the dispatch gap before each launch); each row count's
     call captured into a HIP graph (one launch per rotating copy) and replayed (per_m
     us_per_call_graph_replay: no host work between launches); the dominant call
     on one weight copy, cache-resident (`context.cache_resident`, L2/MALL, not HBM); a plain
     streaming read of one rotating copy of the packed weights per launch, replayed from a HIP
     graph (`context.read_ceiling`, w4a16_stream_read: the measured ceiling for reading those
     bytes);
     a device copy of the same bytes (`context.copy`, bytes read + written).
`roofline.traffic` is the HBM bytes per launch of that call from the committed rocprofv3 counter
summary (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy of known size), or null when the
kernel sources changed since the counters were taken.

With --prefill every call is the many-row (prompt-processing) GEMM, w4a16_gemm_prefill, on the
workload's matrix with M = 512 and 2048 rows by default (activations drawn with the workload's
distribution): the bound is the fp16 matrix cores (2.5 PFLOP/s dense), and the line reports
TFLOP/s (2*M*N*K per call) with an "mfma" roofline.

--prefill --gate-up times the prompt-sized gated pair (w4a16_gemm_gate_up_prefill), 4*M*N*K
flops per call. --prefill --affine [--affine-bits B] times the affine prompt GEMM
(w4a16_gemm_affine_bits_prefill) on the affine FFN up projection of that width (codes read as
stored), activations N(0, 1).

With --gate-up every call is instead the fused gated pair on the workload's shape,
silu(A x W_gate) * (A x W_up) (w4a16_gemm_gate_up): two weight matrices per call, one [M, N]
output, and the algorithmic bytes count both matrices.

With --affine every call is the affine-code GEMM (w4a16_gemm_affine, w = s * q + b, bf16 scales
and biases) on the affine-4 FFN up projection 5120 x 17408 in groups of 64, M = 1, 2, 4, 8, 16.
Algorithmic bytes per call = codes (K*N*bits/8) + scales and biases (4*K*N/g) + activations
(2*M*K) + outputs (4*M*N). --affine-bits 2, 3, 5, 6 or 8 takes the checkpoint of that width of the
same projection: 2 and 3-bit codes widened onto the 4-bit layout once (w4a16_affine_widen), 5, 6
and 8-bit codes split into two 4-bit planes once (w4a16_affine_split, w4a16_gemm_affine_split);
--affine-native reads the codes of any of these widths as stored (w4a16_gemm_affine_bits). The
algorithmic bytes are always those of the stored format.

Prints one JSON line (rank 0; this build runs on one GPU).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
PEAK_F16_TFLOPS = 2500.0        # MI355X dense fp16 matrix cores
POOL_BYTES = 768 * 2 ** 20      # rotating weight pool, 3x the 256 MB last-level cache
WARM_SECONDS = 0.3              # minimum device-busy warm-up before any timing


def algorithmic_bytes(M, K, N, g, symmetric, out_bytes=4, matrices=1):
    w = K * N // 2 + 2 * (K // g) * N
    if not symmetric:
        w += (K // g) * N // 2
    return matrices * w + 2 * M * K + out_bytes * M * N


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="ffn_up",
                   choices=["tiny", "attn", "ffn_up", "ffn_down", "lm_head"])
    p.add_argument("--ms", default=None, help="comma-separated row counts (default: the workload's)")
    p.add_argument("--splits", type=int, default=0, help="workgroups per column tile along K (0 = default)")
    p.add_argument("--waves-k", type=int, default=0, help="waves per workgroup along K (0 = default)")
    p.add_argument("--tile-cols", type=int, default=0, help="column tile width, 64 or 128 (0 = default)")
    p.add_argument("--prefill", action="store_true",
                   help="time the many-row GEMM (w4a16_gemm_prefill) on the workload's matrix, M = --ms "
                        "(default 512,2048)")
    p.add_argument("--gate-up", action="store_true",
                   help="time the fused gated pair silu(A x W_gate) * (A x W_up) on the workload's shape")
    p.add_argument("--affine", action="store_true",
                   help="time the affine-code GEMM on the affine-4 FFN up projection (w = s * q + b)")
    p.add_argument("--affine-bits", type=int, default=4, choices=[2, 3, 4, 5, 6, 8],
                   help="with --affine: code width of the checkpoint (2 and 3 are widened to 4 bits once, 5, 6 "
                        "and 8 split into two 4-bit planes once, unless --affine-native)")
    p.add_argument("--affine-native", action="store_true",
                   help="with --affine: read the codes at their own width (w4a16_gemm_affine_bits)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-context", action="store_true",
                   help="time only regions 1 and 2 (no lone event pairs, graph replays, read ceiling or copies): "
                        "for counter collection")
    p.add_argument("--calibrate", type=int, default=0, metavar="MIB",
                   help="only run a plain elementwise kernel (y = 2x, fp32) over MIB MiB five times: the "
                        "reference for scaling rocprofv3's FETCH_SIZE / WRITE_SIZE to bytes")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    return p.parse_args()


def cpu_one_thread(workload, ms, seconds):
    """The same oracle on one host thread over whole steps (one call per row count in `ms`): a
    child process started with OMP_NUM_THREADS=1 (OpenMP fixes its thread count when it starts)
    that runs only the CPU oracle on its own copy of the seeded inputs. Returns steps, seconds."""
    import subprocess
    code = (f"import sys, time, json\nsys.path.insert(0, {ROOT!r})\n"
            "import oracle\nfrom verify_matmul_amd import synth\n"
            f"oracle._load()\ninp = synth.make_inputs(synth.WORKLOADS[{workload!r}])\n"
            "n, el = 0, 0.0\n"
            f"while el < {seconds} or n == 0:\n"
            f"    for M in {tuple(ms)!r}:\n"
            "        t = time.perf_counter()\n"
            "        oracle.gemm(inp.act[:M], inp.qweight, inp.scales, inp.qzeros, inp.group)\n"
            "        el += time.perf_counter() - t\n"
            "    n += 1\n"
            "print(json.dumps({'calls': n, 'seconds': el}))\n")
    env = dict(os.environ, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        raise RuntimeError(f"one-thread oracle run failed: {r.stderr[-500:]}")
    return json.loads(r.stdout.strip().splitlines()[-1])


def host_cpu():
    """This host's processor model and logical CPU count, recorded beside the oracle's timing."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "logical_cpus": os.cpu_count(),
            "usable_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


def cpu_baseline(wl, inp, ms, seconds, gate=None, one=None):
    """The CPU oracle, as it is, on this host's cores: the whole step repeated for ~`seconds`."""
    import oracle
    oracle._load()
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    reps, elapsed, nbytes = 0, 0.0, 0
    while elapsed < seconds or reps == 0:
        for M in ms:
            t = time.perf_counter()
            if gate is None:
                oracle.gemm(inp.act[:M], inp.qweight, inp.scales, inp.qzeros, inp.group)
            else:
                oracle.gate_up(inp.act[:M], (gate.qweight, gate.scales, gate.qzeros),
                               (inp.qweight, inp.scales, inp.qzeros), inp.group)
            elapsed += time.perf_counter() - t
            nbytes += algorithmic_bytes(M, wl.K, wl.N, wl.group, wl.symmetric, matrices=1 if gate is None else 2)
        reps += 1
    rec = {"value": round(nbytes / elapsed / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"{reps} full step(s) of the workload (M={','.join(map(str, ms))}, all {wl.N} columns), "
                     f"{elapsed:.1f} s of oracle time (unpack + exact dequant + fp64 accumulate)",
           "host": host_cpu()}
    if one is not None:   # the same steps on one thread (measured before any GPU work)
        step_b = sum(algorithmic_bytes(M, wl.K, wl.N, wl.group, wl.symmetric) for M in ms)
        v1 = step_b * one["calls"] / one["seconds"] / 1e9
        rec["one_thread"] = {"value": round(v1, 4), "unit": "GB/s", "cores": 1,
                             "sample": f"{one['calls']} full step(s), {one['seconds']:.1f} s of oracle time"}
        # what the threads above actually bought on this host (its CPU share may be smaller
        # than its thread count)
        rec["speedup_over_one_thread"] = round(rec["value"] / v1, 2)
    return rec


def warm_up(step, n):
    """n untimed steps, then more until the device has been busy for WARM_SECONDS: its clock ramps
    up over the first tens of milliseconds of work, which a short warm-up would leave in the
    timing."""
    import torch
    for i in range(n):
        step(i)
    torch.cuda.synchronize()
    i, t0 = n, time.perf_counter()
    while time.perf_counter() - t0 < WARM_SECONDS:
        step(i)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return i


def load_traffic(workload, M, kernel):
    """HBM bytes per launch of the M-row call, from the committed rocprofv3 counter summary, if it
    still matches the kernel source; None otherwise."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}_M{M}.json")
    if not os.path.exists(path):
        return None
    try:
        from verify_matmul_amd import _build
        with open(path) as f:
            rec = json.load(f)
        if rec.get("source_hash") != _build.source_hash():
            return None
        return rec.get("bytes_per_launch")
    except Exception:
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the path runs on one GPU; --gpus {args.gpus} is not supported "
              f"(more GPUs would each take a column shard of the weights)", file=sys.stderr)
        return 2
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if world != 1:
        print("bench.py: run as a single process on one GPU", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import verify_matmul_amd as vm
    from verify_matmul_amd import synth

    # the one-thread oracle figure runs in a child process, started here before this process
    # loads the library or touches the device
    one_thread = None
    if not (args.no_cpu_baseline or args.calibrate or args.affine or args.prefill or args.gate_up):
        w0 = synth.WORKLOADS[args.workload]
        ms0 = tuple(int(x) for x in args.ms.split(",")) if args.ms else w0.ms
        if algorithmic_bytes(1, w0.K, w0.N, w0.group, w0.symmetric) <= 128 * 2 ** 20:   # not the output layer
            one_thread = cpu_one_thread(args.workload, ms0, max(1.0, args.cpu_seconds / 4))

    if args.calibrate:
        n = args.calibrate * 2 ** 20 // 4
        x = torch.ones(n, dtype=torch.float32, device="cuda:0")
        y = torch.empty_like(x)
        for _ in range(5):
            torch.mul(x, 2.0, out=y)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "torch.mul(x, 2.0, out=y) fp32", "bytes_read": 4 * n,
                          "bytes_written": 4 * n, "launches": 5}), flush=True)
        return 0

    lib = vm.load()
    if args.prefill:
        return run_prefill(args, lib)
    if args.affine:
        return run_affine(args, lib)
    wl = synth.WORKLOADS[args.workload]
    ms = tuple(int(x) for x in args.ms.split(",")) if args.ms else wl.ms
    inp = synth.make_inputs(wl)
    pair = args.gate_up
    gate_inp = synth.make_gate_inputs(wl) if pair else None
    nmat = 2 if pair else 1
    if pair and (wl.argmax or args.tile_cols):
        print("bench.py: --gate-up takes no output-layer workload and no --tile-cols", file=sys.stderr)
        return 2
    K, N, g = wl.K, wl.N, wl.group
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    per_copy = algorithmic_bytes(1, K, N, g, wl.symmetric, matrices=nmat)
    R = max(2, math.ceil(POOL_BYTES / per_copy))
    qw0 = torch.from_numpy(inp.qweight.view(np.int32)).to(dev)
    sc0 = torch.from_numpy(inp.scales.view(np.int16)).to(dev)
    qz0 = None if inp.qzeros is None else torch.from_numpy(inp.qzeros.view(np.int32)).to(dev)
    a0 = torch.from_numpy(inp.act.view(np.int16)).to(dev)
    if pair:
        gw0 = torch.from_numpy(gate_inp.qweight.view(np.int32)).to(dev)
        gs0 = torch.from_numpy(gate_inp.scales.view(np.int16)).to(dev)
        gz0 = None if gate_inp.qzeros is None else torch.from_numpy(gate_inp.qzeros.view(np.int32)).to(dev)
    pool, gates = [], []
    for r in range(R):
        qw = qw0.clone()
        sc = sc0.clone()
        qz = None if qz0 is None else qz0.clone()
        a = a0.clone()
        outs = {M: torch.empty((M, N), dtype=torch.float32, device=dev) for M in ms}
        pool.append((qw, sc, qz, a, outs))
        if pair:
            gates.append((gw0.clone(), gs0.clone(), None if gz0 is None else gz0.clone()))
    del qw0, sc0, qz0
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    # pre-marshalled calls: (M, args) per rotation slot
    def vp(t):
        return None if t is None else ctypes.c_void_p(t.data_ptr())

    calls = []
    for r, (qw, sc, qz, a, outs) in enumerate(pool):
        row = []
        for M in ms:
            if pair:
                gw, gs, gz = gates[r]
                row.append((M, (vp(a), vp(gw), vp(gs), vp(gz), vp(qw), vp(sc), vp(qz), g, M, N, K, vp(outs[M]), 0,
                                args.splits, args.waves_k, sp)))
            else:
                row.append((M, (vp(a), vp(qw), vp(sc), vp(qz), g, M, N, K, vp(outs[M]), 0, args.splits,
                                args.waves_k, args.tile_cols, sp)))
        calls.append(row)
    fn = lib.w4a16_gemm_gate_up_ex if pair else lib.w4a16_gemm_ex

    def step(i, evs=None):
        # every call of every step reads its own weight copy: consecutive calls never find the
        # previous call's weights in the last-level cache
        for j, M in enumerate(ms):
            cargs = calls[(i * len(ms) + j) % R][j][1]
            if evs is not None:
                evs[i][j][0].record(stream)
            rc = fn(*cargs)
            if evs is not None:
                evs[i][j][1].record(stream)
            if rc != 0:
                raise RuntimeError(f"{'w4a16_gemm_gate_up_ex' if pair else 'w4a16_gemm_ex'} failed: "
                                   f"{lib.w4a16_last_error().decode()}")

    # the library calls in the order this run makes them, as (phase, calls): a kernel trace of the
    # run splits its dispatches by these counts
    phases = [("warm-up", warm_up(step, args.warmup) * len(ms))]

    # timed region 1: the steps back to back, as a decode loop issues them -> value
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_bytes = sum(algorithmic_bytes(M, K, N, g, wl.symmetric, matrices=nmat) for M in ms)
    value = step_bytes * args.steps / wall / 1e9
    phases.append(("region 1: steps back to back", args.steps * len(ms)))

    def back_to_back(launch):
        """Average device time per launch: K launches back to back between one HIP event pair on
        the library's stream."""
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        c0.record(stream)
        for i in range(args.steps):
            launch(i)
        c1.record(stream)
        torch.cuda.synchronize()
        return c0.elapsed_time(c1) * 1e3 / args.steps

    # timed region 2: each row count's call alone, K launches back to back (rotating weight
    # copies) -> per_m us_per_call (device time per call) and the roofline of the dominant call
    per_m = {}
    for j, M in enumerate(ms):
        us = back_to_back(lambda i, j=j: fn(*calls[i % R][j][1]))
        phases.append((f"region 2: M={M} back to back", args.steps))
        b = algorithmic_bytes(M, K, N, g, wl.symmetric, matrices=nmat)
        kern, spl, wk, tcols = vm.w4a16_plan(M, N, K, g)
        per_m[str(M)] = {"us_per_call": round(us, 3), "GBps": round(b / us / 1e3, 1),
                         "frac_of_peak": round(b / us / 1e3 / PEAK_HBM_GBPS, 4), "bytes": b}
        if pair:   # 128-column tiles of the 2N-wide pair (64 output columns of each matrix)
            per_m[str(M)].update({"kernel": "w4a16_gemm_kernel (mfma, gated pair)", "tile_cols": 128})
            if args.splits or args.waves_k:
                per_m[str(M)].update({"splits": args.splits or "default", "waves_k": args.waves_k or "default"})
        elif kern >= 2 and not (args.splits or args.waves_k or args.tile_cols):
            per_m[str(M)].update({"kernel": "decode_kernel (" + ("gemv" if kern == 2 else "mfma") + ")",
                                  "slices": spl, "waves_k": wk, "tile_cols": tcols})
        else:
            kern_old = kern if kern < 2 else (0 if M == 1 else 1)
            per_m[str(M)].update({"kernel": "w4a16_gemm_kernel (" + ("gemv" if kern_old == 0 else "mfma") + ")",
                                  "splits": args.splits or (spl if kern < 2 else "default"),
                                  "waves_k": args.waves_k or (wk if kern < 2 else "default"),
                                  "tile_cols": args.tile_cols or (tcols if kern < 2 else "default")})
    # the dominant call: the row count whose call takes the most device time in a step
    dom = max(ms, key=lambda M: per_m[str(M)]["us_per_call"])
    dm = per_m[str(dom)]
    us_dom = dm["us_per_call"]

    achieved = dm["bytes"] / us_dom / 1e3   # GB/s
    dom_kernel = dm["kernel"].split(" ")[0]
    traffic = load_traffic(args.workload + ("_gate_up" if pair else ""), dom, dom_kernel)
    if args.no_context:
        print(json.dumps({"metric": "W4A16 GEMV/small-M GEMM device time per call (counter run, no context)",
                          "value": round(value, 1), "unit": "GB/s", "steps": args.steps, "per_m": per_m,
                          "roofline": {"kernel": f"{dm['kernel']}, M={dom}", "achieved": round(achieved, 1),
                                       "us_per_launch": us_dom}, "phases": phases}), flush=True)
        return 0

    # context: the same steps with a HIP event pair around every launch (each pair also times the
    # dispatch gap in front of its launch)
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in ms]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, evs)
    torch.cuda.synchronize()
    phases.append(("context: steps with an event pair per launch", args.steps * len(ms)))
    for j, M in enumerate(ms):
        d = np.array([evs[i][j][0].elapsed_time(evs[i][j][1]) * 1e3 for i in range(args.steps)])   # us
        per_m[str(M)].update({"us_lone_event_pair": round(float(np.mean(d)), 3),
                              "us_lone_event_pair_median": round(float(np.median(d)), 3)})

    # output layer: the greedy pick over each row of logits on its own (it re-reads the logits;
    # not part of the algorithmic bytes of the matmul), and the same pick fused into the GEMM's
    # epilogue (one launch, no logits re-read), both back to back
    if wl.argmax:
        for j, M in enumerate(ms):
            idx = torch.empty((M,), dtype=torch.int32, device=dev)
            logits = pool[0][4][M]
            vm.w4a16_argmax_rows(logits, idx)
            aargs = (vp(logits), M, N, vp(idx), sp)
            us = back_to_back(lambda i, aargs=aargs: lib.w4a16_argmax_rows(*aargs))
            per_m[str(M)]["argmax_us_per_call"] = round(us, 3)
            per_m[str(M)]["argmax_GBps"] = round(4 * M * N / us / 1e3, 1)

            fargs = [(vp(a), vp(qw), vp(sc), vp(qz), g, M, N, K, vp(outs[M]), 0, vp(idx), sp)
                     for qw, sc, qz, a, outs in pool]   # pre-marshalled, as the plain calls
            for i in range(R):   # warm-up: the first call takes the call's scratch
                if lib.w4a16_gemm_argmax(*fargs[i]) != 0:
                    raise RuntimeError(f"w4a16_gemm_argmax failed: {lib.w4a16_last_error().decode()}")
            per_m[str(M)]["fused_gemm_argmax_us_per_call"] = round(
                back_to_back(lambda i, fargs=fargs: lib.w4a16_gemm_argmax(*fargs[i % R])), 3)
            phases.append((f"pick: M={M} fused greedy pick, warm-up and back to back", R + args.steps))
            # the 8 best columns per row, picked in the same launch
            top = torch.empty((M, 8), dtype=torch.int32, device=dev)
            targs = [(vp(a), vp(qw), vp(sc), vp(qz), g, M, N, K, vp(outs[M]), 0, 8, vp(top), sp)
                     for qw, sc, qz, a, outs in pool]
            for i in range(R):
                if lib.w4a16_gemm_topk(*targs[i]) != 0:
                    raise RuntimeError(f"w4a16_gemm_topk failed: {lib.w4a16_last_error().decode()}")
            per_m[str(M)]["fused_gemm_top8_us_per_call"] = round(
                back_to_back(lambda i, targs=targs: lib.w4a16_gemm_topk(*targs[i % R])), 3)
            phases.append((f"pick: M={M} fused top-8, warm-up and back to back", R + args.steps))

    # context only, never `value`: (a) the dominant launch on one weight copy K times, which then
    # stays in the L2s and the 256 MB last-level cache (a cache-resident rate, not an HBM one);
    # (b) a plain streaming read of one rotating copy of the packed weights per launch
    # (w4a16_stream_read: 16-byte non-temporal loads, nothing else), the measured ceiling of
    # reading these bytes from HBM; (c) a device copy of the same bytes per launch (read + write)
    jd = list(ms).index(dom)
    resident_us = back_to_back(lambda i: fn(*calls[0][jd][1]))
    phases.append((f"context: M={dom} on one cache-resident weight copy", args.steps))

    def graph_replayed(issue):
        """Average device time per launch with no host work between launches: issue(stream) makes
        R launches (one per rotating copy) on a side stream, run once eagerly (it takes its
        scratch then), captured once into a HIP graph, and the graph replayed back to back."""
        gs = torch.cuda.Stream()
        gsp = ctypes.c_void_p(gs.cuda_stream)
        with torch.cuda.stream(gs):
            issue(gsp)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=gs):
            issue(gsp)
        torch.cuda.synchronize()
        graph.replay()
        reps = max(1, args.steps // R)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        c0.record(stream)
        for _ in range(reps):
            graph.replay()
        c1.record(stream)
        torch.cuda.synchronize()
        graph_replay_launches[0] = R * (2 + reps)   # eager, first replay, timed replays
        return c0.elapsed_time(c1) * 1e3 / (reps * R)
    graph_replay_launches = [0]

    def issue_calls(j):
        def issue(gsp):
            for r in range(R):
                if fn(*(calls[r][j][1][:-1] + (gsp,))) != 0:
                    raise RuntimeError(f"call failed: {lib.w4a16_last_error().decode()}")
        return issue

    for j, M in enumerate(ms):
        try:
            per_m[str(M)]["us_per_call_graph_replay"] = round(graph_replayed(issue_calls(j)), 3)
            phases.append((f"context: M={M} from a HIP graph (eager, first replay, timed replays)",
                           graph_replay_launches[0]))
        except RuntimeError as e:   # context only: a call that cannot be captured leaves it out
            per_m[str(M)]["us_per_call_graph_replay"] = None
            per_m[str(M)]["graph_replay_error"] = str(e)[:200]

    sink = torch.zeros((4,), dtype=torch.int32, device=dev)
    read_bytes = pool[0][0].numel() * 4

    def issue_reads(gsp):
        for r in range(R):
            if lib.w4a16_stream_read(vp(pool[r][0]), ctypes.c_size_t(read_bytes), vp(sink), gsp) != 0:
                raise RuntimeError(f"w4a16_stream_read failed: {lib.w4a16_last_error().decode()}")
    ceil_us = graph_replayed(issue_reads)
    dst = torch.empty_like(pool[0][0])
    copy_us = back_to_back(lambda i: dst.copy_(pool[1 + i % (R - 1)][0]))
    ceil_gbps = read_bytes / ceil_us / 1e3
    context = {"cache_resident": {"what": "the dominant launch on one weight copy, back to back: L2/MALL, not HBM",
                                  "us_per_launch": round(resident_us, 3),
                                  "GBps": round(dm["bytes"] / resident_us / 1e3, 1)},
               "read_ceiling": {"what": "w4a16_stream_read over one rotating copy of the packed weights per launch "
                                        "(plain 16-byte non-temporal loads, 16 KiB per workgroup), replayed from "
                                        "a HIP graph",
                                "bytes": read_bytes, "us_per_launch": round(ceil_us, 3),
                                "GBps": round(ceil_gbps, 1), "frac_of_peak": round(ceil_gbps / PEAK_HBM_GBPS, 4),
                                "dominant_call_frac_of_ceiling": round(achieved / ceil_gbps, 4)},
               "copy": {"what": "device copy of one rotating copy of the packed weights per launch (torch copy_), "
                                "bytes read + written",
                        "bytes": 2 * read_bytes, "us_per_launch": round(copy_us, 3),
                        "GBps": round(2 * read_bytes / copy_us / 1e3, 1)}}

    rec = {
        "metric": "W4A16 GEMV/small-M GEMM achieved HBM GB/s (% of peak) and us/call, M=1..16",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": (f"{wl.name} gated pair silu(A x W_gate) * (A x W_up)" if pair else wl.name) +
                               f", M in {','.join(map(str, ms))} (one call each per step)",
                   "K": K, "N": N, "group": g, "symmetric_zero": wl.symmetric, "ms": list(ms), "out": "fp32",
                   "rotation_copies": R, "pool_MiB": round(R * per_copy / 2 ** 20),
                   "launch": "default" if not (args.splits or args.waves_k or args.tile_cols) else
                   f"splits={args.splits or 'default'} waves_k={args.waves_k or 'default'} "
                   f"tile_cols={args.tile_cols or 'default'}"},
        "roofline": {"bound": "hbm", "kernel": f"{dm['kernel']}, M={dom}", "M": dom,
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic,
                     "launches": args.steps, "bytes_per_launch": dm["bytes"],
                     "us_per_launch": round(us_dom, 3), "us_per_launch_lone_event_pair": dm["us_lone_event_pair"]},
        "per_m": per_m,
        "context": context,
        "phases": phases,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl, inp, ms, args.cpu_seconds, gate_inp, one_thread)
    print(json.dumps(rec), flush=True)
    return 0


def affine_bytes(M, K, N, g, bits=4, matrices=1):
    return matrices * (K * N * bits // 8 + 4 * (K // g) * N) + 2 * M * K + 4 * M * N


def run_affine(args, lib):
    """The affine-code GEMM at decode row counts: GB/s against HBM, as the default mode."""
    import numpy as np
    import torch
    import verify_matmul_amd as vm
    from verify_matmul_amd import synth

    bits = args.affine_bits
    native = args.affine_native
    pair = args.gate_up   # the affine gated pair silu(A x W_gate) * (A x W_up)
    if args.prefill or (pair and (bits != 4 or native or args.splits or args.waves_k or args.tile_cols)):
        print("bench.py: --affine takes no --prefill; --affine --gate-up takes 4-bit codes, no --affine-native and "
              "no launch knobs", file=sys.stderr)
        return 2
    nmat = 2 if pair else 1
    split = bits >= 5 and not native   # two 4-bit planes
    widen = bits < 4 and not native    # widened onto 4 bits
    if (bits != 4 or native) and (args.splits or args.waves_k or args.tile_cols):
        print("bench.py: launch knobs apply to 4-bit codes on the small-row kernel only", file=sys.stderr)
        return 2
    wl = synth.AFFINE_WORKLOADS[f"ffn_up_affine{bits}"]
    ms = tuple(int(x) for x in args.ms.split(",")) if args.ms else wl.ms
    x = synth.make_affine_inputs(wl)
    K, N, g = wl.K, wl.N, wl.group
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    per_copy = affine_bytes(1, K, N, g, bits, nmat)
    R = max(2, math.ceil(POOL_BYTES / per_copy))
    if pair:
        xg = synth.make_affine_gate_inputs(wl)
        gq0 = torch.from_numpy(np.ascontiguousarray(xg.packed).view(np.int32)).to(dev)
        gs0 = torch.from_numpy(xg.scales.view(np.int16)).to(dev)
        gb0 = torch.from_numpy(xg.biases.view(np.int16)).to(dev)
        gates = [(gq0.clone(), gs0.clone(), gb0.clone()) for _ in range(R)]
    qw0 = torch.from_numpy(np.ascontiguousarray(x.packed).view(np.int32)).to(dev)   # 4-bit: the qweight layout
    sc0 = torch.from_numpy(x.scales.view(np.int16)).to(dev)
    bi0 = torch.from_numpy(x.biases.view(np.int16)).to(dev)
    a0 = torch.from_numpy(x.act.view(np.int16)).to(dev)
    pool = []
    for _ in range(R):
        if split:   # the split planes, prepared once per copy
            qw = torch.empty((2 * K // 8, N), dtype=torch.int32, device=dev)
            sc = torch.empty((2 * K // g, N), dtype=torch.int16, device=dev)
            bi = torch.empty((2 * K // g, N), dtype=torch.int16, device=dev)
            vm.w4a16_affine_split(qw0, bits, sc0, bi0, g, K, qw, sc, bi)
        elif widen:   # widened onto the 4-bit layout once per copy
            qw = torch.empty((K // 8, N), dtype=torch.int32, device=dev)
            vm.w4a16_affine_widen(qw0, bits, K, qw)
            sc, bi = sc0.clone(), bi0.clone()
        else:   # 4-bit codes (the qweight layout), or the stream as stored (native)
            qw, sc, bi = qw0.clone(), sc0.clone(), bi0.clone()
        pool.append((qw, sc, bi, a0.clone(), {M: torch.empty((M, N), dtype=torch.float32, device=dev) for M in ms}))
    del qw0
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    vp = lambda t: ctypes.c_void_p(t.data_ptr())
    if pair:
        calls = [[(vp(a), vp(gates[r][0]), vp(gates[r][1]), vp(gates[r][2]), vp(qw), vp(sc), vp(bi), g, M, N, K,
                   vp(outs[M]), 0, sp) for M in ms] for r, (qw, sc, bi, a, outs) in enumerate(pool)]
        fn = lib.w4a16_gemm_affine_gate_up
    elif native:
        calls = [[(vp(a), vp(qw), bits, vp(sc), vp(bi), g, M, N, K, vp(outs[M]), 0, sp) for M in ms]
                 for qw, sc, bi, a, outs in pool]
        fn = lib.w4a16_gemm_affine_bits
    elif split:
        calls = [[(vp(a), vp(qw), vp(sc), vp(bi), g, M, N, K, vp(outs[M]), 0, sp) for M in ms]
                 for qw, sc, bi, a, outs in pool]
        fn = lib.w4a16_gemm_affine_split
    else:
        calls = [[(vp(a), vp(qw), vp(sc), vp(bi), g, M, N, K, vp(outs[M]), 0, args.splits, args.waves_k,
                   args.tile_cols, sp)
                  for M in ms] for qw, sc, bi, a, outs in pool]
        fn = lib.w4a16_gemm_affine_ex

    def step(i, evs=None):
        for j, M in enumerate(ms):
            if evs is not None:
                evs[i][j][0].record(stream)
            rc = fn(*calls[(i * len(ms) + j) % R][j])
            if evs is not None:
                evs[i][j][1].record(stream)
            if rc != 0:
                raise RuntimeError(f"affine GEMM failed: {lib.w4a16_last_error().decode()}")

    warm_up(step, args.warmup)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    value = sum(affine_bytes(M, K, N, g, bits, nmat) for M in ms) * args.steps / wall / 1e9

    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in ms]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, evs)
    torch.cuda.synchronize()
    per_m = {}
    for j, M in enumerate(ms):   # device time per call: K launches of the call back to back
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            fn(*calls[i % R][j])
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.steps
        d = np.array([evs[i][j][0].elapsed_time(evs[i][j][1]) * 1e3 for i in range(args.steps)])
        b = affine_bytes(M, K, N, g, bits, nmat)
        per_m[str(M)] = {"us_per_call": round(us, 3), "GBps": round(b / us / 1e3, 1),
                         "frac_of_peak": round(b / us / 1e3 / PEAK_HBM_GBPS, 4), "bytes": b,
                         "us_lone_event_pair": round(float(np.mean(d)), 3)}
    dom = max(ms, key=lambda M: per_m[str(M)]["us_per_call"])
    us_dom = per_m[str(dom)]["us_per_call"]
    bdom = per_m[str(dom)]["bytes"]
    achieved = bdom / us_dom / 1e3
    form = "codes read at their own width" if native else "split planes" if split else \
        "widened to 4 bits" if widen else "4-bit codes"
    kern = "decode_kernel" if native else "w4a16_gemm_kernel"
    rec = {
        "metric": "W4A16 GEMV/small-M GEMM achieved HBM GB/s (% of peak) and us/call, M=1..16",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"{wl.name} (w = s*q + b, bf16 scales and biases; {form})"
                               f"{' gated pair silu(A x W_gate) * (A x W_up)' if pair else ''}, M in "
                               f"{','.join(map(str, ms))} (one call each per step)",
                   "K": K, "N": N, "group": g, "bits": wl.bits, "ms": list(ms), "out": "fp32",
                   "rotation_copies": R, "pool_MiB": round(R * per_copy / 2 ** 20)},
        "roofline": {"bound": "hbm", "kernel": f"{kern} (affine, {form}{', gated pair' if pair else ''}, M={dom})", "M": dom,
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": load_traffic(f"ffn_up_affine{bits}" + ("_native" if native else "") +
                                             ("_gate_up" if pair else ""), dom, kern),
                     "launches": args.steps,
                     "bytes_per_launch": bdom, "us_per_launch": round(us_dom, 3),
                     "us_per_launch_lone_event_pair": per_m[str(dom)]["us_lone_event_pair"]},
        "per_m": per_m,
    }
    if not args.no_cpu_baseline:
        import oracle
        oracle._load()
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        reps, elapsed, nbytes = 0, 0.0, 0
        while elapsed < args.cpu_seconds or reps == 0:
            for M in ms:
                t = time.perf_counter()
                if pair:
                    oracle.affine_gate_up(x.act[:M], (xg.packed, 4, xg.scales, xg.biases),
                                          (x.packed, 4, x.scales, x.biases), g)
                else:
                    oracle.affine_gemm(x.act[:M], x.packed, x.bits, x.scales, x.biases, g)
                elapsed += time.perf_counter() - t
                nbytes += affine_bytes(M, K, N, g, bits, nmat)
            reps += 1
        rec["cpu_baseline"] = {"value": round(nbytes / elapsed / 1e9, 3), "unit": "GB/s", "cores": threads,
                               "kind": "oracle",
                               "sample": f"{reps} full step(s) (M={','.join(map(str, ms))}, all {N} columns), "
                                         f"{elapsed:.1f} s of oracle time"}
    print(json.dumps(rec), flush=True)
    return 0


def run_prefill(args, lib):
    """The many-row GEMM: one call per M per step, TFLOP/s against the fp16 matrix-core peak."""
    import numpy as np
    import torch
    import verify_matmul_amd as vm
    from verify_matmul_amd import synth

    aff = args.affine   # affine codes read at their own width
    wl = synth.AFFINE_WORKLOADS[f"ffn_up_affine{args.affine_bits}"] if aff else synth.WORKLOADS[args.workload]
    if (not aff and wl.argmax) or args.splits or args.waves_k or args.tile_cols or (aff and args.gate_up):
        print("bench.py: --prefill takes an FFN or attention workload (or --affine, a single matrix) and no launch "
              "knobs", file=sys.stderr)
        return 2
    if aff and args.affine_bits == 7:
        print("bench.py: the affine prompt GEMM reads 1-6 and 8-bit codes", file=sys.stderr)
        return 2
    pair = args.gate_up   # the gated pair silu(A x W_gate) * (A x W_up): 4 M N K flops per call
    nmat = 2 if pair else 1
    ms = tuple(int(x) for x in args.ms.split(",")) if args.ms else (512, 2048)
    K, N, g = wl.K, wl.N, wl.group
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    # prompt-sized activations with the workload's distribution (its own seeded draw)
    rng = np.random.Generator(np.random.PCG64(1000 * wl.index + 8))
    if aff:
        xa = synth.make_affine_inputs(wl)
        act = synth.draw_activations(rng, max(ms), K, 1.0, 0.0, 1.0)
        per_copy = affine_bytes(0, K, N, g, wl.bits)
        qw0 = torch.from_numpy(np.ascontiguousarray(xa.packed).view(np.int32)).to(dev)
        sc = torch.from_numpy(xa.scales.view(np.int16)).to(dev)
        bi = torch.from_numpy(xa.biases.view(np.int16)).to(dev)
        qz = None
    else:
        inp = synth.make_inputs(wl)
        act = synth.draw_activations(rng, max(ms), K, wl.act_sigma, wl.outlier_frac, wl.outlier_mul)
        per_copy = algorithmic_bytes(0, K, N, g, wl.symmetric)
        qw0 = torch.from_numpy(inp.qweight.view(np.int32)).to(dev)
        sc = torch.from_numpy(inp.scales.view(np.int16)).to(dev)
        qz = None if inp.qzeros is None else torch.from_numpy(inp.qzeros.view(np.int32)).to(dev)
    R = max(2, math.ceil(POOL_BYTES / per_copy))
    pool = [qw0.clone() for _ in range(R)]
    if pair:
        gate_inp = synth.make_gate_inputs(wl)
        gw0 = torch.from_numpy(gate_inp.qweight.view(np.int32)).to(dev)
        gpool = [gw0.clone() for _ in range(R)]
        gs = torch.from_numpy(gate_inp.scales.view(np.int16)).to(dev)
        gz = None if gate_inp.qzeros is None else torch.from_numpy(gate_inp.qzeros.view(np.int32)).to(dev)
    a = torch.from_numpy(act.view(np.int16)).to(dev)
    outs = {M: torch.empty((M, N), dtype=torch.float32, device=dev) for M in ms}
    stream = torch.cuda.current_stream()

    def call(i, M):
        if pair:
            vm.w4a16_gemm_gate_up_prefill(a[:M], (gpool[i % R], gs, gz), (pool[i % R], sc, qz), g, outs[M],
                                          stream=stream)
        elif aff:
            vm.w4a16_gemm_affine_bits_prefill(a[:M], pool[i % R], wl.bits, sc, bi, g, outs[M], stream=stream)
        else:
            vm.w4a16_gemm_prefill(a[:M], pool[i % R], sc, qz, g, outs[M], stream=stream)

    def step(i, evs=None):
        for j, M in enumerate(ms):
            if evs is not None:
                evs[i][j][0].record(stream)
            call(i * len(ms) + j, M)
            if evs is not None:
                evs[i][j][1].record(stream)

    warm_up(step, args.warmup)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    flops = sum(2.0 * nmat * M * N * K for M in ms)
    value = flops * args.steps / wall / 1e12
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in ms]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, evs)
    torch.cuda.synchronize()
    per_m, dom, dom_time = {}, None, -1.0
    for j, M in enumerate(ms):
        d = np.array([evs[i][j][0].elapsed_time(evs[i][j][1]) * 1e3 for i in range(args.steps)])
        us = float(np.mean(d))
        f = 2.0 * nmat * M * N * K
        per_m[str(M)] = {"us_per_call": round(us, 3), "us_median": round(float(np.median(d)), 3),
                         "us_p10": round(float(np.percentile(d, 10)), 3),
                         "us_p90": round(float(np.percentile(d, 90)), 3), "TFLOPs": round(f / us / 1e6, 1),
                         "frac_of_peak": round(f / us / 1e6 / PEAK_F16_TFLOPS, 4), "flops": f,
                         "hbm_GBps_weights_once": round((affine_bytes(M, K, N, g, wl.bits) if aff else
                                                         algorithmic_bytes(M, K, N, g, wl.symmetric, matrices=nmat))
                                                        / us / 1e3, 1)}
        if float(np.sum(d)) > dom_time:
            dom, dom_time = M, float(np.sum(d))
    # the dominant call alone, back to back between one event pair on its stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        call(i, dom)
    e1.record(stream)
    torch.cuda.synchronize()
    us_dom = e0.elapsed_time(e1) * 1e3 / args.steps
    f_dom = 2.0 * nmat * dom * N * K
    rec = {
        "metric": "W4A16 prefill GEMM TFLOP/s (% of fp16 matrix-core peak), us/call",
        "value": round(value, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": (f"{wl.name} gated pair silu(A x W_gate) * (A x W_up)" if pair else wl.name) +
                               f", prompt rows M in {','.join(map(str, ms))} (one call each per step)",
                   "K": K, "N": N, "group": g, "ms": list(ms), "out": "fp32", "rotation_copies": R,
                   **({"affine_bits": wl.bits, "scales_biases": "bf16"} if aff else {"symmetric_zero": wl.symmetric})},
        "roofline": {"bound": "mfma", "kernel": f"w4a16_prefill_kernel ({'gated pair, ' if pair else ''}"
                                                f"{f'affine-{wl.bits}, ' if aff else ''}M={dom})", "M": dom,
                     "achieved": round(f_dom / us_dom / 1e6, 1), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(f_dom / us_dom / 1e6 / PEAK_F16_TFLOPS, 4),
                     "traffic": None if pair or aff else load_traffic(args.workload, dom, "w4a16_prefill_kernel"),
                     "launches": args.steps, "flops_per_launch": f_dom, "us_per_launch": round(us_dom, 3),
                     "us_per_launch_lone_event_pair": per_m[str(dom)]["us_per_call"]},
        "per_m": per_m,
    }
    if not args.no_cpu_baseline:
        import oracle
        oracle._load()
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        M = min(ms)
        cols = np.arange(0, N, max(1, N // 256))[:256]   # a bounded sample of columns
        reps, elapsed = 0, 0.0
        while elapsed < args.cpu_seconds or reps == 0:
            t = time.perf_counter()
            if pair:
                oracle.gate_up(act[:M], (gate_inp.qweight, gate_inp.scales, gate_inp.qzeros),
                               (inp.qweight, inp.scales, inp.qzeros), g, cols)
            elif aff:
                oracle.affine_gemm(act[:M], xa.packed, wl.bits, xa.scales, xa.biases, g, cols)
            else:
                oracle.gemm(act[:M], inp.qweight, inp.scales, inp.qzeros, g, cols, with_bound=False)
            elapsed += time.perf_counter() - t
            reps += 1
        rec["cpu_baseline"] = {"value": round(2.0 * nmat * M * len(cols) * K * reps / elapsed / 1e12, 6), "unit": "TFLOP/s",
                               "cores": threads, "kind": "oracle",
                               "sample": f"{reps} call(s) of M={M} rows on {len(cols)} of the {N} columns, "
                                         f"{elapsed:.1f} s of oracle time"}
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
