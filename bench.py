"""Benchmark of the Skip-Softmax FlashAttention forward on one MI355X.

Workload: Wan-like video self-attention, B=1, H=40, S=32760, D=128 (latent
grid 21 x 30 x 52, seed 2), bf16, inputs resident in HBM.  One step is one
forward call at the threshold that skips about 75% of the 64 x 128 tiles
(lambda chosen by the CPU oracle, tests/golden/wan_lambdas.json); every step
is paired with a dense (lambda = 0) call of the same kernel, interleaved, so
the speedup is an in-session ratio.

Printed (one JSON line): effective TFLOP/s of the skip step (dense-equivalent
4 B H S^2 D per call over the call's time) as ``value``; executed TFLOP/s and
MFMA utilisation against the bf16 dense peak; the dense call's numbers; the
speedup; a roofline entry for the kernel; the virtual-tile variant
(fwd_virtual) timed beside the plain skip call with both outputs' relative L1
distance to dense attention; the FP8-score variant (quantize_qk_fp8 +
fwd_fp8) at lambda = 0 and at the timed lambda; the other configurations
(``other_configs``: the Wan-like problem at the sweep's other skip fractions,
the long sequence with sink keys at lambda = 1e-3, the calibrated varlen batch
at target sparsity 0.5, 0.7 and 0.9), each paired with its own lambda = 0
call; and the CPU oracle timed on a bounded sample as a baseline only.

Kernel durations come from two clocks.  Before the parent process touches
the GPU it runs itself once under rocprofv3 --kernel-trace --stats
(``--counters trace``: the same dense and skip calls, interleaved, on the
same inputs), and the traced mean duration of each kernel instance goes
into ``rocprof``; ``roofline`` is computed from the traced skip kernel.  The
timed loop itself is bracketed by HIP events on the launch stream
(``skip_step``, ``dense_step``, ``ms_per_step``, and ``roofline.achieved_events``).
``energy`` holds the socket power (hwmon, read-only) over back-to-back dense
and skip calls after the timed loop, and each call's energy.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--cpu-seconds 15] [--no-trace] [--energy-calls 150]
    python bench.py --power 200      # socket power and energy per call instead
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import math
import os
import shutil
import subprocess
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA peak (published)
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA peak (published)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E bandwidth (published)
METRIC = "effective TFLOP/s + MFMA util at S=32760 H=40 D=128, and speedup vs λ=0 at ~75% skip"
KERNEL_SRC = os.path.join(ROOT, "skip_softmax_flashattention_amd", "csrc", "ssa_fwd.hip")
KERNEL_DENSE = "ssa_fwd_kernel<false, false, false, true>"    # the lambda = 0 instance
KERNEL_SKIP = "ssa_fwd_kernel<false, false, false, false>"    # the instance with the skip test
KERNEL_FP8 = "ssa_fwd_kernel<false, false, true, false>"      # FP8 scores
KERNEL_VIRTUAL = "ssa_fwd_kernel<false, true, false, false>"  # virtual tiles for skipped tiles
SIDE_KERNELS = ("tile_means_kernel", "quant_q_kernel", "quant_k_kernel")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_wan_like.json")


def kernel_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def executed_flops(mask, S, D=128, bq=64, bk=128):
    """2 D r c for QK^T of every tile plus 2 D r c for P.V of every kept tile;
    r, c the tile's valid rows and keys.  mask: [B, H, nQB, nKT] bool (True = skipped)."""
    import numpy as np
    nqb, nkt = mask.shape[-2:]
    r = np.minimum(bq, S - bq * np.arange(nqb)).astype(np.float64)
    c = np.minimum(bk, S - bk * np.arange(nkt)).astype(np.float64)
    rc = r[:, None] * c[None, :]
    qk = 2.0 * D * rc.sum() * mask.shape[0] * mask.shape[1]
    pv = 2.0 * D * (rc[None, None] * (~mask)).sum()
    return qk + pv


def issued_mfma_flops(mask, D=128, bq=64, bk=128):
    """Padded MFMA work issued: every tile runs a full 64 x 128 QK^T, kept tiles a full P.V."""
    tiles = mask.size
    kept = int((~mask).sum())
    return 2.0 * D * bq * bk * (tiles + kept)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def rocprof_trace(steps, warmup, timeout=600):
    """Run this script under rocprofv3 --kernel-trace --stats (the dense and
    skip calls of the headline workload, interleaved, then the FP8-score and
    virtual-tile calls) and return the traced mean duration of each
    ssa_fwd_kernel instance and side kernel, or None when rocprofv3 is
    missing or wrote no statistics.  rocprofv3 can end with a segmentation
    fault after the program and its files are complete; the statistics are
    used whenever they were written."""
    exe = shutil.which("rocprofv3") or ("/opt/rocm/bin/rocprofv3" if os.path.exists("/opt/rocm/bin/rocprofv3") else None)
    if exe is None:
        return None
    out_dir = tempfile.mkdtemp(prefix="ssa_trace_")
    cmd = [exe, "--kernel-trace", "--stats", "--output-format", "csv", "-d", out_dir, "-o", "bench", "--",
           sys.executable, os.path.abspath(__file__), "--counters", "trace", "--steps", str(steps),
           "--warmup", str(warmup)]
    try:
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout, cwd=tempfile.gettempdir(),
                           env={**os.environ, "TMPDIR": tempfile.gettempdir()})
        stats = os.path.join(out_dir, "bench_kernel_stats.csv")
        if not os.path.exists(stats):
            print(f"bench: rocprofv3 wrote no kernel statistics (exit {r.returncode})", file=sys.stderr)
            return None
        kernels = {}
        with open(stats) as f:
            for row in csv.DictReader(f):
                name = row["Name"]
                key = None
                if "ssa_fwd_kernel<" in name:
                    key = "ssa_fwd_kernel<" + name.split("ssa_fwd_kernel<", 1)[1].split(">", 1)[0] + ">"
                else:
                    key = next((k_ for k_ in SIDE_KERNELS if k_ + "(" in name or name.endswith(k_)), None)
                if key is not None:
                    kernels[key] = {"calls": int(row["Calls"]), "mean_ms": float(row["AverageNs"]) / 1e6,
                                    "min_ms": float(row["MinNs"]) / 1e6, "max_ms": float(row["MaxNs"]) / 1e6}
        return {"command": "rocprofv3 --kernel-trace --stats --output-format csv -d DIR -o bench -- python3 bench.py "
                           f"--counters trace --steps {steps} --warmup {warmup}",
                "exit_code": r.returncode, "kernels": kernels}
    except (subprocess.TimeoutExpired, OSError, KeyError, ValueError) as e:
        print(f"bench: rocprofv3 trace failed: {e}", file=sys.stderr)
        return None
    finally:
        shutil.rmtree(out_dir, ignore_errors=True)


def cpu_full_configs():
    """The oracle's recurrence (plain C, single precision) on the two small
    workloads in full: Tiny at each of its factors, Mid at threshold 1e-3."""
    import numpy as np
    import oracle
    from oracle import c_oracle
    from skip_softmax_flashattention_amd import inputs
    orc = c_oracle.oracle()
    out = {}
    for name, w, controls in (("tiny", inputs.tiny(), [("factor", f) for f in (0.0, 0.5, 4.0)]),
                              ("mid", inputs.mid(), [("threshold", 1e-3)])):
        B, H, S, D = w.q.shape
        heads = [tuple(oracle.from_bf16(t[b, h]) for t in (w.q, w.k, w.v)) for b in range(B) for h in range(H)]
        nkt = -(-S // 128)
        c = np.minimum(128, S - 128 * np.arange(nkt)).astype(np.float64)
        r_ = np.minimum(64, S - 64 * np.arange(-(-S // 64))).astype(np.float64)
        for kind, x in controls:
            lam = oracle.resolve_lambda(factor=x, seqlen=S) if kind == "factor" else oracle.resolve_lambda(threshold=x)
            ln = oracle.ln_lambda_f32(lam)
            t0 = time.perf_counter()
            fl = 0.0
            for qd, kd, vd in heads:
                res = orc.skip_head(qd, kd, vd, w.scale, ln)
                fl += 2.0 * D * (r_[:, None] * c[None, :] * (1 + (~res.skipped))).sum()
            dt = time.perf_counter() - t0
            out[f"{name}_{kind}_{x:g}"] = {"seconds": round(dt, 3), "tflops": round(float(fl) / dt / 1e12, 6),
                                           "executed_gflop": round(float(fl) / 1e9, 3)}
    return out


def cpu_baseline(w, ln_lambda, seconds):
    """The oracle's recurrence (the plain-C oracle: single precision, OpenMP
    over query blocks on every host core it is given) on seeded query blocks
    of the workload's heads, whole heads in order, sized to about ``seconds``."""
    import numpy as np
    import oracle
    from oracle import c_oracle
    orc = c_oracle.oracle()
    cores = orc.threads()
    S = w.q.shape[2]
    nqb = -(-S // 64)
    c = np.minimum(128, S - 128 * np.arange(-(-S // 128))).astype(np.float64)

    def run_head(h, n, rng):
        qd, kd, vd = (oracle.from_bf16(t[0, h]) for t in (w.q, w.k, w.v))
        qbs = np.sort(rng.choice(nqb, n, replace=False))
        t0 = time.perf_counter()
        r = orc.skip_head(qd, kd, vd, w.scale, ln_lambda, qblocks=qbs)
        dt = time.perf_counter() - t0
        rows = np.minimum(64, S - 64 * qbs).astype(np.float64)
        return dt, 2.0 * 128 * (rows[:, None] * c[None, :] * (1 + (~r.skipped))).sum()

    rng = np.random.default_rng(7)
    n0 = max(2, cores)
    dt0, _ = run_head(0, min(n0, nqb), rng)
    per_block = dt0 / min(n0, nqb)
    budget = int(max(2, round(seconds / max(per_block, 1e-4))))
    tot_dt = tot_fl = 0.0
    heads = blocks = 0
    while budget > 0 and heads < w.q.shape[1]:
        n = min(nqb, budget)
        dt, fl = run_head(heads, n, rng)
        tot_dt += dt
        tot_fl += fl
        budget -= n
        blocks += n
        heads += 1
    return {"value": round(tot_fl / tot_dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{blocks} query blocks (64 rows x all 256 key tiles) over the first {heads} head(s), seeded, "
                      f"at the same lambda; plain-C float32 recurrence (gcc -O2, OpenMP), {tot_dt:.1f} s",
            "full_configs": cpu_full_configs()}


def copy_reference(launches):
    """A plain elementwise copy of known size (512 MiB read, 512 MiB written):
    the rocprofv3 FETCH_SIZE / WRITE_SIZE it reports calibrate those counters."""
    import torch
    x = torch.ones(128 * 1024 * 1024, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(launches):
        torch.mul(x, 1.0, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"counters_run": "copy", "bytes_read": x.numel() * 4, "bytes_written": y.numel() * 4}), flush=True)


def _power_file():
    import glob
    files = sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*/power1_input"))
    return files[0] if files else None


def _read_w(path):
    with open(path) as f:
        return float(f.read()) / 1e6


def idle_power(quiet=2.0, seconds=1.0):
    """Socket power with no kernel running: the mean of 20 ms samples over
    ``seconds`` after ``quiet`` seconds of rest (the board stays above idle
    for a while after heavy work).  None where the sensor cannot be read."""
    path = _power_file()
    if path is None:
        return None
    time.sleep(quiet)
    t_end, vals = time.time() + seconds, []
    while time.time() < t_end:
        vals.append(_read_w(path))
        time.sleep(0.02)
    return round(sum(vals) / len(vals), 1)


def power_run(ssa, q, k, v, scale, factor, calls, idle_w=None):
    """Socket power while the dense and the skip calls each run back to back.

    Reads the GPU's hwmon power1_input (and power1_cap) every 20 ms from a
    host thread; nothing is written.  ``idle_w`` is measured first (1 s)
    unless given.  Returns a dict, or None where the files cannot be read."""
    import threading
    import numpy as np
    import torch
    path = _power_file()
    if path is None:
        return None
    try:
        cap = _read_w(path.replace("power1_input", "power1_cap"))
    except OSError:
        cap = None
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            samples.append((time.time(), _read_w(path)))
            time.sleep(0.02)
    if idle_w is None:
        idle_w = idle_power(quiet=0.0)
    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    out = {"cap_w": cap, "idle_w": idle_w}
    for name, f in (("dense", 0.0), ("skip", factor)):
        for _ in range(10):
            ssa.fwd(q, k, v, factor=f, scale=scale)
        torch.cuda.synchronize()
        t0 = time.time()
        for _ in range(calls):
            ssa.fwd(q, k, v, factor=f, scale=scale)
        torch.cuda.synchronize()
        t1 = time.time()
        ms = (t1 - t0) / calls * 1e3
        settle = min(0.5, 0.3 * (t1 - t0))   # leave out the start of the run, where power still rises
        watts = float(np.mean([w for t, w in samples if t0 + settle <= t <= t1]))
        out[name] = {"ms_per_call": round(ms, 3), "power_w": round(watts, 1), "energy_j_per_call": round(watts * ms / 1e3, 2)}
    stop.set()
    th.join()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--target", type=float, default=0.75, help="skip fraction of the timed step")
    ap.add_argument("--power", type=int, default=0, metavar="CALLS",
                    help="instead of the benchmark: socket power (hwmon, read-only) over CALLS back-to-back dense "
                         "and then skip calls")
    ap.add_argument("--counters", choices=("dense", "skip", "copy", "trace"), default=None,
                    help="launch only one configuration (or the plain copy reference), for rocprofv3 --pmc; "
                         "'trace' launches the dense and skip calls interleaved, for the kernel trace")
    ap.add_argument("--no-trace", action="store_true", help="skip the rocprofv3 kernel-trace child run")
    ap.add_argument("--energy-calls", type=int, default=150,
                    help="back-to-back dense and skip calls for the energy figures of the benchmark line (0: none)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "multi-GPU sharding of this kernel is not built", file=sys.stderr)
        sys.exit(2)

    # The kernel trace runs first, in a child process, before this process
    # makes any GPU call.
    trace = None
    if args.counters is None and args.power == 0 and not args.no_trace:
        trace = rocprof_trace(args.steps, args.warmup)

    import numpy as np
    import torch

    import skip_softmax_flashattention_amd as ssa
    from skip_softmax_flashattention_amd import inputs

    if args.counters == "copy":
        copy_reference(args.steps)
        return

    ssa.device_check()
    dev = torch.device("cuda:0")
    with open(os.path.join(ROOT, "tests", "golden", "wan_lambdas.json")) as f:
        lams = json.load(f)["lambda"]
    lam = lams[str(args.target)]
    w = inputs.wan()
    q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
    B, H, S, D = q.shape
    factor = lam * S
    dense_flops = 4.0 * B * H * S * S * D
    # idle power for the energy figures, before this process runs any kernel
    idle_w = idle_power() if args.counters is None and args.power == 0 and args.energy_calls > 0 else None

    if args.power > 0:
        print(json.dumps({"power_run": power_run(ssa, q, k, v, w.scale, factor, args.power),
                          "workload": "wan-like B=1 H=40 S=32760 D=128", "lambda": lam,
                          "kernel_sha256_16": kernel_hash()}), flush=True)
        return

    if args.counters == "trace":
        # The timed loop's calls, interleaved, with nothing else: warmup + steps pairs.
        for _ in range(args.warmup + args.steps):
            ssa.fwd(q, k, v, factor=0.0, scale=w.scale)
            ssa.fwd(q, k, v, factor=factor, scale=w.scale)
        torch.cuda.synchronize()
        # Then the two variants at the same lambda: quantisation + FP8-score
        # call, and the virtual-tile call (tile-mean pre-pass + its kernel).
        ws = torch.empty(ssa.virtual_workspace_bytes(B, H, S), dtype=torch.uint8, device=dev)
        for _ in range(args.warmup + args.steps):
            q8, k8, qs8, ks8 = ssa.quantize_qk_fp8(q, k)
            ssa.fwd_fp8(q8, k8, qs8, ks8, v, factor=factor, scale=w.scale)
            ssa.fwd_virtual(q, k, v, factor=factor, scale=w.scale, workspace=ws)
        torch.cuda.synchronize()
        print(json.dumps({"counters_run": "trace", "launches": 7 * (args.warmup + args.steps),
                          "kernel_sha256_16": kernel_hash()}), flush=True)
        return

    if args.counters is not None:
        # Only the requested configuration: warmup + steps launches of one kernel.
        f = 0.0 if args.counters == "dense" else factor
        for _ in range(args.warmup + args.steps):
            ssa.fwd(q, k, v, factor=f, scale=w.scale)
        torch.cuda.synchronize()
        print(json.dumps({"counters_run": args.counters, "launches": args.warmup + args.steps,
                          "kernel_sha256_16": kernel_hash()}), flush=True)
        return

    # Tile decisions of the timed configuration (debug entry point, outside the timed region).
    _, _, cnt_dbg, mask, _ = ssa.fwd_debug(q, k, v, factor=factor, scale=w.scale)
    torch.cuda.synchronize()
    mask_np = mask.cpu().numpy().astype(bool)
    skip_frac = float(mask_np.mean())
    exec_flops = executed_flops(mask_np, S)
    mfma_flops = issued_mfma_flops(mask_np)
    del mask

    def dense():
        return ssa.fwd(q, k, v, factor=0.0, scale=w.scale)

    def skip():
        return ssa.fwd(q, k, v, factor=factor, scale=w.scale)

    for _ in range(args.warmup):
        dense()
        skip()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t_wall = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        dense()
        ev[i][1].record(stream)
        ev[i][2].record(stream)
        _, _, cnt = skip()
        ev[i][3].record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_dense = np.array([a[0].elapsed_time(a[1]) for a in ev])
    ms_skip = np.array([a[2].elapsed_time(a[3]) for a in ev])
    assert int(cnt.sum()) == int(cnt_dbg.sum()) == int(mask_np.sum()), "skip counts changed between calls"

    t_d, t_s = float(ms_dense.mean()), float(ms_skip.mean())
    eff = dense_flops / (t_s * 1e-3) / 1e12
    exe = exec_flops / (t_s * 1e-3) / 1e12
    dense_tf = dense_flops / (t_d * 1e-3) / 1e12

    # One GPU's share of an 8-way head split (Ulysses-style): H = 5 at the same length.
    q5, k5, v5 = (t[:, :5].contiguous() for t in (q, k, v))
    for _ in range(2):
        ssa.fwd(q5, k5, v5, factor=0.0, scale=w.scale)
        ssa.fwd(q5, k5, v5, factor=factor, scale=w.scale)
    torch.cuda.synchronize()
    e5 = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        e5[i][0].record(stream)
        ssa.fwd(q5, k5, v5, factor=0.0, scale=w.scale)
        e5[i][1].record(stream)
        e5[i][2].record(stream)
        ssa.fwd(q5, k5, v5, factor=factor, scale=w.scale)
        e5[i][3].record(stream)
    torch.cuda.synchronize()
    d5 = float(np.mean([a[0].elapsed_time(a[1]) for a in e5]))
    s5 = float(np.mean([a[2].elapsed_time(a[3]) for a in e5]))
    del q5, k5, v5

    # Virtual tiles for the skipped tiles (fwd_virtual, tile-mean pre-pass
    # included) at the same lambda, interleaved with the plain skip call; and
    # each call's relative L1 distance to the dense output.
    ws = torch.empty(ssa.virtual_workspace_bytes(B, H, S), dtype=torch.uint8, device=dev)
    for _ in range(2):
        ssa.fwd_virtual(q, k, v, factor=factor, scale=w.scale, workspace=ws)
    torch.cuda.synchronize()
    ev_v = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(max(5, args.steps // 4))]
    for a in ev_v:
        a[0].record(stream)
        ov, _, _ = ssa.fwd_virtual(q, k, v, factor=factor, scale=w.scale, workspace=ws)
        a[1].record(stream)
        a[2].record(stream)
        os_, _, _ = skip()
        a[3].record(stream)
    torch.cuda.synchronize()
    t_virt = float(np.mean([a[0].elapsed_time(a[1]) for a in ev_v]))
    t_skip2 = float(np.mean([a[2].elapsed_time(a[3]) for a in ev_v]))
    od, _, _ = dense()
    torch.cuda.synchronize()
    den = od.float().abs().sum()
    rel_skip = float((os_.float() - od.float()).abs().sum() / den)
    rel_virt = float((ov.float() - od.float()).abs().sum() / den)
    del ov, os_, od, ws

    # FP8 scores (quantize_qk_fp8 + fwd_fp8): the quantisation pass, then the
    # FP8-score kernel at lambda = 0 and at the timed lambda, interleaved with
    # the bf16 dense call; the FP8 call's own skip fraction at that lambda.
    q8, k8, qs8, ks8 = ssa.quantize_qk_fp8(q, k)
    _, _, c8, mask8, _ = ssa.fwd_fp8(q8, k8, qs8, ks8, v, factor=factor, scale=w.scale, debug=True)
    mask8_np = mask8.cpu().numpy().astype(bool)
    del mask8
    ssa.fwd_fp8(q8, k8, qs8, ks8, v, factor=0.0, scale=w.scale)
    torch.cuda.synchronize()
    n8 = max(5, args.steps // 4)
    ev8 = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(n8)]
    for a in ev8:
        a[0].record(stream)
        ssa.quantize_qk_fp8(q, k)
        a[1].record(stream)
        a[2].record(stream)
        ssa.fwd_fp8(q8, k8, qs8, ks8, v, factor=0.0, scale=w.scale)
        a[3].record(stream)
        a[4].record(stream)
        ssa.fwd_fp8(q8, k8, qs8, ks8, v, factor=factor, scale=w.scale)
        a[5].record(stream)
        a[6].record(stream)
        dense()
        a[7].record(stream)
    torch.cuda.synchronize()
    t8 = [float(np.mean([a[2 * i].elapsed_time(a[2 * i + 1]) for a in ev8])) for i in range(4)]
    fp8_skip_frac = float(c8.sum()) / float(mask_np.size)
    del q8, k8, qs8, ks8, c8

    # The other configurations, each timed against its own lambda = 0 call:
    # the Wan-like problem at the other skip fractions of the sweep, the long
    # sequence with sink keys at lambda = 1e-3, and the calibrated varlen
    # batch at each target sparsity.
    n_side = max(5, args.steps // 4)

    def paired(fd, fs):
        fd()
        fs()
        torch.cuda.synchronize()
        e = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_side)]
        for a in e:
            a[0].record(stream)
            fd()
            a[1].record(stream)
            a[2].record(stream)
            r = fs()
            a[3].record(stream)
        torch.cuda.synchronize()
        return (float(np.mean([a[0].elapsed_time(a[1]) for a in e])),
                float(np.mean([a[2].elapsed_time(a[3]) for a in e])), r)

    def leg(td, ts, flops, skipped, tiles):
        return {"dense_ms": round(td, 4), "skip_ms": round(ts, 4), "skip_fraction": round(skipped / tiles, 4),
                "dense_mfma_util": round(flops / (td * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "effective_tflops": round(flops / (ts * 1e-3) / 1e12, 2), "speedup_vs_dense": round(td / ts, 4)}

    others = {}
    for tgt, lam_t in sorted(lams.items()):
        if abs(float(tgt) - args.target) < 1e-9:
            continue
        td, ts, r = paired(dense, lambda: ssa.fwd(q, k, v, factor=lam_t * S, scale=w.scale))
        others[f"wan_like_skip_{tgt}"] = {"lambda": lam_t, **leg(td, ts, dense_flops, int(r[2].sum()), mask_np.size)}

    wl = inputs.long_seq()
    ql, kl, vl = (t.to(dev) for t in (wl.q, wl.k, wl.v))
    Bl, Hl, Sl, _ = ql.shape
    td, ts, r = paired(lambda: ssa.fwd(ql, kl, vl, factor=0.0, scale=wl.scale),
                       lambda: ssa.fwd(ql, kl, vl, threshold=1e-3, scale=wl.scale))
    others["long_seq_threshold_1e-3"] = dict(
        workload=f"B={Bl} H={Hl} S={Sl} grid 24x32x48, 2% sink keys, seed 3",
        **leg(td, ts, 4.0 * Bl * Hl * Sl * Sl * D, int(r[2].sum()), Bl * Hl * -(-Sl // 64) * -(-Sl // 128)))
    del ql, kl, vl, wl

    wv = inputs.varlen()
    qv, kv, vv = (t.to(dev) for t in (wv.q, wv.k, wv.v))
    cu, smax, lens = wv.cu_seqlens.to(dev), max(wv.seqlens), wv.seqlens
    with open(os.path.join(ROOT, "tests", "golden", "varlen_calibration.json")) as f:
        cal = json.load(f)
    fl_v = sum(4.0 * qv.shape[1] * n * n * D for n in lens)
    for tgt in (0.5, 0.7, 0.9):
        # lengths passed on the host: no read-back of cu_seqlens inside the timed region
        td, ts, r = paired(lambda: ssa.fwd_varlen(qv, kv, vv, cu, smax, factor=0.0, scale=wv.scale, seqlens=lens),
                           lambda: ssa.fwd_varlen(qv, kv, vv, cu, smax, calib=(cal["a"], cal["b"], tgt),
                                                  scale=wv.scale, seqlens=lens))
        cnt_v = r[2].cpu().numpy()
        per_seq, off = [], 0
        for n in lens:
            nqb = -(-n // 64)
            per_seq.append(round(float(cnt_v[:, off:off + nqb].sum()) / (cnt_v.shape[0] * nqb * -(-n // 128)), 4))
            off += nqb
        tiles = sum(cnt_v.shape[0] * -(-n // 64) * -(-n // 128) for n in lens)
        others[f"varlen_calibrated_{tgt}"] = dict(skip_fraction_per_sequence=per_seq,
                                                  **leg(td, ts, fl_v, int(cnt_v.sum()), tiles))
    others["varlen_workload"] = f"H={qv.shape[1]} S_b={lens}, calibrated a={cal['a']:.5f} b={cal['b']:.4f}, seed 4"
    del qv, kv, vv, wv

    # Socket power and energy per call of the timed dense and skip calls, and
    # the energy above idle that each call's work takes (E - P_idle t): while
    # both settle at the same power, their time ratio follows that energy ratio.
    energy = None
    if args.energy_calls > 0:
        energy = power_run(ssa, q, k, v, w.scale, factor, args.energy_calls, idle_w=idle_w)
        if energy is not None:
            p_i = energy["idle_w"]
            work = {n: energy[n]["energy_j_per_call"] - p_i * energy[n]["ms_per_call"] * 1e-3
                    for n in ("dense", "skip")}
            energy["work_energy_j"] = {n: round(x, 2) for n, x in work.items()}
            # time ratio = work-energy ratio x ratio of the power above idle each call holds
            energy["work_energy_ratio"] = round(work["dense"] / work["skip"], 4)
            energy["power_above_idle_ratio"] = round((energy["skip"]["power_w"] - p_i)
                                                     / (energy["dense"]["power_w"] - p_i), 4)
            energy["calls"] = args.energy_calls

    # Roofline of the skip kernel: executed FLOP over its traced mean duration
    # (rocprofv3), else over the HIP-event mean of the timed loop.
    t_trace_s = t_trace_d = None
    if trace is not None:
        ks = trace["kernels"]
        if KERNEL_SKIP in ks and KERNEL_DENSE in ks:
            t_trace_s, t_trace_d = ks[KERNEL_SKIP]["mean_ms"], ks[KERNEL_DENSE]["mean_ms"]
    t_roof = t_trace_s if t_trace_s is not None else t_s
    exe_roof = exec_flops / (t_roof * 1e-3) / 1e12
    rocprof = None
    if trace is not None:
        rocprof = dict(trace)
        if t_trace_s is not None:
            rocprof.update({
                "skip_kernel_mean_ms": round(t_trace_s, 4), "dense_kernel_mean_ms": round(t_trace_d, 4),
                "skip_executed_tflops": round(exec_flops / (t_trace_s * 1e-3) / 1e12, 2),
                "skip_effective_tflops": round(dense_flops / (t_trace_s * 1e-3) / 1e12, 2),
                "skip_mfma_util_issued": round(mfma_flops / (t_trace_s * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "dense_tflops": round(dense_flops / (t_trace_d * 1e-3) / 1e12, 2),
                "dense_mfma_util": round(dense_flops / (t_trace_d * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "speedup_vs_dense": round(t_trace_d / t_trace_s, 4)})
        rocprof["kernels"] = {k_: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v_.items()}
                              for k_, v_ in rocprof["kernels"].items()}

    # The variants' kernels against their own rooflines, from the same trace:
    # the FP8-score kernel against the peak of its FLOP mix (QK^T on fp8,
    # P.V on bf16), the quantiser and the tile-mean pre-pass against HBM.
    variants = None
    if trace is not None:
        ks = trace["kernels"]
        variants = {}
        if KERNEL_FP8 in ks:
            t = ks[KERNEL_FP8]["mean_ms"] * 1e-3
            qk8 = dense_flops / 2.0
            pv8 = executed_flops(mask8_np, S) - qk8
            t_bound = qk8 / (PEAK_FP8_TFLOPS * 1e12) + pv8 / (PEAK_BF16_TFLOPS * 1e12)
            variants["fp8_scores_kernel"] = {
                "kernel": KERNEL_FP8, "bound": "mfma", "kernel_ms": round(t * 1e3, 4),
                "qk_fp8_tflop": round(qk8 / 1e12, 4), "pv_bf16_tflop": round(pv8 / 1e12, 4),
                "achieved": round((qk8 + pv8) / t / 1e12, 2), "peak": round((qk8 + pv8) / t_bound / 1e12, 2),
                "unit": "TFLOP/s", "frac": round(t_bound / t, 4)}
        if all(k_ in ks for k_ in ("quant_q_kernel", "quant_k_kernel")):
            t = (ks["quant_q_kernel"]["mean_ms"] + ks["quant_k_kernel"]["mean_ms"]) * 1e-3
            by = 2 * B * H * S * D * 2 + 2 * B * H * S * D + 4 * B * H * S + 4 * B * H * -(-S // 128)
            variants["fp8_quantize"] = {"kernels": ["quant_q_kernel", "quant_k_kernel"], "bound": "hbm",
                                        "kernel_ms": round(t * 1e3, 4), "bytes": by,
                                        "achieved": round(by / t / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                        "frac": round(by / t / 1e9 / PEAK_HBM_GBS, 4)}
        if "tile_means_kernel" in ks:
            t = ks["tile_means_kernel"]["mean_ms"] * 1e-3
            by = 2 * B * H * S * D * 2 + B * H * -(-S // 128) * 3 * D * 2
            variants["virtual_tile_means"] = {"kernel": "tile_means_kernel", "bound": "hbm",
                                              "kernel_ms": round(t * 1e3, 4), "bytes": by,
                                              "achieved": round(by / t / 1e9, 1), "peak": PEAK_HBM_GBS,
                                              "unit": "GB/s", "frac": round(by / t / 1e9 / PEAK_HBM_GBS, 4)}
        if KERNEL_VIRTUAL in ks and KERNEL_SKIP in ks:
            t = ks[KERNEL_VIRTUAL]["mean_ms"]
            variants["virtual_tiles_kernel"] = {"kernel": KERNEL_VIRTUAL, "kernel_ms": round(t, 4),
                                                "over_plain_skip_kernel": round(t / ks[KERNEL_SKIP]["mean_ms"] - 1, 4)}

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_sha256_16") == kernel_hash():
            traffic = tr.get("traffic")

    out = {
        "metric": METRIC,
        "value": round(eff, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_s, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded grid-local positional embedding + noise (no model activations)",
        "config": {
            "workload": "wan-like video DiT self-attention, B=1 H=40 S=32760 D=128, grid 21x30x52, seed 2",
            "lambda": lam, "factor": factor, "target_skip_fraction": args.target,
            "achieved_skip_fraction": round(skip_frac, 4), "tile": "64x128", "causal": False,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(exe_roof, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(exe_roof / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "kernel": KERNEL_SKIP,
            "timing": "rocprofv3 kernel trace" if t_trace_s is not None else "hip events",
            "kernel_ms": round(t_roof, 4),
            "achieved_events": round(exe, 2),
            "frac_events": round(exe / PEAK_BF16_TFLOPS, 4),
        },
        "rocprof": rocprof,
        "variant_rooflines": variants,
        "skip_step": {
            "ms_mean": round(t_s, 4), "ms_min": round(float(ms_skip.min()), 4),
            "ms_median": round(float(np.median(ms_skip)), 4),
            "effective_tflops": round(eff, 2), "executed_tflops": round(exe, 2),
            "mfma_util_issued": round(mfma_flops / (t_s * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "executed_tflop_per_call": round(exec_flops / 1e12, 4),
        },
        "dense_step": {
            "ms_mean": round(t_d, 4), "ms_min": round(float(ms_dense.min()), 4),
            "ms_median": round(float(np.median(ms_dense)), 4),
            "tflops": round(dense_tf, 2), "mfma_util": round(dense_tf / PEAK_BF16_TFLOPS, 4),
            "tflop_per_call": round(dense_flops / 1e12, 4),
        },
        "speedup_vs_dense": round(t_d / t_s, 4),
        "virtual_tiles": {"ms_mean": round(t_virt, 4), "plain_skip_ms_mean": round(t_skip2, 4),
                          "overhead": round(t_virt / t_skip2 - 1.0, 4),
                          "rel_l1_to_dense": round(rel_virt, 5), "plain_skip_rel_l1_to_dense": round(rel_skip, 5)},
        "fp8_scores": {"quantize_ms": round(t8[0], 4), "dense_ms": round(t8[1], 4), "skip_ms": round(t8[2], 4),
                       "bf16_dense_ms": round(t8[3], 4), "skip_fraction": round(fp8_skip_frac, 4),
                       "dense_effective_tflops": round(dense_flops / (t8[1] * 1e-3) / 1e12, 2),
                       "skip_effective_tflops_incl_quantize": round(dense_flops / ((t8[0] + t8[2]) * 1e-3) / 1e12, 2),
                       "skip_speedup_vs_bf16_dense_incl_quantize": round(t8[3] / (t8[0] + t8[2]), 4)},
        "ulysses8_share": {"heads": 5, "dense_ms": round(d5, 4), "skip_ms": round(s5, 4),
                           "dense_mfma_util": round(dense_flops / 8 / (d5 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                           "speedup_vs_dense": round(d5 / s5, 4)},
        "other_configs": others,
        "energy": energy,
        "timed_wall_s": round(t_wall, 3),
        "kernel_sha256_16": kernel_hash(),
    }
    if not args.no_cpu_baseline:
        import oracle
        out["cpu_baseline"] = cpu_baseline(w, oracle.ln_lambda_f32(oracle.resolve_lambda(factor=factor, seqlen=S)),
                                           args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
