#!/usr/bin/env python3
"""Benchmark of the gfx950 selective scan on one MI355X.

One step = one ssm_scan_fwd call (prologue, discretisation, in-chunk scan,
chunk carry, readout and gated epilogue) over the Mamba-2.8B-shaped bf16
layer: batch 4, L 4096, dim 5120, dstate 16, z gate on, final state
returned.  Inputs are seeded synthetic tensors already resident in HBM.
The one-token decode step (ssm_state_update, batch 256, dim 5120,
dstate 16) is timed separately in the same run and reported under "decode",
the backward pass (ssm_scan_bwd) of the same layer under "backward", and the
same layer's tokens as one packed row of variable-length sequences, each from
its own initial state (ssm_scan_fwd_ex), under "packed", and the same layer
with the Mamba-3 trapezoidal three-term recurrence (ssm_scan_trap_fwd) under
"trapezoid".  The Mamba-2 SSD layer (ssm_ssd_fwd, MFMA) on a 2.7B-shaped layer
(batch 4, L 4096, 80 heads of 64 channels, state 128, bf16) is under "ssd".

Timing: inputs are resident in HBM; every timed call is preceded, outside
its HIP events, by a read of a 1 GiB buffer that evicts L2 and the Infinity
Cache, so each call reads its inputs from HBM.  ms_per_step is the median of
the timed calls (p10/p90/min beside it); back-to-back timing is reported
under "back_to_back".

Prints ONE JSON line.  Fields beyond the common ones:
  roofline      the step's algorithmic HBM bytes (every input read once, y and
                the final state written once) per call time against the
                8 TB/s HBM peak -- the metric's second half.  The step is the
                packing of B and C (~1% of it) and the scan kernel; the
                scan's rocprofv3 duration is in profiles/;
  alu_issue     the same time against the chip's fp32 VALU issue rate: the
                scan needs 4 fp32 VALU ops + 1 exp per state update, more issue
                time than byte time, so this fraction is the higher one;
  cpu_baseline  the fp64 CPU oracle on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E peak, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, TFLOP/s
# fp32 VALU issue peak without packed-fp32 instructions (this build disables them): 256 CUs x 4 SIMDs x 16 lanes
# per clock x 2.4 GHz = 39.3e12 lane-ops/s, i.e. 78.6 TFLOP/s counting an FMA as 2 flops.  (The 157.3 TFLOP/s
# datasheet figure needs v_pk_fma_f32, two fp32 FMAs per lane per instruction.)
VALU_LANE_OPS_PEAK = 256 * 4 * 16 * 2.4e9
VALU_PEAK_TFLOPS = 2 * VALU_LANE_OPS_PEAK / 1e12
TRANS_SLOTS = 2                 # exp2/log2/rcp: a wave64 issues every ~8-9.6 clocks on a SIMD vs 4 for an fp32 FMA
# VALU issue slots the method itself needs (FMA-equivalents).  Per state update: delta*A, the exp, delta*u*B
# (delta*u is per channel), the fade-and-add fma, the readout fma.  Per (token, channel): bias add, softplus
# (exp, log + 3 ops), delta*u, the D skip fma, SiLU (exp, rcp + 2 ops), the gate multiply.
SLOTS_PER_UPDATE = 4 + 1 * TRANS_SLOTS
SLOTS_PER_TOKEN_CHANNEL = 4 * TRANS_SLOTS + 9
# The backward with the states recomputed once: per state update the recompute (delta*A, exp, delta*u*B, the
# fade-and-add and readout fmas), the adjoint (dh = C dv + dh', dh*h_prev, *a, t_a*A and dh*B accumulations, the dA
# fma, dh*delta*u, dv*h, a*dh) and the sums over channels of the dB, dC terms (2 adds).  Per (token, channel):
# softplus and its derivative (exp, log, exp, rcp + 4 ops), SiLU and its derivative (exp, rcp + 4 ops), and the dv,
# dz, du, d delta, dD and d bias terms (8 ops).
# The trapezoidal rule adds per (token, channel) u/2, the weight (delta' + delta) u'/2 of the previous token's
# input, and the delta (u/2) (C.B) term of the readout (2 ops); the update itself costs what the two-term one does.
TRAP_SLOTS_PER_TOKEN_CHANNEL = SLOTS_PER_TOKEN_CHANNEL + 4
BWD_SLOTS_PER_UPDATE = 4 + TRANS_SLOTS + 9 + 2
BWD_SLOTS_PER_TOKEN_CHANNEL = 6 * TRANS_SLOTS + 16


def scan_bytes(w, with_final=True):
    s = 2 if w.dtype == "bf16" else 4
    n_io = 4 if w.gate else 3  # u, delta, (z), y
    b = w.batch * w.L * w.dim * n_io * s + w.batch * w.L * w.dstate * 2 * s
    b += w.dim * w.dstate * 4 + 2 * w.dim * 4
    if with_final:
        b += w.batch * w.dim * w.dstate * 4
    return b


def decode_bytes(w):
    s = 2 if w.dtype == "bf16" else 4
    return (2 * w.batch * w.dim * w.dstate * 4 + w.batch * w.dim * 4 * s + w.batch * w.dstate * 2 * s
            + w.dim * w.dstate * 4 + 2 * w.dim * 4)


def bwd_bytes(w):
    """Algorithmic bytes of the backward: u, delta, z, B, C, dy read and du, ddelta, dz, dB, dC written once,
    A/D/bias read and dA/dD/dbias written once."""
    s = 2 if w.dtype == "bf16" else 4
    n_io = 7 if w.gate else 5  # u, delta, dy (+ z) read; du, ddelta (+ dz) written
    return (w.batch * w.L * w.dim * n_io * s + w.batch * w.L * w.dstate * 4 * s
            + 2 * (w.dim * w.dstate * 4 + 2 * w.dim * 4))


def scan_slots(w):
    return w.updates * SLOTS_PER_UPDATE + w.batch * w.L * w.dim * SLOTS_PER_TOKEN_CHANNEL


def kernel_source_hash():
    h = hashlib.sha256()
    cdir = os.path.join(ROOT, "selective_state_space_33_amd", "csrc")
    for name in sorted(os.listdir(cdir)):
        with open(os.path.join(cdir, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload_name):
    """HBM bytes per launch from committed rocprofv3 --pmc counters, if taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(workload_name)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def gpu_inputs(x, dtype, dev):
    import numpy as np
    import torch

    def t(a, f32=False):
        if a is None:
            return None
        g = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
        return g if (f32 or dtype == "f32") else g.to(torch.bfloat16)

    return dict(u=t(x["u"]), delta=t(x["delta"]), z=t(x["z"]), B=t(x["B"]), C=t(x["C"]), A=t(x["A"], True),
                D=t(x["D"], True), delta_bias=t(x["delta_bias"], True), h0=t(x.get("h0"), True))


def time_calls(fn, steps, warmup, stream, min_warm_ms=150.0):
    """Average ms per call of `steps` back-to-back calls, after `warmup` calls and at least
    min_warm_ms of warm-up work (the GPU clock takes ~100 ms of load to settle)."""
    import torch

    t_w = time.perf_counter()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    while (time.perf_counter() - t_w) * 1e3 < min_warm_ms:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, wall / steps * 1e3


def time_cold_calls(fn, calls, stream, warmup=0, flush_bytes=1 << 30, min_warm_ms=150.0):
    """Per-call times (ms) with the caches flushed before every call.

    A read over a 1 GiB buffer, outside the events, evicts the inputs from L2 and the 256 MB
    Infinity Cache, so each call reads them from HBM.  It reads rather than writes so that the
    call does not start with the flush's own dirty lines still waiting to be written back.
    `warmup` untimed flushed calls (and at least min_warm_ms of them: the clock takes ~100 ms of
    load to settle) come first; the timed calls are bracketed by device synchronisations.
    Returns min, p10, median, p90 and the wall time of the timed region."""
    import numpy as np
    import torch

    buf = torch.ones(flush_bytes // 4, dtype=torch.float32, device=stream.device)
    t_w = time.perf_counter()
    n_w = 0
    while n_w < max(warmup, 1) or (time.perf_counter() - t_w) * 1e3 < min_warm_ms:
        buf.sum()
        fn()
        n_w += 1
        if n_w % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    t0 = time.perf_counter()
    for start, end in evs:
        buf.sum()
        start.record(stream)
        fn()
        end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del buf
    t = np.asarray([s_.elapsed_time(e_) for s_, e_ in evs])
    return {"calls": calls, "warmup_calls": n_w, "flush_bytes": flush_bytes, "ms_min": float(t.min()),
            "ms_p10": float(np.percentile(t, 10)), "ms_median": float(np.median(t)),
            "ms_p90": float(np.percentile(t, 90)), "wall_s": wall}


def copy_bandwidth(dev, stream, nbytes=1 << 30, steps=20):
    """Device-to-device copy rate of a plain 1 GiB copy, counting bytes read plus bytes written (GB/s)."""
    import torch

    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    ms, _ = time_calls(lambda: dst.copy_(src), steps, 5, stream)
    del src, dst
    return 2 * nbytes / (ms * 1e-3) / 1e9


def host_cores():
    """Cores this process may run on: its CPU affinity, further limited by a cgroup CPU quota if one is set."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            quota, period = f.read().split()[:2]
        if quota != "max":
            n = min(n, max(1, int(int(quota) / int(period))))
    except (OSError, ValueError):
        pass
    return max(1, n)


def cpu_baseline(w, x, budget_s):
    """The fp64 oracle on the first channels of every batch row (full sequence), sized to ~budget_s of wall time.

    Timed with one thread per core this process may use (host_cores) and, on a smaller sample, with one
    thread.  When the whole workload fits in the budget it is run whole, repeatedly, and the median run is
    reported.
    """
    import numpy as np

    from oracle import ref as R

    threads = host_cores()

    def run(nch, nthreads):
        sub = dict(u=x["u"][:, :, :nch], delta=x["delta"][:, :, :nch],
                   z=None if x["z"] is None else x["z"][:, :, :nch], B=x["B"], C=x["C"],
                   A=x["A"][:nch], D=x["D"][:nch], delta_bias=x["delta_bias"][:nch])
        sub = {k: (None if v is None else np.ascontiguousarray(v, dtype=np.float64)) for k, v in sub.items()}
        t0 = time.perf_counter()
        R.scan_fwd(sub["u"], sub["delta"], sub["A"], sub["B"], sub["C"], D=sub["D"], z=sub["z"],
                   delta_bias=sub["delta_bias"], nthreads=nthreads)
        return time.perf_counter() - t0

    per_channel = w.batch * w.L * w.dstate
    probe = min(w.dim, max(1, threads // max(1, w.batch)) * 4)
    dt = run(probe, threads)
    rate = probe * per_channel / dt
    nch = int(min(w.dim, max(probe, 0.8 * budget_s * rate / per_channel)))
    runs = [run(nch, threads)]
    while nch == w.dim and sum(runs) < 0.6 * budget_s and len(runs) < 50:
        runs.append(run(nch, threads))
    dt = float(np.median(runs))
    ups = nch * per_channel / dt
    # one thread, on a sample sized to ~15% of the budget
    nch1 = int(min(w.dim, max(1, 0.15 * budget_s * (rate / threads) / per_channel)))
    dt1 = run(nch1, 1)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    what = "the whole workload" if nch == w.dim else f"channels 0..{nch - 1} of every batch row"
    return {"value": ups, "unit": "updates/s", "cores": threads, "kind": "oracle",
            "host_cpu_count": os.cpu_count(), "single_thread_value": nch1 * per_channel / dt1, "cpu_model": model,
            "sample": f"{w.name}: {what}, all {w.L} tokens, dstate {w.dstate} "
                      f"({nch * per_channel:.3e} updates, median of {len(runs)} runs of {dt:.2f} s; fp64 "
                      f"sequential recurrence, {threads} threads over channels); single thread: channels "
                      f"0..{nch1 - 1} of every batch row ({nch1 * per_channel:.3e} updates in {dt1:.2f} s)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps first (the GPU clock takes ~100 ms of load to settle)")
    ap.add_argument("--workload", default="mamba2p8b_bf16", help="scan workload to time (default: the 2.8B layer)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-packed", action="store_true")
    ap.add_argument("--no-trapezoid", action="store_true")
    ap.add_argument("--no-ssd", action="store_true")
    ap.add_argument("--no-structured", action="store_true")
    ap.add_argument("--packed-mean-len", type=float, default=1024.0,
                    help="mean sequence length of the packed row (log-normal lengths, sigma 1)")
    ap.add_argument("--no-copy", action="store_true", help="skip the plain-copy bandwidth reference")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="instead of the scan, time a plain device copy of this many MiB (calibrates HBM counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: there is no multi-GPU path here (the scan would shard over "
              "batch and channels with no communication, or over the sequence with one exchange of chunk "
              "pairs).", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_mib > 0:
        # A plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters scale the scan's to bytes.
        dev = torch.device("cuda:0")
        n = args.copy_mib * (1 << 20) // 4
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        ms, _ = time_calls(lambda: dst.copy_(src), args.steps, args.warmup, torch.cuda.current_stream(dev))
        nbytes = 4 * n
        print(json.dumps({"metric": "device copy GB/s", "value": 2 * nbytes / (ms * 1e-3) / 1e9, "unit": "GB/s",
                          "copy_bytes_each_way": nbytes, "ms_per_copy": ms, "steps": args.steps}), flush=True)
        return

    from selective_state_space_33_amd import inputs as I
    from selective_state_space_33_amd import ops

    ops.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    w = I.WORKLOADS[args.workload]
    assert w.op == "scan"
    x = I.make_inputs(w, 0)
    g = gpu_inputs(x, w.dtype, dev)
    y = torch.empty_like(g["u"])
    fs = torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device=dev)
    need = ops.ssm_scan_workspace_size(w.batch, w.L, w.dim, w.dstate, g["u"].dtype)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev) if need else None

    def step():
        ops.ssm_scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], D=g["D"], z=g["z"], delta_bias=g["delta_bias"],
                         y=y, final_state=fs, workspace=ws, stream=stream)

    # the contract's timing: each call from HBM (caches flushed before it), median of the timed calls
    cold = time_cold_calls(step, args.steps, stream, warmup=args.warmup)
    ms = cold["ms_median"]
    ups = w.updates / (ms * 1e-3)
    nbytes = scan_bytes(w)
    slots = scan_slots(w)
    achieved_tf = 2.0 * slots / (ms * 1e-3) / 1e12
    achieved_gbs = nbytes / (ms * 1e-3) / 1e9
    traffic = measured_traffic(w.name)
    # back to back, for comparison (inputs may partly hit the Infinity Cache)
    bb_ms, bb_wall_ms = time_calls(step, args.steps, 5, stream)

    out = {
        "metric": "selective-scan state updates/s (B*L*D*N) and % of MI355X HBM roofline",
        "value": ups,
        "unit": "updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "op": "ssm_scan_fwd", "batch": w.batch, "seq_len": w.L, "dim": w.dim,
                   "dstate": w.dstate, "storage_dtype": w.dtype, "compute_dtype": "f32", "z_gate": w.gate,
                   "final_state": True, "workspace_bytes": need, "seed": 0},
        "timing": dict(cold, protocol="1 GiB read before every timed call, outside its HIP events; "
                                      "median of the timed calls"),
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": traffic, "algorithmic_bytes": nbytes,
                     "kernels": "pack_bc_kernel + scan_kernel (one ssm_scan_fwd call)"},
        "alu_issue": {"achieved": achieved_tf, "peak": VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                      "frac": achieved_tf / VALU_PEAK_TFLOPS,
                      "counted": f"algorithmic fp32 VALU issue slots x 2 flops: {SLOTS_PER_UPDATE} per state update, "
                                 f"{SLOTS_PER_TOKEN_CHANNEL} per (token, channel), a transcendental = {TRANS_SLOTS} "
                                 f"slots; peak = non-packed fp32 issue rate"},
        "back_to_back": {"ms_per_step": bb_ms, "wall_ms_per_step": bb_wall_ms, "value": w.updates / (bb_ms * 1e-3),
                         "hbm_frac": nbytes / (bb_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
    }

    if not args.no_copy:
        copy_gbs = copy_bandwidth(dev, stream)
        out["copy_bandwidth"] = {"achieved": copy_gbs, "unit": "GB/s", "bytes_each_way": 1 << 30,
                                 "scan_frac_of_copy": achieved_gbs / copy_gbs}

    if not args.no_structured:
        # The labelled specialisation A[d, n] = (n + 1) * A0[d] (which the synthetic workloads satisfy), detected
        # once on the weight, outside the timed region; the general path above is the headline.
        a0 = ops.structured_A_base(g["A"])
        if a0 is not None and w.dstate <= 16:
            needs_ = ops.ssm_scan_fwd_structured_workspace_size(w.batch, w.L, w.dim, w.dstate, g["u"].dtype)
            wss_ = torch.empty(needs_, dtype=torch.uint8, device=dev)
            ys_ = torch.empty_like(g["u"])
            fs_ = torch.empty_like(fs)

            def sastep():
                ops.ssm_scan_fwd_structured(g["u"], g["delta"], a0, g["B"], g["C"], D=g["D"], z=g["z"],
                                            delta_bias=g["delta_bias"], y=ys_, final_state=fs_, workspace=wss_,
                                            stream=stream)

            sat = time_cold_calls(sastep, args.steps, stream, warmup=10)
            sams = sat["ms_median"]
            out["structured"] = {
                "workload": w.name, "op": "ssm_scan_fwd_structured",
                "specialisation": "A[d,n] = (n+1)*A0[d], detected on the host: one exp per (token, channel), "
                                  "fades by repeated multiplication; not the general path",
                "ms_per_step": sams, "timing": sat, "value": w.updates / (sams * 1e-3), "unit": "updates/s",
                "workspace_bytes": needs_,
                "roofline": {"bound": "hbm", "achieved": nbytes / (sams * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "algorithmic_bytes": nbytes,
                             "frac": nbytes / (sams * 1e-3) / 1e9 / HBM_PEAK_GBS,
                             "traffic": measured_traffic(w.name + ":structured")}}
            del wss_, ys_, fs_

    if not args.no_decode:
        wd = I.WORKLOADS["decode_bf16"]
        xd = I.make_inputs(wd, 0)
        gd = gpu_inputs(xd, wd.dtype, dev)
        yd = torch.empty_like(gd["u"])
        state = gd["h0"]

        def dstep():
            ops.ssm_state_update(state, gd["u"], gd["delta"], gd["A"], gd["B"], gd["C"], D=gd["D"], z=gd["z"],
                                 delta_bias=gd["delta_bias"], y=yd, stream=stream)

        # 179 MB fits the Infinity Cache, so back-to-back steps can hit it; flushed steps cannot
        dcold = time_cold_calls(dstep, max(args.steps, 20), stream, warmup=20)
        dms = dcold["ms_median"]
        db = decode_bytes(wd)
        dgbs = db / (dms * 1e-3) / 1e9
        dbb, _ = time_calls(dstep, max(args.steps, 20), 20, stream)
        out["decode"] = {"workload": wd.name, "op": "ssm_state_update", "ms_per_step": dms,
                         "value": wd.updates / (dms * 1e-3), "unit": "updates/s", "timing": dcold,
                         "roofline": {"bound": "hbm", "achieved": dgbs, "peak": HBM_PEAK_GBS,
                                      "unit": "GB/s", "frac": dgbs / HBM_PEAK_GBS,
                                      "algorithmic_bytes": db, "traffic": measured_traffic(wd.name)},
                         "back_to_back": {"ms_per_step": dbb, "hbm_frac": db / (dbb * 1e-3) / 1e9 / HBM_PEAK_GBS}}
        if "copy_bandwidth" in out:
            out["decode"]["frac_of_copy"] = dgbs / out["copy_bandwidth"]["achieved"]
        del gd, yd, state

    if not args.no_backward:
        dy = torch.empty_like(g["u"]).copy_(g["u"].flip(1))  # any seeded tensor of y's shape serves as dy
        needb = ops.ssm_scan_bwd_workspace_size(w.batch, w.L, w.dim, w.dstate, g["u"].dtype)
        wsb = torch.empty(needb, dtype=torch.uint8, device=dev)

        def bstep():
            ops.ssm_scan_bwd(g["u"], g["delta"], g["A"], g["B"], g["C"], dy, D=g["D"], z=g["z"],
                             delta_bias=g["delta_bias"], workspace=wsb, stream=stream)

        bt = time_cold_calls(bstep, max(args.steps // 5, 10), stream, warmup=5)
        bms = bt["ms_median"]
        bslots = w.updates * BWD_SLOTS_PER_UPDATE + w.batch * w.L * w.dim * BWD_SLOTS_PER_TOKEN_CHANNEL
        btf = 2.0 * bslots / (bms * 1e-3) / 1e12
        bbytes = bwd_bytes(w)
        out["backward"] = {"workload": w.name, "op": "ssm_scan_bwd", "ms_per_step": bms, "timing": bt,
                           "value": w.updates / (bms * 1e-3), "unit": "updates/s", "workspace_bytes": needb,
                           "roofline": {"bound": "hbm", "achieved": bbytes / (bms * 1e-3) / 1e9,
                                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "algorithmic_bytes": bbytes,
                                        "frac": bbytes / (bms * 1e-3) / 1e9 / HBM_PEAK_GBS},
                           "alu_issue": {"achieved": btf, "peak": VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                                         "frac": btf / VALU_PEAK_TFLOPS,
                                         "counted": f"algorithmic fp32 VALU issue slots x 2 flops, states "
                                                    f"recomputed once: {BWD_SLOTS_PER_UPDATE} per state update, "
                                                    f"{BWD_SLOTS_PER_TOKEN_CHANNEL} per (token, channel)"}}
        del dy, wsb

    if not args.no_packed:
        import numpy as np

        # batch x L tokens as one row, cut into a seeded log-normal length mix; every sequence starts from a
        # random state of its own and hands back its final state.
        rng = np.random.default_rng(1)
        cu = I.packed_offsets(rng, w.batch * w.L, args.packed_mean_len)
        nseq = len(cu) - 1
        row = lambda t: t.reshape(1, w.batch * w.L, t.shape[-1])
        pu, pdl, pz, pB, pC = (row(g[k]) for k in ("u", "delta", "z", "B", "C"))
        cu_t = torch.tensor(cu, dtype=torch.int64, device=dev)
        h0 = (torch.randn((nseq, w.dim, w.dstate), generator=torch.Generator().manual_seed(2)) * 0.1).to(dev)
        py = torch.empty_like(pu)
        pfs = torch.empty((nseq, w.dim, w.dstate), dtype=torch.float32, device=dev)
        needp = ops.ssm_scan_fwd_ex_workspace_size(1, w.batch * w.L, w.dim, w.dstate, nseq, pu.dtype)
        wsp = torch.empty(max(needp, 1), dtype=torch.uint8, device=dev)

        def pstep():
            ops.ssm_scan_fwd_ex(pu, pdl, g["A"], pB, pC, D=g["D"], z=pz, delta_bias=g["delta_bias"],
                                initial_state=h0, cu_seqlens=cu_t, y=py, final_state=pfs, workspace=wsp,
                                stream=stream)

        pt = time_cold_calls(pstep, args.steps, stream, warmup=10)
        pms = pt["ms_median"]
        lens = np.diff(cu)
        ptf = 2.0 * slots / (pms * 1e-3) / 1e12
        # the same bytes as the batch layer, plus the initial states read
        pbytes = scan_bytes(w) - w.batch * w.dim * w.dstate * 4 + 2 * nseq * w.dim * w.dstate * 4
        out["packed"] = {"workload": f"{w.name} as 1 x {w.batch * w.L} packed tokens", "op": "ssm_scan_fwd_ex",
                         "sequences": nseq, "len_min": int(lens.min()), "len_median": float(np.median(lens)),
                         "len_max": int(lens.max()), "initial_state": True, "ms_per_step": pms, "timing": pt,
                         "value": w.updates / (pms * 1e-3), "unit": "updates/s",
                         "roofline": {"bound": "hbm", "achieved": pbytes / (pms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                                      "unit": "GB/s", "algorithmic_bytes": pbytes,
                                      "frac": pbytes / (pms * 1e-3) / 1e9 / HBM_PEAK_GBS},
                         "alu_issue": {"achieved": ptf, "peak": VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                                       "frac": ptf / VALU_PEAK_TFLOPS}}
        del py, pfs, wsp, h0

    if not args.no_trapezoid:
        needt = ops.ssm_scan_trap_fwd_workspace_size(w.batch, w.L, w.dim, w.dstate, 0, g["u"].dtype)
        wst = torch.empty(needt, dtype=torch.uint8, device=dev)

        def tstep():
            ops.ssm_scan_trap_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], D=g["D"], z=g["z"],
                                  delta_bias=g["delta_bias"], y=y, final_state=fs, workspace=wst, stream=stream)

        tt = time_cold_calls(tstep, args.steps, stream, warmup=10)
        tms = tt["ms_median"]
        tslots = w.updates * SLOTS_PER_UPDATE + w.batch * w.L * w.dim * TRAP_SLOTS_PER_TOKEN_CHANNEL
        ttf = 2.0 * tslots / (tms * 1e-3) / 1e12
        out["trapezoid"] = {"workload": w.name, "op": "ssm_scan_trap_fwd", "ms_per_step": tms, "timing": tt,
                            "value": w.updates / (tms * 1e-3), "unit": "updates/s", "workspace_bytes": needt,
                            "roofline": {"bound": "hbm", "achieved": nbytes / (tms * 1e-3) / 1e9,
                                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "algorithmic_bytes": nbytes,
                                         "frac": nbytes / (tms * 1e-3) / 1e9 / HBM_PEAK_GBS},
                            "alu_issue": {"achieved": ttf, "peak": VALU_PEAK_TFLOPS,
                                          "unit": "TFLOP/s", "frac": ttf / VALU_PEAK_TFLOPS,
                                          "counted": f"{SLOTS_PER_UPDATE} slots per state update, "
                                                     f"{TRAP_SLOTS_PER_TOKEN_CHANNEL} per (token, channel)"}}
        del wst

    if not args.no_ssd:
        import numpy as np

        cfg = I.SSD_WORKLOADS["mamba2_2p7b_bf16"]
        sb, sL, sH, sP, sN = cfg["batch"], cfg["L"], cfg["heads"], cfg["headdim"], cfg["dstate"]
        xs = I.random_ssd_inputs(np.random.default_rng(0), sb, sL, sH, sP, sN)
        to = lambda a, f32=False: None if a is None else (
            torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev) if f32 else
            torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(torch.bfloat16))
        gs = dict(x=to(xs["x"]), delta=to(xs["delta"]), B=to(xs["B"]), C=to(xs["C"]), z=to(xs["z"]),
                  A=to(xs["A"], True), D=to(xs["D"], True), bias=to(xs["delta_bias"], True))
        del xs
        ys = torch.empty_like(gs["x"])
        fss = torch.empty((sb, sH, sP, sN), dtype=torch.float32, device=dev)
        needs = ops.ssm_ssd_fwd_workspace_size(sb, sL, sH, sP, sN, gs["x"].dtype)
        wss = torch.empty(needs, dtype=torch.uint8, device=dev) if needs else None

        def sstep():
            ops.ssm_ssd_fwd(gs["x"], gs["delta"], gs["A"], gs["B"], gs["C"], D=gs["D"], z=gs["z"],
                            delta_bias=gs["bias"], y=ys, final_state=fss, workspace=wss, stream=stream)

        st_ = time_cold_calls(sstep, max(args.steps // 2, 10), stream, warmup=5)
        sms = st_["ms_median"]
        supd = sb * sL * sH * sP * sN
        # algorithmic bytes: x, z, y, B, C, delta once each (bf16), A, D, bias, the final state (fp32)
        sbytes = sb * sL * sH * sP * 2 * 3 + sb * sL * sN * 2 * 2 + sb * sL * sH * 2 + sb * sH * sP * sN * 4 + sH * 12
        # algorithmic matrix flops of the chunked form (64-token chunks): per (row, chunk) C B^T (2 Q^2 N, shared
        # by the heads); per (row, chunk, head) the intra-chunk product (2 Q^2 P), the inter-chunk readout and the
        # state update (2 Q N P each)
        Q = 64
        nch = (sL + Q - 1) // Q
        sflops = sb * nch * (2 * Q * Q * sN + sH * (2 * Q * Q * sP + 4 * Q * sN * sP))
        sgbs = sbytes / (sms * 1e-3) / 1e9
        stf = sflops / (sms * 1e-3) / 1e12
        out["ssd"] = {"workload": "mamba2_2p7b_bf16 (batch 4, L 4096, 80 heads x 64, state 128)", "op": "ssm_ssd_fwd",
                      "ms_per_step": sms, "timing": st_, "value": supd / (sms * 1e-3), "unit": "updates/s",
                      "roofline": {"bound": "hbm", "achieved": sgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": sgbs / HBM_PEAK_GBS, "algorithmic_bytes": sbytes,
                                   "traffic": measured_traffic("mamba2_2p7b_bf16")},
                      "mfma": {"achieved": stf, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                               "frac": stf / MFMA_BF16_PEAK_TFLOPS, "algorithmic_flops": sflops}}
        del gs, ys, fss, wss

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, x, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
