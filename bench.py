#!/usr/bin/env python3
"""Selective-scan benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one ``ssm_scan_fwd`` call over the whole workload (every step of the
hot path: stream the inputs, discretise, recur, read out, D skip, gate, write y
and h_last), with the inputs already resident in HBM.  The headline workload is
the large-channel long scan (batch 4, 5120 channels, 16 states, 4096 steps,
bf16 storage, float32 arithmetic).  Prints one JSON line.

Besides the headline, the line carries:
  * ``roofline``: the dominant kernel (the scan sweep) against the bound that
    limits it, from HIP events recorded on the launch stream around the timed
    region;
  * ``cpu_baseline``: the float64 CPU oracle timed on a bounded sample of the
    same workload on every host core the process may use (independent batch
    rows and channel ranges on parallel threads, each running the unchanged
    oracle), with the single-threaded figure beside it;
  * ``workloads``: the other named workloads (the tiny, page-1 and long-prefill
    scans and the chunked SSD), timed the same way, for context.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks and unit counts.
HBM_PEAK_GBS = 8000.0
N_CU, CLOCK_GHZ = 256, 2.4
# fp32 VALU issue capacity: 128 lanes per CU per clock for ordinary (not
# packed) fp32 instructions on gfx950, i.e. the published 157.3 TFLOP/s fp32
# vector peak with an FMA counted as 2 flops.
VALU_LANES_PER_CU_CLK = 128
VALU_SLOTS_PER_S = N_CU * VALU_LANES_PER_CU_CLK * CLOCK_GHZ * 1e9   # 7.86e13
FP32_VECTOR_TFLOPS = 2 * VALU_SLOTS_PER_S / 1e12                    # 157.3
BF16_MFMA_TFLOPS = 2500.0
# Issue cost of one v_exp_f32 / v_rcp_f32 in full-rate VALU slots on gfx950:
# the transcendental rate is a quarter of the fp32 rate (measured; see the
# VALU-rate probe summary under profiles/).
TRANS_SLOTS = 4.0

HEADLINE = "large_channel_4x5120x4096_bf16"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def measured_traffic(workload: str):
    """HBM bytes per launch counted by rocprofv3 for this workload's kernel, or
    None when no count exists or the kernel source changed since it was taken."""
    import hashlib
    try:
        with open(TRAFFIC_FILE) as f:
            entry = json.load(f).get(workload)
        if entry is None:
            return None
        with open(os.path.join(ROOT, entry["source"]), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != entry["source_sha256"]:
                return None
        return int(entry["bytes_per_launch"])
    except (OSError, ValueError, KeyError):
        return None


def scan_alu_slots_per_element(N: int, has_z: bool, has_d: bool) -> float:
    """VALU slots the method itself needs per (batch, channel, step) element.

    Per state: exp(dt A) (1 transcendental), its argument dt*A (1 mul), the
    input term (dt u) B (1 mul), the update a h + bx (1 fma) and the readout
    C h (1 fma).  Per element: dt*u (1 mul), D u (1 fma), and the gate
    z * 1/(1 + exp(-z)) (exp + rcp transcendentals, 3 mul/add).
    """
    full = 4 * N + 1 + (1 if has_d else 0) + (3 if has_z else 0)
    trans = N + (2 if has_z else 0)
    return full + TRANS_SLOTS * trans


def scan_bwd_alu_slots_per_element(N: int, has_z: bool, has_d: bool) -> float:
    """VALU slots the selective-scan backward needs per element.

    Per state and step: the forward rebuilt from the checkpoint (dt*A, exp,
    (dt u) B, the update: 3 full + 1 transcendental), the readout C h for the
    gate's yhat (1), the adjoint lam = a lam + dyhat C (2), and the sums it
    feeds: du (lam B, 1), ddelta (lam (A (h - bx) + B u): 4), dA (lam dt (h - bx):
    2), dB (lam dt u, 1) and dC (dyhat h, 1).  Per element: dt*u, the gate and
    its derivative (exp, rcp and ~6 mul/add), the D terms (2), du and ddelta
    scaling (2).
    """
    full = 16 * N + 2 + (6 if has_z else 0) + (2 if has_d else 0) + 2
    trans = N + (2 if has_z else 0)
    return full + TRANS_SLOTS * trans


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-context", action="store_true", help="skip the other named workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="target wall time of each oracle baseline leg (single thread, all cores)")
    ap.add_argument("--warm-floor-s", type=float, default=0.05,
                    help="least time of back-to-back untimed headline calls before timing "
                         "(the GPU clocks settle after a few ms of load)")
    ap.add_argument("--cold-reps", type=int, default=30,
                    help="calls timed one at a time after a 512 MiB cache flush (0: skip)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus_requested": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch
    import state_space_model_ssm_amd as ssm
    from state_space_model_ssm_amd.synth import WORKLOADS, ScanShape, SsdShape, make_scan_inputs, make_ssd_inputs

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(1)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    def time_calls(fn, steps, warmup, min_warm_s=0.02):
        """W untimed calls, then more until at least min_warm_s of back-to-back
        calls have run (the GPU clocks settle after a few ms of load, and the
        workloads timed after microsecond-scale ones would otherwise be timed
        partly at lower clocks); then `steps` calls timed with HIP events."""
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t_warm = time.perf_counter()
        while time.perf_counter() - t_warm < min_warm_s:
            for _ in range(4):
                fn()
            torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return e0.elapsed_time(e1) / steps, wall

    flush = {}

    def time_cold(fn, reps):
        """Cold-cache timing: before each call, overwrite a 512 MiB buffer on
        the same stream (evicting L2 and the 256 MB Infinity Cache), then time
        that one call with events.  Returns the median and the 10th/90th
        percentiles in ms."""
        if "buf" not in flush:
            flush["buf"] = torch.empty(128 << 20, dtype=torch.float32, device=dev)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        fn()
        ts = []
        for i in range(reps):
            flush["buf"].fill_(float(i))
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ts.sort()
        pick = lambda q: ts[min(len(ts) - 1, int(q * (len(ts) - 1) + 0.5))]
        return {"median_ms": round(pick(0.5), 5), "p10_ms": round(pick(0.1), 5), "p90_ms": round(pick(0.9), 5),
                "reps": reps}

    def scan_runner(s: ScanShape, host):
        d = {k: (None if v is None else v.to(dev)) for k, v in host.items()}
        y = torch.empty((s.batch, s.dim, s.seqlen), dtype=d["u"].dtype, device=dev)
        h = torch.empty((s.batch, s.dim, s.dstate), dtype=torch.float32, device=dev)
        dims = ssm.ScanDims(batch=s.batch, dim=s.dim, dstate=s.dstate, seqlen=s.seqlen,
                            ngroups=s.ngroups, in_dtype=ssm.SSM_BF16 if s.dtype == "bf16" else ssm.SSM_F32,
                            out_dtype=ssm.SSM_BF16 if s.dtype == "bf16" else ssm.SSM_F32,
                            n_chunks=0, flags=0, workspace=None, workspace_bytes=0)
        chunks = ssm.scan_resolved_chunks(dims)
        need = ssm.scan_workspace_size(dims)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

        def fn():
            ssm.scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"], y=y, h_last=h,
                         workspace=ws, stream=stream)
        return fn, chunks

    def ssd_runner(s: SsdShape, host):
        d = {k: (None if v is None else v.to(dev)) for k, v in host.items()}
        y = torch.empty((s.batch, s.seqlen, s.nheads, s.headdim), dtype=torch.bfloat16, device=dev)
        h = torch.empty((s.batch, s.nheads, s.headdim, s.dstate), dtype=torch.float32, device=dev)

        def fn():
            ssm.ssd_chunked_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"], y=y, h_last=h,
                                stream=stream)
        return fn

    # ---- headline ------------------------------------------------------------
    s = WORKLOADS[args.workload]
    if not isinstance(s, ScanShape):
        raise SystemExit("the headline workload must be a selective scan")
    host = make_scan_inputs(s)
    fn, chunks = scan_runner(s, host)
    ms, wall = time_calls(fn, args.steps, args.warmup, min_warm_s=args.warm_floor_s)
    sec = ms / 1e3
    gelem = s.elements / sec / 1e9
    mbytes = s.metric_bytes()
    hbm_gbs = mbytes / sec / 1e9
    has_z, has_d = host["z"] is not None, host["D"] is not None
    slots = scan_alu_slots_per_element(s.dstate, has_z, has_d) * s.elements
    alu_tflops = 2 * slots / sec / 1e12
    t_hbm = mbytes / (HBM_PEAK_GBS * 1e9)
    t_alu = slots / VALU_SLOTS_PER_S
    if t_alu >= t_hbm:
        roof = {"bound": "alu", "achieved": round(alu_tflops, 3), "peak": round(FP32_VECTOR_TFLOPS, 1),
                "unit": "TFLOP/s", "frac": round(alu_tflops / FP32_VECTOR_TFLOPS, 4),
                "unit_note": "fp32 VALU issue-slot equivalents: the method's slots per element x 2 "
                             "(an FMA is 2 flops in one slot; a transcendental takes 4 slots, "
                             "counted as 8)"}
    else:
        roof = {"bound": "hbm", "achieved": round(hbm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(hbm_gbs / HBM_PEAK_GBS, 4)}
    roof["traffic"] = measured_traffic(args.workload) if chunks == 1 else None
    roof["kernel"] = "scan_row_kernel<bf16,bf16,16,sweep>" if s.dtype == "bf16" else "scan_row_kernel<f32,f32,16,sweep>"
    roof["hbm_gbs"] = round(hbm_gbs, 1)
    roof["hbm_frac"] = round(hbm_gbs / HBM_PEAK_GBS, 4)
    roof["alu_model_us"] = round(t_alu * 1e6, 2)
    roof["hbm_model_us"] = round(t_hbm * 1e6, 2)
    cold = time_cold(fn, args.cold_reps) if args.cold_reps > 0 else None

    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    # ---- context: the other named workloads ------------------------------------
    context = {}
    if not args.no_context:
        for name, w in WORKLOADS.items():
            if name == args.workload:
                continue
            if isinstance(w, ScanShape):
                f, k = scan_runner(w, make_scan_inputs(w))
                reps = 200 if w.elements < 1 << 22 else 20
                wms, _ = time_calls(f, reps, 5)
                context[name] = {"ms": round(wms, 5), "Gelem/s": round(w.elements / wms / 1e6, 2),
                                 "hbm_GB/s": round(w.metric_bytes() / wms / 1e6, 1), "n_chunks": k}
            else:
                f = ssd_runner(w, make_ssd_inputs(w))
                wms, _ = time_calls(f, 50, 5)
                context[name] = {"ms": round(wms, 5), "Gelem/s": round(w.elements / wms / 1e6, 2),
                                 "hbm_GB/s": round(w.metric_bytes() / wms / 1e6, 1),
                                 "hbm_GB/s_with_h_last": round((w.metric_bytes() + w.hlast_bytes()) / wms / 1e6, 1),
                                 "hbm_frac_with_h_last": round((w.metric_bytes() + w.hlast_bytes()) / wms / 1e6 /
                                                               HBM_PEAK_GBS, 4),
                                 "mfma_TFLOP/s": round(ssd_flops(w) / wms / 1e9, 2),
                                 "traffic": measured_traffic(name)}
                if args.cold_reps > 0:
                    context[name]["cold"] = time_cold(f, args.cold_reps)
        context.update(decode_context(ssm, dev, stream, time_calls))
        context.update(extra_context(ssm, dev, stream, time_calls, WORKLOADS, make_scan_inputs, make_ssd_inputs))
    torch.cuda.synchronize()

    # ---- CPU baseline: the float64 oracle on a bounded sample ------------------
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(host, s, args.cpu_seconds)

    out = {
        "metric": "selective-scan Gelem/s (B*D*L) + achieved HBM GB/s as % of MI355X peak",
        "value": round(gelem, 3),
        "unit": "Gelem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": s.batch, "dim": s.dim, "dstate": s.dstate,
                   "seqlen": s.seqlen, "ngroups": s.ngroups, "io_dtype": s.dtype, "gate": has_z,
                   "dskip": has_d, "n_chunks": chunks, "seed": s.seed,
                   "metric_bytes": mbytes, "parallelism": "none (1 GPU)"},
        "hbm_GB/s": round(hbm_gbs, 1),
        "hbm_pct_of_peak": round(100 * hbm_gbs / HBM_PEAK_GBS, 2),
        "wall_s_timed": round(wall, 4),
        "roofline": roof,
        "cold": cold,
        "cpu_baseline": cpu,
        "workloads": context,
    }
    print(json.dumps(out), flush=True)


def extra_context(ssm, dev, stream, time_calls, WORKLOADS, make_scan_inputs, make_ssd_inputs):
    """The scan backward on the long-prefill and large-channel workloads; the
    trapezoidal SSD, both SSD backwards, the rotary step on B and C and the SSD on the rotated
    (per-head) B and C, on the SSD workload's shapes."""
    import torch
    from state_space_model_ssm_amd.synth import make_lam
    out = {}
    for name in ("long_prefill_8x1536x2048_f32", "large_channel_4x5120x4096_bf16"):
        w = WORKLOADS[name]
        d = {k: (None if v is None else v.to(dev)) for k, v in make_scan_inputs(w).items()}
        g = torch.Generator(device="cpu").manual_seed(9)
        dy = torch.randn(w.batch, w.dim, w.seqlen, generator=g).to(d["u"].dtype).to(dev)
        dims = ssm._scan_dims(d["u"], d["B"], ssm._dtype_code(d["u"].dtype), ssm._dtype_code(dy.dtype), 0)
        ws = torch.empty(max(ssm.scan_bwd_workspace_size(dims), 1), dtype=torch.uint8, device=dev)
        ms, _ = time_calls(lambda: ssm.scan_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                                                dy=dy, workspace=ws, stream=stream), 5, 1)
        # ALU model: the backward's own VALU work at the fp32 VALU peak.
        t_alu = scan_bwd_alu_slots_per_element(w.dstate, w.has_z, w.dskip != "none") * w.elements / VALU_SLOTS_PER_S
        out["backward_" + name] = {"ms": round(ms, 4), "Gelem/s": round(w.elements / ms / 1e6, 2),
                                   "workspace_MB": round(ws.numel() / 1e6, 1),
                                   "alu_model_us": round(t_alu * 1e6, 1), "alu_frac": round(t_alu * 1e3 / ms, 4)}
        del d, dy, ws
    # The chunked carry on the shape it is for: one long sequence with too few
    # channels to fill the GPU (1 x 1536 channels x 4096 steps, 16 states,
    # float32: 96 channel blocks of 16 channels).  The library's own chunk
    # count against one chunk and two forced counts.
    from state_space_model_ssm_amd.synth import ScanShape
    w = ScanShape(1, 1536, 16, 4096, 1, "f32", has_z=True, dskip="normal", seed=12)
    d = {k: (None if v is None else v.to(dev)) for k, v in make_scan_inputs(w).items()}
    y = torch.empty_like(d["u"])
    dims = ssm._scan_dims(d["u"], d["B"], ssm._dtype_code(d["u"].dtype), ssm._dtype_code(d["u"].dtype), 0)
    auto = ssm.scan_resolved_chunks(dims)
    entry = {"resolved_chunks": auto}
    for k in (1, auto, 4, 32):
        ws = torch.empty(max(ssm.scan_workspace_size(ssm._scan_dims(d["u"], d["B"], ssm._dtype_code(d["u"].dtype),
                                                                     ssm._dtype_code(d["u"].dtype), k)), 1),
                         dtype=torch.uint8, device=dev)
        ms, _ = time_calls(lambda: ssm.scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"], y=y,
                                                n_chunks=k, workspace=ws, stream=stream), 20, 3)
        entry[f"ms_{k}_chunks"] = round(ms, 5)
    entry["hbm_GB/s_auto"] = round(w.metric_bytes() / entry[f"ms_{auto}_chunks"] / 1e6, 1)
    out["chunked_carry_1x1536x4096_f32"] = entry
    del d, y

    w = WORKLOADS["ssd_32x256_h32p64n128_bf16"]
    d = {k: (None if v is None else v.to(dev)) for k, v in make_ssd_inputs(w).items()}
    lam = make_lam((w.batch, w.seqlen, w.nheads), seed=10).to(dev)
    y = torch.empty_like(d["x"])
    h = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.float32, device=dev)
    ms, _ = time_calls(lambda: ssm.ssd_trap_chunked_fwd(d["x"], d["dt"], lam, d["A"], d["B"], d["C"], d["D"],
                                                        d["z"], y=y, h_last=h, stream=stream), 50, 5)
    nbytes = w.metric_bytes() + w.hlast_bytes() + lam.numel() * 2
    out["ssd_trap_32x256_h32p64n128_bf16"] = {"ms": round(ms, 5), "Gelem/s": round(w.elements / ms / 1e6, 2),
                                              "hbm_GB/s_with_h_last": round(nbytes / ms / 1e6, 1)}
    # The SSD backward on the same shapes (bf16 dy, dh_last absent).  Bytes:
    # x, dt, B, C, dy read and dx, ddt, dB, dC (float32) written once each, the
    # least any backward moves.
    g = torch.Generator(device="cpu").manual_seed(12)
    dy = torch.randn(w.batch, w.seqlen, w.nheads, w.headdim, generator=g).to(torch.bfloat16).to(dev)
    dims = ssm._ssd_dims(d["x"], d["B"], 64, ssm._dtype_code(d["x"].dtype), ssm._dtype_code(dy.dtype))
    ws = torch.empty(max(ssm.ssd_bwd_workspace_size(dims), 1), dtype=torch.uint8, device=dev)
    ms, _ = time_calls(lambda: ssm.ssd_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"], dy=dy,
                                           workspace=ws, stream=stream), 20, 3)
    nbytes = (2 * d["x"].numel() + 2 * d["dt"].numel()) * 2 + 2 * d["B"].numel() * (2 + 4) + dy.numel() * 2
    # MFMA model: per (batch, head, 64-step chunk) the two state updates
    # (2 P N Q each), the shared B C^T tile (2 Q Q N over the 4 heads of a
    # block), dyhat X^T (2 Q Q P), W^T dyhat (half of 2 Q Q P: causal), the
    # three products over headdim or dstate with S_in and dS (2 Q N P each)
    # and dG B, dG^T C (half of 2 Q Q N each): about 7.3 MFLOP for headdim
    # 64, dstate 128, at the bf16 dense peak (without a gate).
    Q, P, N = 64, w.headdim, w.dstate
    chunks = w.batch * w.nheads * ((w.seqlen + Q - 1) // Q)
    flops = chunks * 2.0 * (2 * P * N * Q + Q * Q * N / 4 + Q * Q * P + Q * Q * P / 2 + 3 * Q * N * P + Q * Q * N)
    out["ssd_backward_32x256_h32p64n128_bf16"] = {"ms": round(ms, 5), "Gelem/s": round(w.elements / ms / 1e6, 2),
                                                  "hbm_GB/s_min_bytes": round(nbytes / ms / 1e6, 1),
                                                  "mfma_model_us": round(flops / (BF16_MFMA_TFLOPS * 1e12) * 1e6, 2),
                                                  "min_bytes_model_us": round(nbytes / (HBM_PEAK_GBS * 1e9) * 1e6, 2),
                                                  "workspace_MB": round(ws.numel() / 1e6, 1)}
    # The trapezoidal backward on the same shapes (with the token before the
    # sequence).
    xp = torch.randn(w.batch, w.nheads, w.headdim, generator=g).to(torch.bfloat16).to(dev)
    bp = (torch.randn(w.batch, w.ngroups, w.dstate, generator=g) / w.dstate ** 0.5).to(torch.bfloat16).to(dev)
    ms, _ = time_calls(lambda: ssm.ssd_trap_bwd(d["x"], d["dt"], lam, d["A"], d["B"], d["C"], d["D"], d["z"], dy=dy,
                                                x_prev=xp, B_prev=bp, workspace=ws, stream=stream), 20, 3)
    out["ssd_trap_backward_32x256_h32p64n128_bf16"] = {"ms": round(ms, 5), "Gelem/s": round(w.elements / ms / 1e6, 2),
                                                       "mfma_model_us": round(flops / (BF16_MFMA_TFLOPS * 1e12) * 1e6, 2)}
    del dy, ws, xp, bp
    # The rotary step on the same shapes (one set of angles for all heads),
    # then the SSD on the rotated, per-head B and C.
    from state_space_model_ssm_amd.synth import make_theta
    theta = make_theta((w.batch, w.seqlen, 1, w.dstate // 2), seed=11, dtype="bf16").to(dev)
    rows = w.batch * w.seqlen
    br = torch.empty((w.batch, w.seqlen, w.nheads, w.dstate), dtype=torch.bfloat16, device=dev)
    cr = torch.empty_like(br)
    ang = torch.empty((w.batch, w.nheads, w.dstate // 2), dtype=torch.float32, device=dev)
    ms, _ = time_calls(lambda: ssm.rope_bc(d["dt"], theta, d["B"], d["C"], B_rot=br, C_rot=cr, angle_last=ang,
                                           stream=stream), 50, 5)
    # Bytes: dt, theta, B and C read once; B_rot, C_rot and the angles written.
    nbytes = (d["dt"].numel() + theta.numel() + d["B"].numel() + d["C"].numel()) * 2 + \
        (br.numel() + cr.numel()) * 2 + ang.numel() * 4
    out["rope_bc_32x256_h32n128_bf16"] = {"ms": round(ms, 5), "hbm_GB/s": round(nbytes / ms / 1e6, 1),
                                          "hbm_frac": round(nbytes / ms / 1e6 / 8000.0, 4),
                                          "rows": rows, "traffic": measured_traffic("rope_bc_32x256_h32n128_bf16")}
    # The rotary step's backward on the same shapes, for float32 upstream
    # gradients of B_rot and C_rot (as the SSD backward writes dB and dC).
    # Least bytes: dt, theta, B, C and the two upstream gradients read once;
    # ddt, dtheta, dB, dC and dangle0 (float32) written once.
    gdev = torch.Generator(device=dev)
    gdev.manual_seed(13)
    gbr = torch.randn(br.shape, generator=gdev, device=dev)
    gcr = torch.randn(br.shape, generator=gdev, device=dev)
    rdims = ssm.RopeDims(batch=w.batch, seqlen=w.seqlen, nheads=w.nheads, ngroups=w.ngroups, dstate=w.dstate,
                         theta_heads=1, in_dtype=ssm.SSM_BF16, out_dtype=ssm.SSM_F32, flags=0, reserved=0)
    rws = torch.empty(max(ssm.rope_bc_bwd_workspace_size(rdims), 1), dtype=torch.uint8, device=dev)
    ms, _ = time_calls(lambda: ssm.rope_bc_bwd(d["dt"], theta, d["B"], d["C"], dB_rot=gbr, dC_rot=gcr,
                                               angle0=ang, workspace=rws, stream=stream), 20, 3)
    nbytes = (d["dt"].numel() + theta.numel() + d["B"].numel() + d["C"].numel()) * 2 + \
        (gbr.numel() + gcr.numel()) * 4 + (d["dt"].numel() + theta.numel() + d["B"].numel() + d["C"].numel()) * 4 + \
        2 * ang.numel() * 4
    out["rope_bc_backward_32x256_h32n128_bf16"] = {"ms": round(ms, 5), "hbm_GB/s_min_bytes": round(nbytes / ms / 1e6, 1),
                                                   "min_bytes_MB": round(nbytes / 1e6, 1),
                                                   "workspace_MB": round(rws.numel() / 1e6, 1),
                                                   "traffic": measured_traffic("rope_bc_bwd_32x256_h32n128_bf16")}
    del gbr, gcr, rws
    # The Mamba-3 layer's backward on the same shapes, given the fused rotary
    # SSD forward: the rotated B and C recomputed, the SSD backward on them
    # (ngroups = nheads), then the rotary backward on its dB and dC.
    rdy = torch.randn(w.batch, w.seqlen, w.nheads, w.headdim, generator=gdev, device=dev).to(torch.bfloat16)
    gdims = ssm._ssd_dims(d["x"], br, 64, ssm._dtype_code(d["x"].dtype), ssm._dtype_code(rdy.dtype))
    gws = torch.empty(max(ssm.ssd_bwd_workspace_size(gdims), 1), dtype=torch.uint8, device=dev)
    rws = torch.empty(max(ssm.rope_bc_bwd_workspace_size(rdims), 1), dtype=torch.uint8, device=dev)

    def layer_bwd():
        ssm.rope_bc(d["dt"], theta, d["B"], d["C"], B_rot=br, C_rot=cr, return_angle_last=False, stream=stream)
        gs = ssm.ssd_bwd(d["x"], d["dt"], d["A"], br, cr, d["D"], d["z"], dy=rdy, workspace=gws, stream=stream)
        ssm.rope_bc_bwd(d["dt"], theta, d["B"], d["C"], dB_rot=gs["dB"], dC_rot=gs["dC"], workspace=rws,
                        stream=stream)
    ms, _ = time_calls(layer_bwd, 10, 2)
    out["mamba3_layer_backward_32x256_h32p64n128_bf16"] = {"ms": round(ms, 5),
                                                            "parts": "rope_bc + ssd_bwd (ngroups = nheads) + "
                                                                     "rope_bc_bwd"}
    del rdy, gws, rws
    ms, _ = time_calls(lambda: ssm.ssd_chunked_fwd(d["x"], d["dt"], d["A"], br, cr, d["D"], d["z"], y=y,
                                                   h_last=h, stream=stream), 50, 5)
    out["ssd_rotated_32x256_h32p64n128_bf16"] = {"ms": round(ms, 5), "Gelem/s": round(w.elements / ms / 1e6, 2),
                                                 "ngroups": w.nheads}
    unfused = out["rope_bc_32x256_h32n128_bf16"]["ms"] + ms
    # The same rotated prefill fused in one kernel (the rotated B and C stay in
    # LDS): bytes are the plain SSD's plus theta and the angles.
    nbytes = w.metric_bytes() + w.hlast_bytes() + theta.numel() * 2 + ang.numel() * 4
    ms, _ = time_calls(lambda: ssm.ssd_rope_chunked_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], theta, d["D"],
                                                        d["z"], angle_last=ang, y=y, h_last=h, stream=stream), 50, 5)
    out["ssd_rope_fused_32x256_h32p64n128_bf16"] = {"ms": round(ms, 5), "Gelem/s": round(w.elements / ms / 1e6, 2),
                                                    "hbm_GB/s": round(nbytes / ms / 1e6, 1),
                                                    "unfused_ms": round(unfused, 5)}
    bl = torch.empty((w.batch, w.nheads, w.dstate), dtype=torch.bfloat16, device=dev)
    ms, _ = time_calls(lambda: ssm.ssd_rope_trap_chunked_fwd(d["x"], d["dt"], lam, d["A"], d["B"], d["C"], theta,
                                                             d["D"], d["z"], angle_last=ang, B_last=bl, y=y,
                                                             h_last=h, stream=stream), 50, 5)
    out["ssd_rope_trap_fused_32x256_h32p64n128_bf16"] = {"ms": round(ms, 5),
                                                         "Gelem/s": round(w.elements / ms / 1e6, 2)}
    return out


def decode_context(ssm, dev, stream, time_calls):
    """Single-token decode steps at the large workloads' state shapes: the scan
    step on the large-channel state (batch 4, 5120 channels, 16 states) and
    the SSD step on the SSD workload's state (batch 32, 32 heads x 64, 128
    states).  HBM-bound on the state: it is read and written once per step."""
    import torch
    from state_space_model_ssm_amd.synth import make_state
    g = torch.Generator(device="cpu").manual_seed(6)
    out = {}

    def rnd(*shape, dtype=torch.bfloat16, pos=False):
        t = torch.randn(*shape, generator=g)
        return (t.abs() * 0.01 if pos else t).to(dtype).to(dev)

    b, d, n = 4, 5120, 16
    u, dl, z = rnd(b, d), rnd(b, d, pos=True), rnd(b, d)
    A = -torch.rand(d, n, generator=g).add(0.5).to(dev)
    Bm, Cm, D = rnd(b, 1, n), rnd(b, 1, n), torch.ones(d, device=dev)
    state = make_state((b, d, n), seed=7).to(dev)
    y = torch.empty(b, d, dtype=torch.bfloat16, device=dev)
    ms, _ = time_calls(lambda: ssm.scan_step(u, dl, A, Bm, Cm, D, z, state=state, y=y, stream=stream), 200, 10)
    nbytes = 2 * state.numel() * 4 + 4 * b * d * 2 + b * d * 2
    out["decode_scan_step_4x5120_n16_bf16"] = {"ms": round(ms, 5), "state_MB": round(state.numel() * 4 / 1e6, 2),
                                               "hbm_GB/s": round(nbytes / ms / 1e6, 1)}
    b, H, P, n = 32, 32, 64, 128
    x, dt, z = rnd(b, H, P), rnd(b, H, pos=True), None
    Ah = -torch.rand(H, generator=g).add(0.5).to(dev)
    Bm, Cm, Dh = rnd(b, 1, n), rnd(b, 1, n), torch.ones(H, device=dev)
    state = make_state((b, H, P, n), seed=8, scale=0.1).to(dev)
    y = torch.empty(b, H, P, dtype=torch.bfloat16, device=dev)
    ms, _ = time_calls(lambda: ssm.ssd_step(x, dt, Ah, Bm, Cm, Dh, z, state=state, y=y, stream=stream), 200, 10)
    nbytes = 2 * state.numel() * 4 + 2 * x.numel() * 2
    out["decode_ssd_step_32xh32p64_n128_bf16"] = {"ms": round(ms, 5), "state_MB": round(state.numel() * 4 / 1e6, 2),
                                                  "hbm_GB/s": round(nbytes / ms / 1e6, 1),
                                                  "hbm_frac": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4)}
    return out


def ssd_flops(w) -> float:
    """Matrix-core flops of the chunked SSD per call (the s2-s6 contractions)."""
    Q, P, N = w.chunk, w.headdim, w.dstate
    chunks = -(-w.seqlen // Q)
    per_bc = 2 * Q * Q * N                       # C B^T, once per (batch, chunk) and group
    per_bch = 2 * Q * Q * P + 2 * N * P * Q + 2 * Q * N * P   # M X, chunk state, C S^T
    return w.batch * chunks * (per_bc * w.ngroups + per_bch * w.nheads)


def _channel_units(s, nch, per_unit):
    """The first nch (batch, channel) rows of the workload, batch-major, as
    (batch row, first channel, channel count) units of at most per_unit
    channels (one group)."""
    units, done, b = [], 0, 0
    while done < nch:
        take = min(nch - done, s.dim)
        for d0 in range(0, take, per_unit):
            units.append((b, d0, min(per_unit, take - d0)))
        done += take
        b += 1
    return units


def _run_units(oracle, h64, units, threads):
    """The unchanged oracle on each unit's contiguous slice of the float64
    inputs; `threads` host threads (the oracle's C call releases the GIL)."""
    from concurrent.futures import ThreadPoolExecutor

    def one(unit):
        b, d0, n = unit
        sl = lambda k: None if h64[k] is None else h64[k][b:b + 1, d0:d0 + n]
        oracle.scan(sl("u"), sl("delta"), h64["A"][d0:d0 + n], h64["B"][b:b + 1], h64["C"][b:b + 1],
                    None if h64["D"] is None else h64["D"][d0:d0 + n], sl("z"))

    if threads == 1:
        for unit in units:
            one(unit)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, units))


def cpu_baseline(host, s, seconds):
    """The float64 oracle on the host: a bounded sample of the workload (the
    first channels, batch-major, every step) timed single-threaded and on
    every core in the process's affinity set, each leg aiming at `seconds` of
    wall time.  The inputs are widened to float64 before the clock starts."""
    import oracle
    oracle.build(force=False)
    if s.ngroups != 1:
        raise SystemExit("cpu baseline sample assumes one group")
    h64 = {k: (None if v is None else oracle.f64(v)) for k, v in host.items()}
    total = s.batch * s.dim
    probe = 16
    t0 = time.perf_counter()
    _run_units(oracle, h64, _channel_units(s, probe, probe), 1)
    per_ch = (time.perf_counter() - t0) / probe
    legs = {}
    cores = len(os.sched_getaffinity(0))
    for threads in (1, cores):
        nch = int(max(probe, min(total, threads * seconds / max(per_ch, 1e-9))))
        per_unit = nch if threads == 1 else max(1, -(-min(nch, s.dim) // (4 * threads)))
        units = _channel_units(s, nch, per_unit)
        t0 = time.perf_counter()
        _run_units(oracle, h64, units, threads)
        dt = time.perf_counter() - t0
        legs[threads] = {"value": round(nch * s.seqlen / dt / 1e9, 6), "unit": "Gelem/s", "cores": threads,
                         "kind": "oracle", "seconds": round(dt, 3),
                         "sample": f"first {nch} of {total} channels (batch-major), all {s.seqlen} steps; "
                                   f"float64 recurrence on {threads} host thread(s)"
                                   + ("" if threads == 1 else f" over {len(units)} channel ranges")}
    out = dict(legs[cores])
    out["single_thread"] = legs[1]
    return out


if __name__ == "__main__":
    main()
