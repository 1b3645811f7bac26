#!/usr/bin/env python3
"""Throughput of the chunkwise gated delta-rule forward and the decode step
on one MI355X, with roofline fractions and the fp64 CPU oracle as baseline.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

A step is one kda_chunk_fwd call over the Complex KDA workload (B=2, H=16,
T=8192, dk=dv=128, bf16 inputs, fp32 state, chunk 64): 16,384 tokens. Two
seeded input sets alternate so the 256 MB last-level cache cannot hold the
whole working set. The other forward workloads are timed the same way and
reported under "configs": KDA (B=4, H=16, T=4096), GDN with eight packed
sequences (H=32, T=110,440; one input set, its 2.7 GB of inputs dwarf the
cache) and the tiny fp32 case. The forward workloads run back to back with
no host work in between, the headline last, so that its W warm-up calls and
K timed calls run at the clock the device holds under sustained work (after
an idle period the clock needs about 20 ms of load to ramp up). The GPU
clock is read from sysfs while the timed calls are still executing.
The decode step (N=256 sequences, H=32, d=128, fp32 state of 512 MiB updated
in place) is timed as one block of 128 consecutive steps, and set beside a
plain device copy of the same 512 MiB (read and written) as a practical
bandwidth ceiling. The backward
(kda_chunk_bwd, gradients of every input for given dO and dS_T) is timed on
the same forward workload, in both forms, and so is the erase/write-gate
backward (kda_chunk_bwd_ew) on that shape; the erase/write forward
(kda_chunk_fwd_ew) is timed beside the direct one. Forward and backward are also timed at 32k tokens
per step (B=4, H=16, T=8192) with the KDA and the Complex KDA gate recipes,
for the throughput ratio of the two.
Timing uses HIP events recorded on the stream the kernels run on. The fp64
CPU oracle is timed on the host cores beside the headline, the backward and
each other forward workload (a bounded sample each). Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tokens/s KDA chunk fwd (H=16,d=128,T=8192) + decode GB/s, % roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
FP32_VECTOR_PEAK_TFLOPS = 157.3
FP32_MFMA_PEAK_TFLOPS = 157.3


def fwd_bytes_per_head_token(dk: int, dv: int, scalar_gate: bool, in_bytes: int = 2) -> int:
    """Compulsory HBM bytes per (token, head): q, k, v, gate, beta read once
    in the input dtype, o written once in fp32."""
    gate = 1 if scalar_gate else dk
    return in_bytes * (2 * dk + dv + gate + 1) + 4 * dv


def fwd_flops_per_head_token(dk: int, dv: int, C: int = 64) -> int:
    """Algorithmic flops of the chunkwise form per (token, head) at chunk 64:
    full CxC tiles for the gated Gram matrices A and P and for T(Gamma K),
    T V and P U, plus the three state contractions."""
    return 2 * C * (3 * dk + 2 * dv) + 6 * dk * dv


def bwd_bytes_per_head_token(dk: int, dv: int, in_bytes: int = 2) -> int:
    """Compulsory HBM bytes of the backward per (token, head): q, k, v, gate,
    beta read in the input dtype, dO read in fp32, dq, dk, dgate, dv, dbeta
    written in fp32."""
    return in_bytes * (3 * dk + dv + 1) + 4 * dv + 4 * (3 * dk + dv + 1)


def bwd_flops_per_head_token(dk: int, dv: int) -> int:
    """fp32 flops of the token-form adjoint per (token, head): the forward
    step that rebuilds the state (gate scale, S'^T k, rank-one update: 5 per
    state element) and the adjoint step (18 per state element: S', q dO^T,
    dS^T k, S_t dO, dS u, S' dpred, dS', dalpha, Diag(alpha) dS')."""
    return 23 * dk * dv


def cbwd_flops_per_head_chunk(dk: int, dv: int, C: int = 64) -> int:
    """Algorithmic fp32 matrix flops of the chunkwise backward per (chunk,
    head), each contraction counted once (2 flops per multiply-add) and a
    lower-triangular C x C operand at half:
      C x dk x dv, 8 of them: W S and K_end^T U (forward state step),
        K_end dS', (Gamma Q)^T dO and W^T dU (adjoint step), dO S^T, dU S^T
        and U dS'^T (gradients);
      lower C x C by dv columns, 5: X(beta V), P^T dO, dO U^T, dU (beta V)^T,
        X^T dU;
      lower C x C by dk columns, 8: the gated Gram matrices G and P,
        W = X(beta Gamma K), dW (beta Gamma K)^T, X^T dW and the three level
        products of the gate side;
      C^3 / 3 multiply-adds, 3: the inverse X, dX X^T and X^T T."""
    return 16 * C * dk * dv + 5 * C * C * dv + 8 * C * C * dk + 2 * C ** 3


def decode_bytes_per_head_step(dk: int, dv: int, in_bytes: int = 2) -> int:
    return 8 * dk * dv + in_bytes * (3 * dk + dv + 1) + 4 * dv


def measured_traffic():
    """Measured HBM bytes per forward call, per decode step and per
    chunkwise-backward call, from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary (profiles/hbm_traffic_ckda.txt); None for a group whose
    kernel sources have changed since its counters were taken."""
    import hashlib
    try:
        with open(os.path.join(ROOT, "profiles", "hbm_traffic_ckda.txt")) as f:
            groups = json.load(f).get("groups", {})
    except (OSError, ValueError):
        return None, None, None

    def get(name, key):
        g = groups.get(name)
        if not g:
            return None
        for rel, digest in g.get("sources_sha256", {}).items():
            try:
                with open(os.path.join(ROOT, rel), "rb") as f:
                    if hashlib.sha256(f.read()).hexdigest() != digest:
                        return None
            except OSError:
                return None
        return g.get(key)

    return (get("forward", "bytes_per_call"), get("decode", "bytes_per_step"), get("backward", "bytes_per_call"))


def time_region(fn, iters: int, stream):
    import torch
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(iters):
        fn(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / iters   # ms per call


def copy_bandwidth(dev, stream, mib: int = 512, iters: int = 20) -> dict:
    """Read + write GB/s of a plain device copy of `mib` MiB (the size of the
    decode state), two ways: hipMemcpy's copy kernel (Tensor.copy_) and torch's
    vectorized elementwise kernel (a multiply by one). A practical ceiling for
    streaming kernels on this machine, beside the 8 TB/s peak."""
    import torch
    src = torch.ones(mib << 18, device=dev, dtype=torch.float32)
    dst = torch.empty_like(src)
    nbytes = 2 * src.numel() * 4
    res = {}
    for name, fn in (("memcpy", lambda i: dst.copy_(src)), ("elementwise", lambda i: torch.mul(src, 1.0, out=dst))):
        for i in range(5):
            fn(i)
        res[name] = round(nbytes / (time_region(fn, iters, stream) * 1e-3) / 1e9, 1)
    del src, dst
    return res


def per_call_ms(fn, iters: int, stream):
    """Median and minimum of single-call durations (events around each call),
    measured after the bracketed region."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        fn(i)
        b.record(stream)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    return t[len(t) // 2], t[0]


def gpu_clock():
    """The GPU clock line of rocm-smi, or None where it is not available."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=20)
    except (OSError, subprocess.SubprocessError):
        return None
    for line in r.stdout.splitlines():
        if "sclk" in line.lower():
            return " ".join(line.split())
    return None


def sclk_now():
    """The active shader-clock level of the first GPU in sysfs (the line the
    driver marks with '*', e.g. '1: 2400Mhz'), or None where unreadable."""
    import glob
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        return line.strip().rstrip("*").strip()
        except OSError:
            continue
    return None


def timed_with_clock(fn, iters: int, stream):
    """time_region, plus the shader clock read after the calls are enqueued
    and before the device has finished them (so, during the timed work)."""
    import torch
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(iters):
        fn(i)
    end.record(stream)
    clk = sclk_now()
    busy = not end.query()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / iters, clk if busy else None


def walker_name(bf16: bool, dk: int, chunk: int, slices: int, cus: int) -> str:
    """The state kernel kda_chunk_fwd launches for a shape (same rule as the
    library's dispatcher)."""
    if not bf16:
        return "chunk_state_kernel"
    if dk == 128 and chunk == 64:
        return "chunk_state_slice_kernel" if slices <= cus else "chunk_state_quad_kernel"
    if chunk == 64 and dk >= 64:
        return "chunk_state_pair_kernel"
    return "chunk_state_kernel"


def forward_leg(kda, name, sets, w, warmup, steps, stream, dev, with_clock=False):
    """Warm-up, then `steps` timed kda_chunk_fwd calls rotating over the input
    sets; the prep and state launches timed on their own. Returns the
    measurements and the (call, stage) closures."""
    import torch
    B, H, T, dk, dv, C = w.B, w.H, w.T, w.dk, w.dv, w.chunk
    N = w.n_seqs
    varlen = w.cu_seqlens is not None
    o = torch.empty((B, T, H, dv), device=dev, dtype=torch.float32)
    ST = torch.empty((N, H, dk, dv), device=dev, dtype=torch.float32)
    ws = torch.empty(kda.workspace_bytes(B, H, T, dk, dv, C, N, varlen, w.dtype), device=dev, dtype=torch.uint8)

    def fwd(i, stage=kda.STAGE_ALL):
        q, k, v, g, b, cu = sets[i % len(sets)]
        kda.chunk_fwd(q, k, v, g, b, cu_seqlens=cu, chunk=C, gate_kind=w.gate_kind, out=o, S_T=ST, workspace=ws,
                      stage=stage)

    for i in range(warmup):
        fwd(i)
    if with_clock:
        ms, clk = timed_with_clock(fwd, steps, stream)
    else:
        ms, clk = time_region(fwd, steps, stream), None
    ms_med, ms_min = per_call_ms(fwd, min(steps, 200), stream)
    ms_prep = time_region(lambda i: fwd(i, kda.STAGE_PREP), min(steps, 50), stream)
    fwd(0, kda.STAGE_PREP)
    ms_state = time_region(lambda i: fwd(0, kda.STAGE_STATE), min(steps, 50), stream)
    status = kda.fwd_status(ws)
    tokens = B * T
    head_tokens = tokens * H
    in_bytes = 2 if w.dtype == torch.bfloat16 else 4
    alg_bytes = head_tokens * fwd_bytes_per_head_token(dk, dv, w.gate_kind == 1, in_bytes) + N * H * dk * dv * 4
    alg_flops = head_tokens * fwd_flops_per_head_token(dk, dv)
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    walker = walker_name(w.dtype == torch.bfloat16, dk, C, N * H * (dv // 16), cus)
    rec = {
        "workload": name, "B": B, "H": H, "T": T, "dk": dk, "dv": dv, "chunk": C, "sequences": N,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32", "input_sets": len(sets),
        "ms_per_call": round(ms, 4), "tokens_per_s": round(tokens / (ms * 1e-3), 1),
        "hbm": {"achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                "bytes_per_launch": alg_bytes},
        "mfma_frac_algorithmic": round(alg_flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "kernels_ms": {"chunk_prep_kernel": round(ms_prep, 4), walker: round(ms_state, 4)},
        "per_call_ms": {"median": round(ms_med, 4), "min": round(ms_min, 4)},
        "status": kda.strerror(status),
    }
    if with_clock:
        rec["sclk_during_timed_calls"] = clk
    print("[bench] %s %.4f ms/call (prep %.4f, state %.4f), %.1f M tokens/s"
          % (name, ms, ms_prep, ms_state, tokens / (ms * 1e-3) / 1e6), file=sys.stderr, flush=True)
    return rec, fwd, (o, ST, ws)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # After the device has idled, calls run about 15% slower for the first
    # ~20 ms of sustained work (the clock ramps up); the default warm-up covers
    # that, and the timed calls span about 60 ms.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-gauge", action="store_true")
    ap.add_argument("--bwd-steps", type=int, default=5)
    ap.add_argument("--no-ratio", action="store_true", help="skip the Complex KDA / KDA throughput ratio")
    ap.add_argument("--no-configs", action="store_true", help="time the headline forward workload only")
    args = ap.parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the gated delta-rule path here is single-GPU "
              "(independent (sequence, head) scans shard over GPUs without communication). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from gated_delta_rule_46_amd import inputs, kda

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    kda.library()

    # ---------------------------------------------------------------- forward
    print("[bench] generating inputs", file=sys.stderr, flush=True)

    def dev_set(w):
        return tuple(None if t is None else t.to(dev) for t in (w.q, w.k, w.v, w.gate, w.beta, w.cu_seqlens))

    w3 = [inputs.ckda_fwd(seed=s_) for s_ in (0, 1)]
    sets = [dev_set(x) for x in w3]
    w = w3[0]
    others = {}
    if not args.no_configs:
        w2 = [inputs.kda_fwd(seed=s_) for s_ in (0, 1)]
        w1 = [inputs.tiny_kda(seed=s_) for s_ in (0, 1)]
        w4 = inputs.gdn_varlen(seed=0)
        # the lightest first and the heaviest last, right before the headline, so
        # that the clock has ramped up when the headline's warm-up starts
        others = {"tiny_kda_fp32_b1_h1_t64_d16_chunk16": (w1[0], [dev_set(x) for x in w1]),
                  "kda_fwd_b4_h16_t4096_d128_chunk64": (w2[0], [dev_set(x) for x in w2]),
                  "gdn_varlen_h32_t110440_d128_chunk64": (w4, [dev_set(w4)])}
        del w2, w1, w4
    B, H, T, dk, dv, C = w.B, w.H, w.T, w.dk, w.dv, w.chunk
    tokens = B * T

    # the other forward workloads first, then the headline, with no idle gap
    configs = {}
    print("[bench] forward", file=sys.stderr, flush=True)
    for name, (wx, sx) in others.items():
        rec, _, bufs = forward_leg(kda, name, sx, wx, args.warmup, args.steps, stream, dev)
        configs[name] = rec
        del bufs
    head, fwd, (o, ST, ws) = forward_leg(kda, "ckda_fwd_b2_h16_t8192_d128_chunk64", sets, w, args.warmup, args.steps,
                                         stream, dev, with_clock=True)
    cpu_w = {name: wx for name, (wx, _) in others.items()}   # host copies, for the oracle baselines
    others.clear()
    ms = head["ms_per_call"]
    ms_prep = head["kernels_ms"]["chunk_prep_kernel"]
    ms_state = [v_ for k_, v_ in head["kernels_ms"].items() if k_ != "chunk_prep_kernel"][0]

    traffic_fwd, traffic_dec, traffic_bwd = measured_traffic()
    head_tokens = tokens * H
    alg_bytes = head["hbm"]["bytes_per_launch"]
    tok_s = tokens / (ms * 1e-3)
    achieved_gbs = alg_bytes / (ms * 1e-3) / 1e9
    roofline = {
        "bound": "hbm",
        "achieved": round(achieved_gbs, 2),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
        "traffic": traffic_fwd,
        "kernel": "kda_chunk_fwd: chunk_prep_kernel then chunk_state_slice_kernel (one call, one stream)",
        "bytes_per_launch": alg_bytes,
        "launch_ms": round(ms, 4),
        "mfma_frac_algorithmic": head["mfma_frac_algorithmic"],
        "kernels_ms": head["kernels_ms"],
        "per_call_ms": head["per_call_ms"],
    }
    # the same workload through the gauge route (signs folded into q and k,
    # positive-gate forward, S_T rows flipped back)
    gauge = None
    if not args.no_gauge:
        wsg = torch.empty(kda.fwd_gauge_workspace_bytes(B, H, T, dk, dv, C), device=dev, dtype=torch.uint8)

        def fwd_g(i):
            q, k, v, g, b, _ = sets[i % 2]
            kda.chunk_fwd_gauge(q, k, v, g, b, chunk=C, gate_kind=0, out=o, S_T=ST, workspace=wsg)

        for i in range(args.warmup):
            fwd_g(i)
        ms_g = time_region(fwd_g, args.steps, stream)
        ms_d = time_region(fwd, args.steps, stream)   # direct route again, same box, same moment
        gauge = {"workload": "ckda_fwd_b2_h16_t8192_d128_chunk64", "ms_per_call": round(ms_g, 4),
                 "tokens_per_s": round(tokens / (ms_g * 1e-3), 1), "direct_ms_per_call": round(ms_d, 4),
                 "throughput_vs_direct": round(ms_d / ms_g, 4)}
        print("[bench] gauge route %.3f ms/step (direct %.3f)" % (ms_g, ms_d), file=sys.stderr, flush=True)
        del wsg
    # the erase/write-gate forward (Gated DeltaNet-2 gates with the Complex KDA
    # gate recipe) on the same shape, two input sets, beside the direct route
    erase_write = None
    if not args.no_configs:
        ew_sets = []
        for s_ in (0, 1):
            xe = inputs.gdn2_ckda_fwd(seed=s_)
            ew_sets.append(tuple(t.to(dev) for t in (xe.w.q, xe.w.k, xe.w.v, xe.w.gate, xe.erase, xe.write)))
        del xe

        def fwd_e(i):
            q, k, v, g, e, wr = ew_sets[i % 2]
            kda.chunk_fwd_ew(q, k, v, g, e, wr, chunk=C, gate_kind=0, out=o, S_T=ST, workspace=ws)

        for i in range(args.warmup):
            fwd_e(i)
        ms_e = time_region(fwd_e, args.steps, stream)
        ms_d = time_region(fwd, args.steps, stream)
        erase_write = {"workload": "gdn2_ckda_fwd_b2_h16_t8192_d128_chunk64", "ms_per_call": round(ms_e, 4),
                       "tokens_per_s": round(tokens / (ms_e * 1e-3), 1), "direct_ms_per_call": round(ms_d, 4),
                       "throughput_vs_direct": round(ms_d / ms_e, 4)}
        print("[bench] erase/write forward %.4f ms/call (direct %.4f)" % (ms_e, ms_d), file=sys.stderr, flush=True)
        del ew_sets
    del sets, ws, o

    # ---------------------------------------------------------------- decode
    decode = None
    if not args.no_decode:
        print("[bench] decode inputs", file=sys.stderr, flush=True)
        dw = inputs.ckda_decode(n_steps=16)
        S = dw.S.to(dev)
        steps = [tuple(st[x].to(dev) for x in ("q", "k", "v", "gate", "beta")) for st in dw.steps]
        od = torch.empty((dw.N, dw.H, dw.dv), device=dev, dtype=torch.float32)

        def dec(i):
            q, k, v, g, b = steps[i % len(steps)]
            kda.decode_step(q, k, v, g, b, S, out=od, gate_kind=0)

        n_dec = args.decode_steps
        for i in range(n_dec):   # one untimed block: the clock ramps up again after the host-side input generation
            dec(i)
        ms_block = time_region(lambda i: [dec(j) for j in range(n_dec)], 1, stream)
        per = ms_block / n_dec
        dbytes = dw.N * dw.H * decode_bytes_per_head_step(dw.dk, dw.dv)
        gbs = dbytes / (per * 1e-3) / 1e9
        decode = {
            "workload": "ckda_decode_n256_h32_d128",
            "steps_in_block": n_dec,
            "ms_per_step": round(per, 4),
            "tokens_per_s": round(dw.N / (per * 1e-3), 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic_dec,
                         "kernel": "decode_step_kernel", "bytes_per_launch": dbytes},
        }
        del S, steps
        copy = copy_bandwidth(dev, stream)
        decode["roofline"]["copy_gbs"] = copy
        decode["roofline"]["frac_of_copy"] = round(gbs / max(copy.values()), 4)
        print("[bench] decode %.4f ms/step, %.1f GB/s (device copy: %s GB/s)" % (per, gbs, copy), file=sys.stderr,
              flush=True)

    # ---------------------------------------------------------------- backward
    backward = None
    if not args.no_backward:
        print("[bench] backward inputs", file=sys.stderr, flush=True)
        wb = inputs.ckda_fwd(seed=0)
        dO_c, dST_c = inputs.cotangents(wb, seed=0)
        bt = [t.to(dev) for t in (wb.q, wb.k, wb.v, wb.gate, wb.beta, dO_c)]
        dST = dST_c.to(dev)
        bbytes = tokens * H * bwd_bytes_per_head_token(dk, dv) + 3 * B * H * dk * dv * 4
        legs = {}
        for form, chunked in (("chunkwise", True), ("token", False)):
            wsb = (kda.bwd_cw_workspace_bytes if chunked else kda.bwd_workspace_bytes)(B, H, T, dk, dv)
            ws_b = torch.empty(wsb, device=dev, dtype=torch.uint8)
            gout = kda.chunk_bwd(*bt, dS_T=dST, workspace=ws_b, chunked=chunked)

            def bwd(i):
                kda.chunk_bwd(*bt, dS_T=dST, workspace=ws_b, out=gout, chunked=chunked)

            for i in range(5):   # the clock ramps up again after the host-side input generation
                bwd(i)
            legs[form] = (time_region(bwd, args.bwd_steps, stream), wsb)
            print("[bench] backward (%s) %.3f ms/call" % (form, legs[form][0]), file=sys.stderr, flush=True)
            del ws_b, gout
        # the erase/write form (Gated DeltaNet-2 gates with the Complex KDA gate recipe), token form
        xe = inputs.gdn2_ckda_fwd(seed=0)
        et = [t.to(dev) for t in (xe.w.q, xe.w.k, xe.w.v, xe.w.gate, xe.erase, xe.write)]
        wse = kda.bwd_ew_workspace_bytes(B, H, T, dk, dv)
        ws_e = torch.empty(wse, device=dev, dtype=torch.uint8)
        gout = kda.chunk_bwd_ew(*et, bt[5], dS_T=dST, workspace=ws_e)

        def bwd_ew(i):
            kda.chunk_bwd_ew(*et, bt[5], dS_T=dST, workspace=ws_e, out=gout)

        for i in range(5):
            bwd_ew(i)
        ms_e = time_region(bwd_ew, args.bwd_steps, stream)
        print("[bench] backward (erase/write, token form) %.3f ms/call" % ms_e, file=sys.stderr, flush=True)
        del ws_e, gout, et, xe
        ms_b, wsb_b = legs["chunkwise"]
        ms_t, wsb_t = legs["token"]
        bflops = B * H * ((T + 63) // 64) * cbwd_flops_per_head_chunk(dk, dv, 64)   # its chunk is 64
        tf = bflops / (ms_b * 1e-3) / 1e12
        gbs_b = bbytes / (ms_b * 1e-3) / 1e9
        tflops = tokens * H * bwd_flops_per_head_token(dk, dv)
        backward = {
            "workload": "ckda_bwd_b2_h16_t8192_d128",
            "ms_per_call": round(ms_b, 4),
            "tokens_per_s": round(tokens / (ms_b * 1e-3), 1),
            "calls": args.bwd_steps,
            "roofline": {"bound": "mfma", "achieved": round(tf, 3), "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / FP32_MFMA_PEAK_TFLOPS, 4), "traffic": traffic_bwd,
                         "kernel": "kda_chunk_bwd_cw: cb_prep, cb_walk (state and adjoint walks), cb_grad_state, "
                                   "cb_grad_gate (fp32 MFMA, one stream)",
                         "flops_per_launch": bflops, "hbm_bytes_algorithmic": bbytes,
                         "hbm_frac_algorithmic": round(gbs_b / HBM_PEAK_GBS, 4)},
            "workspace_bytes": wsb_b,
            "token_form": {"ms_per_call": round(ms_t, 4), "workspace_bytes": wsb_t,
                           "kernel": "kda_chunk_bwd: chunk_bwd_kernel then chunk_bwd_reduce_kernel",
                           "alu_frac": round(tflops / (ms_t * 1e-3) / 1e12 / FP32_VECTOR_PEAK_TFLOPS, 4)},
            "erase_write_token_form": {"workload": "gdn2_ckda_bwd_b2_h16_t8192_d128", "ms_per_call": round(ms_e, 4),
                                       "tokens_per_s": round(tokens / (ms_e * 1e-3), 1), "workspace_bytes": wse,
                                       "kernel": "kda_chunk_bwd_ew: chunk_bwd_kernel (erase/write) then "
                                                 "chunk_bwd_reduce_kernel"},
        }
        if not args.no_cpu_baseline:
            import oracle
            # the oracle keeps every state of a sequence (dk*dv doubles per
            # token), so the sample is the first 2048 tokens of each sequence
            Ts = 2048
            sl = lambda t: t[:, :Ts].contiguous()  # noqa: E731
            bs = [sl(x) for x in (wb.q, wb.k, wb.v, wb.gate, wb.beta, dO_c)]
            t0 = time.time()
            reps = 0
            while True:
                oracle.bwd(*bs, None, dST_c, None, 0)
                reps += 1
                if time.time() - t0 > 10.0:
                    break
            dt = (time.time() - t0) / reps
            backward["cpu_baseline"] = {
                "value": round(B * Ts / dt, 1), "unit": "tokens/s", "cores": min(oracle.threads(), B * H),
                "kind": "oracle",
                "sample": "first 2048 tokens of both sequences, all 16 heads, fp64 reverse-mode token recurrence, "
                          "%d pass(es), %.2f s each" % (reps, dt)}
            print("[bench] backward oracle %.2f s per pass" % dt, file=sys.stderr, flush=True)
        del bt

    # ------------------------------------------------- Complex KDA against KDA
    # The pages compare forward-plus-backward kernel throughput of Complex KDA
    # with KDA's at 16 heads, dk = dv = 128, bf16, 32k tokens per step (Complex
    # KDA summary, efficiency). Same shape here (B=4, T=8192), the KDA gate
    # recipe (a ~ N(3, 1)) against the Complex KDA one, measured alternately.
    ratio = None
    if not args.no_ratio:
        print("[bench] ratio inputs", file=sys.stderr, flush=True)
        Br, Tr = 4, 8192
        runs = {}
        for name, w in (("kda", inputs.make_forward("kda_b4_h16_t8192", B=Br, H=H, T=Tr, dk=dk, dv=dv, chunk=C,
                                                     gate="kda", gate_mu=3.0, seed=1)),
                        ("ckda", inputs.ckda_fwd(seed=1, B=Br, H=H, T=Tr))):
            dO_r, dST_r = inputs.cotangents(w, seed=1)
            t = [x.to(dev) for x in (w.q, w.k, w.v, w.gate, w.beta)]
            runs[name] = (t, dO_r.to(dev), dST_r.to(dev))
        ws_f = torch.empty(kda.workspace_bytes(Br, H, Tr, dk, dv, C), device=dev, dtype=torch.uint8)
        ws_r = torch.empty(kda.bwd_cw_workspace_bytes(Br, H, Tr, dk, dv), device=dev, dtype=torch.uint8)
        o_r = torch.empty((Br, Tr, H, dv), device=dev, dtype=torch.float32)
        ST_r = torch.empty((Br, H, dk, dv), device=dev, dtype=torch.float32)
        g_r = kda.chunk_bwd(*runs["kda"][0], runs["kda"][1], dS_T=runs["kda"][2], workspace=ws_r, chunked=True)
        times = {"kda": [[], []], "ckda": [[], []]}
        for rep_i in range(2):
            for name in (("kda", "ckda") if rep_i == 0 else ("ckda", "kda")):
                t, dO_r, dST_r = runs[name]

                def f_r(i):
                    kda.chunk_fwd(*t, chunk=C, gate_kind=0, out=o_r, S_T=ST_r, workspace=ws_f)

                def b_r(i):
                    kda.chunk_bwd(*t, dO_r, dS_T=dST_r, workspace=ws_r, out=g_r, chunked=True)

                for i in range(args.warmup):
                    f_r(i)
                times[name][0].append(time_region(f_r, 50, stream))
                for i in range(2):
                    b_r(i)
                times[name][1].append(time_region(b_r, 3, stream))
        fk, bk = (sum(x) / len(x) for x in times["kda"])
        fc, bc = (sum(x) / len(x) for x in times["ckda"])
        ratio = {"workload": "b4_h16_t8192_d128 bf16, 32,768 tokens per step",
                 "kda_ms": {"forward": round(fk, 4), "backward": round(bk, 4)},
                 "ckda_ms": {"forward": round(fc, 4), "backward": round(bc, 4)},
                 "forward_ratio": round(fk / fc, 4), "forward_backward_ratio": round((fk + bk) / (fc + bc), 4),
                 "pages": "96-97% forward+backward on H100, BF16, their kernels"}
        print("[bench] Complex KDA / KDA throughput: forward %.3f, forward+backward %.3f"
              % (fk / fc, (fk + bk) / (fc + bc)), file=sys.stderr, flush=True)
        del runs, ws_f, ws_r, o_r, ST_r, g_r

    # ---------------------------------------------------------------- CPU oracle
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        w0 = inputs.ckda_fwd(seed=0)
        t0 = time.time()
        reps = 0
        while True:
            oracle.fwd(w0.q, w0.k, w0.v, w0.gate, w0.beta, None, None, 0)
            reps += 1
            if time.time() - t0 > 10.0:
                break
        dt = (time.time() - t0) / reps
        cpu = {"value": round(tokens / dt, 1), "unit": "tokens/s", "cores": min(oracle.threads(), B * H),
               "kind": "oracle",
               "sample": "whole Complex KDA workload (B=2, H=16, T=8192, d=128), fp64 token recurrence, "
                         "%d pass(es), %.2f s each" % (reps, dt)}
        print("[bench] oracle %.2f s per pass" % dt, file=sys.stderr, flush=True)
        # the other forward workloads, each on a bounded sample
        samples = {
            "tiny_kda_fp32_b1_h1_t64_d16_chunk16": (None, "whole workload"),
            "kda_fwd_b4_h16_t4096_d128_chunk64": (None, "whole workload"),
            "gdn_varlen_h32_t110440_d128_chunk64": (range(4), "heads 0-3 of all 8 sequences"),
        }
        for name, (heads, what) in samples.items():
            if name not in cpu_w:
                continue
            wx = cpu_w[name]
            nh = wx.H if heads is None else len(heads)

            def run(wx=wx, heads=heads):
                if heads is None:
                    oracle.fwd(wx.q, wx.k, wx.v, wx.gate, wx.beta, None, wx.cu_seqlens, wx.gate_kind)
                else:
                    oracle.fwd_heads(wx.q, wx.k, wx.v, wx.gate, wx.beta, heads, None, wx.cu_seqlens, wx.gate_kind)

            t0 = time.time()
            reps = 0
            while reps == 0 or time.time() - t0 < 2.0:
                run()
                reps += 1
            dtx = (time.time() - t0) / reps
            # tokens/s of the whole workload at the sample's rate per head-token
            tok_x = wx.B * wx.T
            configs[name]["cpu_baseline"] = {
                "value": round(tok_x * nh / wx.H / dtx, 1), "unit": "tokens/s",
                "cores": min(oracle.threads(), wx.n_seqs * nh), "kind": "oracle",
                "sample": "%s, fp64 token recurrence, %d pass(es), %.3g s each" % (what, reps, dtx)}
            print("[bench] oracle %s %.3g s per pass" % (name, dtx), file=sys.stderr, flush=True)
    cpu_w = None

    line = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "ckda_fwd_b2_h16_t8192_d128_chunk64", "B": B, "H": H, "T": T, "dk": dk, "dv": dv,
                   "chunk": C, "tokens_per_step": tokens, "parallelism": "single-gpu"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "status": head["status"],
        "sclk_during_timed_calls": head.get("sclk_during_timed_calls"),
        "configs": configs,
        "decode": decode,
        "backward": backward,
        "gauge_route": gauge,
        "erase_write_forward": erase_write,
        "ckda_vs_kda": ratio,
        "gpu_clock_after_run": gpu_clock(),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
