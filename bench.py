#!/usr/bin/env python3
"""Throughput of the chunkwise gated delta-rule forward and the decode step
on one MI355X, with roofline fractions and the fp64 CPU oracle as baseline.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

A step is one kda_chunk_fwd call over the Complex KDA workload (B=2, H=16,
T=8192, dk=dv=128, bf16 inputs, fp32 state, chunk 64): 16,384 tokens. Two
seeded input sets alternate so the 256 MB last-level cache cannot hold the
whole working set. The decode step (N=256 sequences, H=32, d=128, fp32 state
of 512 MiB updated in place) is timed as one block of 128 consecutive steps.
The backward (kda_chunk_bwd, gradients of every input for given dO and
dS_T) is timed on the same forward workload. Forward and backward are also
timed at 32k tokens per step (B=4, H=16, T=8192) with the KDA and the Complex
KDA gate recipes, for the throughput ratio of the two.
Timing uses HIP events recorded on the stream the kernels run on. Prints one
JSON line.
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


def decode_bytes_per_head_step(dk: int, dv: int, in_bytes: int = 2) -> int:
    return 8 * dk * dv + in_bytes * (3 * dk + dv + 1) + 4 * dv


def _traffic_record(name: str) -> dict:
    """A committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or {} when the
    kernel sources it names have changed since the counters were taken."""
    import hashlib
    try:
        with open(os.path.join(ROOT, "profiles", name)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return {}
    for rel, digest in rec.get("sources_sha256", {}).items():
        try:
            with open(os.path.join(ROOT, rel), "rb") as f:
                if hashlib.sha256(f.read()).hexdigest() != digest:
                    return {}
        except OSError:
            return {}
    return rec


def measured_traffic():
    """Measured HBM bytes per forward call, per decode step and per backward
    call (None where the profiled sources no longer match)."""
    fd = _traffic_record("hbm_traffic_ckda_fwd_decode.txt")
    bw = _traffic_record("hbm_traffic_ckda_bwd.txt")
    return fd.get("forward_bytes_per_call"), fd.get("decode_bytes_per_step"), bw.get("backward_bytes_per_call")


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
    sets = []
    for seed in (0, 1):
        w = inputs.ckda_fwd(seed=seed)
        sets.append(tuple(t.to(dev) for t in (w.q, w.k, w.v, w.gate, w.beta)))
    B, H, T, dk, dv, C = w.B, w.H, w.T, w.dk, w.dv, w.chunk
    tokens = B * T
    o = torch.empty((B, T, H, dv), device=dev, dtype=torch.float32)
    ST = torch.empty((B, H, dk, dv), device=dev, dtype=torch.float32)
    wsb = kda.workspace_bytes(B, H, T, dk, dv, C)
    ws = torch.empty(wsb, device=dev, dtype=torch.uint8)

    def fwd(i, stage=kda.STAGE_ALL):
        q, k, v, g, b = sets[i % 2]
        kda.chunk_fwd(q, k, v, g, b, chunk=C, gate_kind=0, out=o, S_T=ST, workspace=ws, stage=stage)

    print("[bench] warmup", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        fwd(i)
    torch.cuda.synchronize()
    ms = time_region(fwd, args.steps, stream)
    print("[bench] forward %.3f ms/step" % ms, file=sys.stderr, flush=True)
    ms_med, ms_min = per_call_ms(fwd, args.steps, stream)
    ms_prep = time_region(lambda i: fwd(i, kda.STAGE_PREP), min(args.steps, 50), stream)
    fwd(0, kda.STAGE_PREP)
    ms_state = time_region(lambda i: fwd(0, kda.STAGE_STATE), min(args.steps, 50), stream)
    print("[bench] prep %.3f ms, state %.3f ms" % (ms_prep, ms_state), file=sys.stderr, flush=True)

    traffic_fwd, traffic_dec, traffic_bwd = measured_traffic()
    head_tokens = tokens * H
    alg_bytes = head_tokens * fwd_bytes_per_head_token(dk, dv, False) + B * H * dk * dv * 4
    alg_flops = head_tokens * fwd_flops_per_head_token(dk, dv)
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
        "mfma_frac_algorithmic": round(alg_flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "kernels_ms": {"chunk_prep_kernel": round(ms_prep, 4), "chunk_state_slice_kernel": round(ms_state, 4)},
        "per_call_ms": {"median": round(ms_med, 4), "min": round(ms_min, 4)},
    }
    # the same workload through the gauge route (signs folded into q and k,
    # positive-gate forward, S_T rows flipped back)
    gauge = None
    if not args.no_gauge:
        wsg = torch.empty(kda.fwd_gauge_workspace_bytes(B, H, T, dk, dv, C), device=dev, dtype=torch.uint8)

        def fwd_g(i):
            q, k, v, g, b = sets[i % 2]
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
        print("[bench] decode %.4f ms/step, %.1f GB/s" % (per, gbs), file=sys.stderr, flush=True)
        del S, steps

    # ---------------------------------------------------------------- backward
    backward = None
    if not args.no_backward:
        print("[bench] backward inputs", file=sys.stderr, flush=True)
        wb = inputs.ckda_fwd(seed=0)
        dO_c, dST_c = inputs.cotangents(wb, seed=0)
        bt = [t.to(dev) for t in (wb.q, wb.k, wb.v, wb.gate, wb.beta, dO_c)]
        dST = dST_c.to(dev)
        wsb_b = kda.bwd_workspace_bytes(B, H, T, dk, dv)
        ws_b = torch.empty(wsb_b, device=dev, dtype=torch.uint8)
        gout = kda.chunk_bwd(*bt, dS_T=dST, workspace=ws_b)

        def bwd(i):
            kda.chunk_bwd(*bt, dS_T=dST, workspace=ws_b, out=gout)

        for i in range(5):   # about 35 ms: the clock ramps up again after the host-side input generation
            bwd(i)
        ms_b = time_region(bwd, args.bwd_steps, stream)
        bflops = tokens * H * bwd_flops_per_head_token(dk, dv)
        bbytes = tokens * H * bwd_bytes_per_head_token(dk, dv) + 3 * B * H * dk * dv * 4
        tf = bflops / (ms_b * 1e-3) / 1e12
        gbs_b = bbytes / (ms_b * 1e-3) / 1e9
        backward = {
            "workload": "ckda_bwd_b2_h16_t8192_d128",
            "ms_per_call": round(ms_b, 4),
            "tokens_per_s": round(tokens / (ms_b * 1e-3), 1),
            "calls": args.bwd_steps,
            "roofline": {"bound": "alu", "achieved": round(tf, 3), "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / FP32_VECTOR_PEAK_TFLOPS, 4), "traffic": traffic_bwd,
                         "kernel": "kda_chunk_bwd: chunk_bwd_kernel then chunk_bwd_reduce_kernel",
                         "flops_per_launch": bflops, "hbm_bytes_algorithmic": bbytes,
                         "hbm_frac_algorithmic": round(gbs_b / HBM_PEAK_GBS, 4)},
            "workspace_bytes": wsb_b,
        }
        print("[bench] backward %.3f ms/call" % ms_b, file=sys.stderr, flush=True)
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
        del bt, ws_b, gout

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
        ws_r = torch.empty(kda.bwd_workspace_bytes(Br, H, Tr, dk, dv), device=dev, dtype=torch.uint8)
        o_r = torch.empty((Br, Tr, H, dv), device=dev, dtype=torch.float32)
        ST_r = torch.empty((Br, H, dk, dv), device=dev, dtype=torch.float32)
        g_r = kda.chunk_bwd(*runs["kda"][0], runs["kda"][1], dS_T=runs["kda"][2], workspace=ws_r)
        times = {"kda": [[], []], "ckda": [[], []]}
        for rep_i in range(2):
            for name in (("kda", "ckda") if rep_i == 0 else ("ckda", "kda")):
                t, dO_r, dST_r = runs[name]

                def f_r(i):
                    kda.chunk_fwd(*t, chunk=C, gate_kind=0, out=o_r, S_T=ST_r, workspace=ws_f)

                def b_r(i):
                    kda.chunk_bwd(*t, dO_r, dS_T=dST_r, workspace=ws_r, out=g_r)

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
        "decode": decode,
        "backward": backward,
        "gauge_route": gauge,
        "ckda_vs_kda": ratio,
        "gpu_clock": gpu_clock(),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
