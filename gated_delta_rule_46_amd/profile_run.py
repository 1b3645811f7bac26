"""A short, fixed workload to run under rocprofv3.

    python -m gated_delta_rule_46_amd.profile_run [--fwd 3] [--bwd 2] [--bwd-token 0] [--decode 8]
                                                  [--copy-mib 256]

Runs, on cuda:0 and with seeded synthetic inputs: --fwd forward calls on the
workload --fwd-workload names (ckda: Complex KDA, B=2, H=16, T=8192, d=128,
bf16, chunk 64, the default; kda: KDA, B=4, H=16, T=4096; gdn: GDN with eight
packed sequences, H=32, T=110,440), --bwd
chunkwise backward calls (kda_chunk_bwd_cw) and --bwd-token token-form
backward calls (kda_chunk_bwd) on the same workload, --decode decode steps on the decode
workload (N=256, H=32, d=128, fp32 state in place), and --copy-mib MiB of
plain device-to-device copy (one read and one write of that many bytes per
call, three calls), whose counter readings calibrate FETCH_SIZE and
WRITE_SIZE against a known byte count.
"""
from __future__ import annotations

import argparse
import os
import sys


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--fwd", type=int, default=3)
    ap.add_argument("--fwd-workload", choices=("ckda", "kda", "gdn"), default="ckda")
    ap.add_argument("--bwd", type=int, default=2)
    ap.add_argument("--bwd-token", type=int, default=0)
    ap.add_argument("--decode", type=int, default=8)
    ap.add_argument("--copy-mib", type=int, default=256)
    args = ap.parse_args(argv)

    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import torch
    from gated_delta_rule_46_amd import inputs, kda

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    kda.library()
    if args.fwd > 0:
        w = {"ckda": inputs.ckda_fwd, "kda": inputs.kda_fwd, "gdn": inputs.gdn_varlen}[args.fwd_workload](seed=0)
        q, k, v, g, b = (t.to(dev) for t in (w.q, w.k, w.v, w.gate, w.beta))
        cu = None if w.cu_seqlens is None else w.cu_seqlens.to(dev)
        N = w.n_seqs
        ws = torch.empty(kda.workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, w.chunk, N, cu is not None, w.dtype),
                         device=dev, dtype=torch.uint8)
        o = torch.empty((w.B, w.T, w.H, w.dv), device=dev, dtype=torch.float32)
        ST = torch.empty((N, w.H, w.dk, w.dv), device=dev, dtype=torch.float32)
        for _ in range(args.fwd):
            kda.chunk_fwd(q, k, v, g, b, cu_seqlens=cu, chunk=w.chunk, gate_kind=w.gate_kind, out=o, S_T=ST,
                          workspace=ws)
        torch.cuda.synchronize()
        print("forward calls: %d (%s)" % (args.fwd, args.fwd_workload), flush=True)
        del q, k, v, g, b, cu, ws, o, ST
    for calls, chunked in ((args.bwd, True), (args.bwd_token, False)):
        if calls <= 0:
            continue
        w = inputs.ckda_fwd(seed=0)
        dO, dST = inputs.cotangents(w, seed=0)
        t = [x.to(dev) for x in (w.q, w.k, w.v, w.gate, w.beta, dO)]
        dST = dST.to(dev)
        need = (kda.bwd_cw_workspace_bytes if chunked else kda.bwd_workspace_bytes)(w.B, w.H, w.T, w.dk, w.dv)
        ws = torch.empty(need, device=dev, dtype=torch.uint8)
        g = kda.chunk_bwd(*t, dS_T=dST, workspace=ws, chunked=chunked)
        for _ in range(calls - 1):
            kda.chunk_bwd(*t, dS_T=dST, workspace=ws, out=g, chunked=chunked)
        torch.cuda.synchronize()
        print("%s backward calls: %d" % ("chunkwise" if chunked else "token-form", calls), flush=True)
        del t, dST, ws, g
    if args.decode > 0:
        dw = inputs.ckda_decode(n_steps=min(args.decode, 16))
        S = dw.S.to(dev)
        steps = [tuple(st[x].to(dev) for x in ("q", "k", "v", "gate", "beta")) for st in dw.steps]
        od = torch.empty((dw.N, dw.H, dw.dv), device=dev, dtype=torch.float32)
        for i in range(args.decode):
            qd, kd, vd, gd, bd = steps[i % len(steps)]
            kda.decode_step(qd, kd, vd, gd, bd, S, out=od, gate_kind=0)
        torch.cuda.synchronize()
        print("decode steps: %d" % args.decode, flush=True)
        del S, steps, od
    if args.copy_mib > 0:
        src = torch.ones(args.copy_mib << 20, device=dev, dtype=torch.uint8)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print("copy: 3 x %d MiB" % args.copy_mib, flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
