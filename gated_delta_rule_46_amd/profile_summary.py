"""Summaries of rocprofv3 runs of profile_run.py / bench.py for profiles/.

    python -m gated_delta_rule_46_amd.profile_summary stats DIR OUT.md --title T --command C [--note N]
    python -m gated_delta_rule_46_amd.profile_summary traffic FETCH_DIR WRITE_DIR NAME --command C [--command C2]
    python -m gated_delta_rule_46_amd.profile_summary mfma PMC_DIR STATS_DIR OUT.md --command C

``stats`` turns the kernel-stats CSV of a ``rocprofv3 --kernel-trace --stats
--output-format csv`` run into a markdown table (calls, average, minimum and
maximum duration per kernel).

``traffic`` reads the counter CSVs of two ``rocprofv3 --pmc FETCH_SIZE`` and
``--pmc WRITE_SIZE`` runs of profile_run.py (KiB per dispatch), calibrates
each counter on the plain device copy profile_run.py makes (``--copy-mib`` MiB
read and written per call: scale = bytes moved / counter reading), and writes
profiles/NAME.md (per-kernel table) and profiles/NAME.txt (a JSON record:
per kernel group the scaled bytes per call and the SHA-256 of its kernel
sources, by which bench.py decides whether the figure still applies).

``mfma`` reads one counter run (SQ_VALU_MFMA_BUSY_CYCLES,
SQ_INSTS_VALU_MFMA_MOPS_F16, SQ_INSTS_VALU_MFMA_F16, SQ_INSTS_VALU_MFMA_F32,
SQ_BUSY_CU_CYCLES, SQ_INSTS_VALU, SQ_WAVE_CYCLES, SQ_ACTIVE_INST_VALU,
GRBM_GUI_ACTIVE) and the kernel durations of a stats run, and tabulates per
kernel the MFMA work (fp16 MOPS x 512 flops, fp32 16x16x4 instructions x
2048 flops), its rate, MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE
/ 8 XCDs x 1024 SIMDs) and VALU issue per wave.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Kernel groups of one call. A group's bytes per call are the sum over its
# kernels of the average per dispatch (each kernel runs once per call).
GROUPS = {
    "forward": {"match": ("chunk_prep_kernel", "chunk_state"), "per": "call",
                "sources": ["gated_delta_rule_46_amd/csrc/kda_chunk.hip", "gated_delta_rule_46_amd/csrc/kda_common.h",
                            "gated_delta_rule_46_amd/csrc/kda_chunkmap.h"]},
    "decode": {"match": ("decode_step_kernel",), "per": "step",
               "sources": ["gated_delta_rule_46_amd/csrc/kda_decode.hip", "gated_delta_rule_46_amd/csrc/kda_common.h"]},
    "backward": {"match": ("cb_prep_kernel", "cb_walk_kernel", "cb_grad_state_kernel", "cb_grad_gate_kernel",
                           "chunk_index_kernel"), "per": "call",
                 "sources": ["gated_delta_rule_46_amd/csrc/kda_cbwd.hip", "gated_delta_rule_46_amd/csrc/kda_common.h",
                             "gated_delta_rule_46_amd/csrc/kda_chunkmap.h"]},
    "backward_token": {"match": ("chunk_bwd_kernel", "chunk_bwd_reduce_kernel"), "per": "call",
                       "sources": ["gated_delta_rule_46_amd/csrc/kda_bwd.hip",
                                   "gated_delta_rule_46_amd/csrc/kda_common.h"]},
}
COPY_NAMES = ("copyBuffer", "elementwise_kernel", "copy")


def _short(name: str) -> str:
    n = name.replace("(anonymous namespace)::", "").split("(")[0]
    if n.startswith("void "):
        n = n[5:]
    return n if len(n) < 90 else n[:87] + "..."


def _rows(path_glob: str):
    files = sorted(glob.glob(path_glob, recursive=True))
    if not files:
        raise SystemExit("no file matches %s" % path_glob)
    with open(files[0], newline="") as f:
        return list(csv.DictReader(f))


def cmd_stats(a) -> int:
    rows = _rows(os.path.join(a.dir, "**", "*kernel_stats.csv"))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = ["# " + a.title, "", "Command (MI355X, gfx950, one GPU; `$REPO` is the repository root):", "", "```"]
    out += list(a.command) + ["```", ""]
    if a.note:
        out += [a.note, ""]
    out += ["| kernel | calls | average ns | min ns | max ns | total ms |", "|---|---|---|---|---|---|"]
    for r in rows:
        out.append("| %s | %s | %.0f | %.0f | %.0f | %.3f |" % (
            _short(r["Name"]), r["Calls"], float(r["AverageNs"]), float(r["MinNs"]), float(r["MaxNs"]),
            float(r["TotalDurationNs"]) / 1e6))
    with open(a.out, "w") as f:
        f.write("\n".join(out) + "\n")
    print("wrote", a.out)
    return 0


def _per_kernel(d: str, counter: str):
    """Average counter value (KiB) per dispatch and dispatch count, by kernel
    name; and the largest single-dispatch value, by kernel name."""
    acc, top = {}, {}
    for r in _rows(os.path.join(d, "**", "*counter_collection.csv")):
        if r.get("Counter_Name") != counter:
            continue
        name, x = r["Kernel_Name"], float(r["Counter_Value"])
        s, n = acc.get(name, (0.0, 0))
        acc[name] = (s + x, n + 1)
        top[name] = max(top.get(name, 0.0), x)
    return {k: (s / n, n) for k, (s, n) in acc.items()}, top


def cmd_traffic(a) -> int:
    fetch, ftop = _per_kernel(a.fetch_dir, "FETCH_SIZE")
    write, wtop = _per_kernel(a.write_dir, "WRITE_SIZE")
    copy = [k for k in fetch if any(c in k for c in COPY_NAMES) and k in write]
    if not copy:
        raise SystemExit("no copy kernel to calibrate on")
    # the calibration copy is the largest single copy dispatch of the run (the
    # input uploads go through the same copy kernel with smaller sizes)
    ck = max(copy, key=lambda k: ftop[k])
    nbytes = a.copy_mib << 20
    fscale = nbytes / (ftop[ck] * 1024.0)
    wscale = nbytes / (wtop[ck] * 1024.0)
    rec = {"fetch_scale": fscale, "write_scale": wscale, "calibration": {"kernel": _short(ck), "bytes": nbytes},
           "groups": {}}
    table = []
    for g, spec in GROUPS.items():
        ks = [k for k in fetch if any(m in k for m in spec["match"])]
        if not ks:
            continue
        rd = sum(fetch[k][0] * 1024.0 * fscale for k in ks)
        wr = sum(write.get(k, (0.0, 0))[0] * 1024.0 * wscale for k in ks)
        sha = {}
        for rel in spec["sources"]:
            with open(os.path.join(ROOT, rel), "rb") as f:
                sha[rel] = hashlib.sha256(f.read()).hexdigest()
        rec["groups"][g] = {"bytes_per_" + spec["per"]: int(round(rd + wr)), "read_bytes": int(round(rd)),
                            "write_bytes": int(round(wr)), "sources_sha256": sha}
        for k in sorted(ks):
            table.append((g, _short(k), fetch[k][1], fetch[k][0] * 1024.0 * fscale / 1e6,
                          write.get(k, (0.0, 0))[0] * 1024.0 * wscale / 1e6))
    rec["workload"] = {"forward": "ckda_fwd_b2_h16_t8192_d128_chunk64", "decode": "ckda_decode_n256_h32_d128",
                       "backward": "ckda_bwd_b2_h16_t8192_d128 (kda_chunk_bwd_cw)",
                       "backward_token": "ckda_bwd_b2_h16_t8192_d128 (kda_chunk_bwd)"}
    base = os.path.join(ROOT, "profiles", a.name)
    with open(base + ".txt", "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    out = ["# HBM traffic per dispatch: " + a.title, "",
           "Commands (MI355X, gfx950, one GPU; FETCH_SIZE and WRITE_SIZE each in a run of its own; `$REPO` is the "
           "repository root):", "", "```"] + list(a.command) + ["```", "",
           "Calibration on %s (%d MiB read and written per call): FETCH x %.4f, WRITE x %.4f."
           % (_short(ck), a.copy_mib, fscale, wscale), "",
           "| group | kernel | dispatches | read MB per dispatch (scaled) | written MB per dispatch (scaled) |",
           "|---|---|---|---|---|"]
    for g, k, n, rd, wr in table:
        out.append("| %s | %s | %d | %.1f | %.1f |" % (g, k, n, rd, wr))
    out.append("")
    for g, spec in GROUPS.items():
        if g in rec["groups"]:
            r = rec["groups"][g]
            out.append("- %s: %.1f MB per %s (read %.1f, written %.1f)" % (
                g, r["bytes_per_" + spec["per"]] / 1e6, spec["per"], r["read_bytes"] / 1e6, r["write_bytes"] / 1e6))
    with open(base + ".md", "w") as f:
        f.write("\n".join(out) + "\n")
    print("wrote", base + ".txt", base + ".md")
    return 0


def cmd_mfma(a) -> int:
    acc = {}
    grid = {}
    for r in _rows(os.path.join(a.pmc_dir, "**", "*counter_collection.csv")):
        name = r["Kernel_Name"]
        d = acc.setdefault(name, {})
        s, n = d.get(r["Counter_Name"], (0.0, 0))
        d[r["Counter_Name"]] = (s + float(r["Counter_Value"]), n + 1)
        grid[name] = int(float(r.get("Grid_Size", 0) or 0))
    dur = {r["Name"]: float(r["AverageNs"]) for r in _rows(os.path.join(a.stats_dir, "**", "*kernel_stats.csv"))}
    out = ["# MFMA and VALU counters per dispatch: " + a.title, "", "Commands (`$REPO` is the repository root):", "",
           "```"] + list(a.command) + ["```", "",
           "Per dispatch (mean over the dispatches of the run). MFMA flops = SQ_INSTS_VALU_MFMA_MOPS_F16 x 512 + "
           "SQ_INSTS_VALU_MFMA_F32 x 2048 (every fp32 MFMA here is 16x16x4). Rate = flops / the kernel's mean duration "
           "in the stats run; peaks 2.5 PFLOP/s dense fp16/bf16, 157.3 TFLOP/s fp32 MFMA. MFMA busy = "
           "SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs). VALU busy = SQ_ACTIVE_INST_VALU / "
           "SQ_WAVE_CYCLES.", "",
           "| kernel | fp16 MFMA instr. | fp32 MFMA instr. | MFMA GFLOP | mean us | MFMA TFLOP/s | MFMA busy | "
           "VALU instr. per wave | VALU busy |", "|---|---|---|---|---|---|---|---|---|"]
    def v(d, k):
        s, n = d.get(k, (0.0, 0))
        return s / n if n else 0.0
    for name in sorted(acc, key=lambda k: -dur.get(k, 0.0)):
        d = acc[name]
        if any(c in name for c in COPY_NAMES):
            continue
        gf = (v(d, "SQ_INSTS_VALU_MFMA_MOPS_F16") * 512 + v(d, "SQ_INSTS_VALU_MFMA_F32") * 2048) / 1e9
        us = dur.get(name, 0.0) / 1e3
        act = v(d, "GRBM_GUI_ACTIVE") / 8 * 1024
        waves = max(grid.get(name, 0) // 64, 1)
        wc = v(d, "SQ_WAVE_CYCLES")
        out.append("| %s | %.0f | %.0f | %.2f | %.1f | %.1f | %.3f | %.0f | %.2f |" % (
            _short(name), v(d, "SQ_INSTS_VALU_MFMA_F16"), v(d, "SQ_INSTS_VALU_MFMA_F32"), gf, us,
            gf / (us * 1e-6) / 1e3 if us else 0.0, v(d, "SQ_VALU_MFMA_BUSY_CYCLES") / act if act else 0.0,
            v(d, "SQ_INSTS_VALU") / waves, v(d, "SQ_ACTIVE_INST_VALU") / wc if wc else 0.0))
    with open(a.out, "w") as f:
        f.write("\n".join(out) + "\n")
    print("wrote", a.out)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="mode", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("out")
    s.add_argument("--title", required=True)
    s.add_argument("--command", action="append", required=True)
    s.add_argument("--note", default="")
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("name")
    t.add_argument("--title", default="Complex KDA forward, backward (B=2, H=16, T=8192, d=128) and decode "
                                      "(N=256, H=32, d=128)")
    t.add_argument("--command", action="append", required=True)
    t.add_argument("--copy-mib", type=int, default=256)
    m = sub.add_parser("mfma")
    m.add_argument("pmc_dir")
    m.add_argument("stats_dir")
    m.add_argument("out")
    m.add_argument("--title", default="Complex KDA forward and backward (B=2, H=16, T=8192, d=128), decode")
    m.add_argument("--command", action="append", required=True)
    a = ap.parse_args(argv)
    return {"stats": cmd_stats, "traffic": cmd_traffic, "mfma": cmd_mfma}[a.mode](a)


if __name__ == "__main__":
    sys.exit(main())
