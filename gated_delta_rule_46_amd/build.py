"""Build libkda.so in-tree with hipcc for gfx950, and its LDS-poisoning
debug variant libkda_lds_poison.so (every kernel fills its LDS with NaN
before use; the same sources built with -DKDA_LDS_POISON).

    python -m gated_delta_rule_46_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libkda.so")
POISON_LIB = os.path.join(HERE, "libkda_lds_poison.so")
OBJDIR = os.path.join(HERE, "_build")
SOURCES = ["kda_api.cpp", "kda_decode.hip", "kda_chunk.hip", "kda_bwd.hip", "kda_gauge.hip", "kda_noalloc.hip", "kda_cbwd.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    # packed fp32 VALU forms stay off (the compiler must not emit v_pk_* f32 ops)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results straight into VGPRs (no accumulator-register copies in the state walk)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    "-I" + os.path.join(ROOT, "include"),
]


# Per-source additions. The chunk kernels and the backward are bound by
# dependent chains and schedule better for latency (3-6% faster on every
# forward configuration, 7% on the backward); the streaming decode kernel
# loses 17% with that schedule, so it keeps the default.
ILP = ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]
EXTRA = {"kda_chunk.hip": ILP, "kda_bwd.hip": ILP}


def _compile(src: str, objdir: str = OBJDIR, extra=()) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, r.stdout, r.stderr))
    return obj


def build(verbose: bool = False, poison: bool = False) -> str:
    """Compile every HIP source and link libkda.so next to this file (with
    poison=True: libkda_lds_poison.so, the LDS-poisoning debug build)."""
    objdir = OBJDIR + ("_lds_poison" if poison else "")
    extra = ("-DKDA_LDS_POISON",) if poison else ()
    out = POISON_LIB if poison else LIB
    os.makedirs(objdir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda src: _compile(src, objdir, extra), SOURCES))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    build(verbose=True, poison=True)
    sys.exit(0)
