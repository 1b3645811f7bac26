"""Compile tests/c/abi_check.c (the C ABI used from plain C, checked against
the C oracle) into tests/c/abi_check, linked against the in-tree libkda.so
and oracle/libkda_oracle.so by relative run paths. Test infrastructure; the
package build step calls build() after building both libraries.

    python tests/c/build.py
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_check.c")
EXE = os.path.join(HERE, "abi_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROCM, "include"), SRC, "-o", EXE + ".tmp",
           "-L" + os.path.join(ROOT, "gated_delta_rule_46_amd"), "-lkda", "-L" + os.path.join(ROOT, "oracle"),
           "-lkda_oracle", "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../gated_delta_rule_46_amd", "-Wl,-rpath,$ORIGIN/../../oracle",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    subprocess.check_call(cmd)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print("built", build())
