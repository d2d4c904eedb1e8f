"""Compile wmtp_c_caller.c (a plain C caller of libwmtp.so) with gcc next to its source.

    python tests/c_caller/build.py

It links libwmtp.so from draft_attention_amd/ (found at run time through an $ORIGIN-relative
rpath) and the HIP runtime from ROCm.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "wmtp_c_caller.c")
EXE = os.path.join(HERE, "wmtp_c_caller")


def build() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"), SRC,
           "-o", EXE + ".tmp", "-L", os.path.join(ROOT, "draft_attention_amd"), "-lwmtp",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../draft_attention_amd", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    subprocess.run(cmd, check=True)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build(), file=sys.stderr)
