"""Host-side sanitizer run of the CPU test suites (no GPU is used):

  1. the oracle's C core (oracle/wmtp_oracle.c) built by gcc with AddressSanitizer and
     UndefinedBehaviorSanitizer, under the oracle's pin and planted-mistake tests;
  2. libwmtp.so built with the same sanitizers on its host code only (hipcc, each flag behind
     -Xarch_host; the gfx950 code is compiled as usual and never runs here), under the C ABI's
     host tests, which drive every argument check of every entry point.

    python tests/sanitize_host.py

Each suite runs in a child process with the compiler's sanitizer runtime preloaded (the Python
interpreter itself is not instrumented), leak detection off (the interpreter keeps its own
allocations to the end) and every report fatal. The sanitized libraries go to a temporary
directory, removed at the end; the in-tree builds are not touched. Exit status 0 when both suites
pass.
"""
import glob
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer", "-g"]
ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
       "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _gcc_asan_runtime() -> str:
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()
    if not os.path.isabs(path):
        raise RuntimeError("gcc has no AddressSanitizer runtime")
    return path


def _clang_asan_runtime() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    found = sorted(glob.glob(os.path.join(rocm, "llvm", "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    if not found:
        raise RuntimeError("ROCm's clang has no AddressSanitizer runtime")
    return found[-1]


def _pytest(files, extra_env) -> int:
    env = dict(os.environ, **ENV, **extra_env)
    cmd = [sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider"] + files
    print("+", " ".join(f"{k}={v}" for k, v in extra_env.items()), " ".join(cmd), flush=True)
    return subprocess.run(cmd, cwd=ROOT, env=env).returncode


def main() -> int:
    import oracle
    from draft_attention_amd import build as lib_build

    tmp = tempfile.mkdtemp(prefix="wmtp_san_")
    try:
        return _run(tmp, oracle, lib_build)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def _run(tmp, oracle, lib_build) -> int:
    oracle_lib = oracle.build(verbose=True, out=os.path.join(tmp, "liboracle_san.so"),
                              flags=["-O1"] + SAN)
    rc = _pytest(["tests/test_oracle_pins.py", "tests/test_oracle_mutations.py"],
                 {"LD_PRELOAD": _gcc_asan_runtime(), "WMTP_ORACLE_LIB": oracle_lib})
    if rc != 0:
        print(f"oracle suite under sanitizers: exit status {rc}", file=sys.stderr)
        return rc
    wmtp_lib = lib_build.build(verbose=True, out=os.path.join(tmp, "libwmtp_san.so"),
                               host_flags=SAN)
    rc = _pytest(["tests/test_abi_host.py"],
                 {"LD_PRELOAD": _clang_asan_runtime(), "WMTP_LIB": wmtp_lib})
    if rc != 0:
        print(f"C ABI host suite under sanitizers: exit status {rc}", file=sys.stderr)
        return rc
    print("sanitizer run: both suites passed", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
