"""Builds librva.so (gfx950 only) in-tree with hipcc."""
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = ["csrc/pack.hip", "csrc/attend.hip", "csrc/threshold.hip", "csrc/linear.hip", "csrc/probe.hip",
           "csrc/rva_host.hip"]
LIB = os.path.join(PKG, "librva.so")


def hipcc_command(out=LIB):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    return [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            # no packed fp32 arithmetic anywhere in device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # inputs are finite by contract: lets fmax lower to plain v_max/v_max3
            "-fno-honor-nans",
            "-Wall", "-Wno-unused-command-line-argument",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")] + \
        [os.path.join(PKG, s) for s in SOURCES] + ["-o", out]


FLOOR_BENCH = os.path.join(PKG, "floor_bench")


def floor_bench_command(out=FLOOR_BENCH):
    """The C++ dispatch-floor probe (csrc/floor_bench.cpp),
    linked against librva.so in this directory."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    return [hipcc, "--offload-arch=gfx950", "-O2", "-std=c++17",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), os.path.join(PKG, "csrc", "floor_bench.cpp"),
            "-L", PKG, "-lrva", "-Wl,-rpath,$ORIGIN", "-o", out]


def _run(cmd, out):
    tmp = out + ".tmp"
    cmd = cmd[:-1] + [tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    return r


def build(verbose: bool = False) -> str:
    """Compile every HIP source into librva.so next to this file (and the
    dispatch-floor probe linked against it); returns the library's path."""
    r = _run(hipcc_command(LIB), LIB)
    if verbose:
        print(r.stderr)
    _run(floor_bench_command(), FLOOR_BENCH)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
