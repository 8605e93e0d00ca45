"""Build libattn_sink.so in-tree with hipcc for gfx950.

Usage: python -m softmax_learnable_sink_amd.build   (or build() from Python)
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn_sink.so")
LIB_DEBUG = os.path.join(PKG, "libattn_sink_debug.so")  # with device-side checks
SOURCES = ["api.hip", "prefill.hip", "decode.hip", "backward.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-result",
    # packed fp32 vector ops are disabled for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build libattn_sink.so")
    return path


def _compile(out, extra_flags, verbose):
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True), tmp


def build(verbose=False, extra_flags=()):
    """Compile every HIP source into softmax_learnable_sink_amd/libattn_sink.so and,
    with device-side precondition checks, libattn_sink_debug.so (in parallel)."""
    jobs = [(LIB, _compile(LIB, list(extra_flags), verbose)),
            (LIB_DEBUG, _compile(LIB_DEBUG, list(extra_flags) + ["-DATTN_SINK_DEVICE_CHECKS=1"],
                                 verbose))]
    for out, (proc, tmp) in jobs:
        text = proc.communicate()[0]
        text = "\n".join(line for line in text.splitlines()
                         if "is not a recognized feature for this target" not in line)
        if proc.returncode != 0:
            raise RuntimeError(f"hipcc failed ({proc.returncode}) for {out}:\n{text}")
        if verbose and text.strip():
            print(text)
        os.replace(tmp, out)
    return LIB


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer (device code is built
# as usual): every sanitizer flag applies to the host compilation only.
SANITIZE_HOST_FLAGS = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-g",
]


def build_sanitized(out):
    """Build the library with host-side ASan/UBSan into `out` (for the CPU tests of
    the argument validation; load it with the ASan runtime preloaded)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    flags = [f for f in HIPCC_FLAGS if f != "-O3"] + ["-O1"] + SANITIZE_HOST_FLAGS
    cmd = [hipcc(), *flags, "-I", INCLUDE, "-I", CSRC, *srcs, "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}{res.stderr}")
    return out


def device_asm(source, out):
    """Compile one HIP source's gfx950 device code to assembly text at `out`
    (the release build's flags), for checks of the generated code."""
    flags = [f for f in HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [hipcc(), *flags, "--cuda-device-only", "-S", "-I", INCLUDE, "-I", CSRC,
           os.path.join(CSRC, source), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}{res.stderr}")
    return out


def asan_runtime():
    """Path of the ASan runtime library of hipcc's clang."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    return res.stdout.strip()


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
