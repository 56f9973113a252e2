"""Build libattn.so (the HIP kernels and the C ABI) for gfx950 with hipcc, and
libattn_peaks.so (the benchmark's measured-ceiling kernels)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libattn.so")
PEAKS_LIB = os.path.join(PKG, "libattn_peaks.so")

SOURCES = ["api.cpp", "fwd_bf16.hip", "fwd_f32.hip", "decode.hip", "bwd_bf16.hip", "bwd_f32.hip",
           "noalloc.hip", "rope.hip"]
PEAKS_SOURCES = ["peaks.hip"]

# Packed fp32 VALU forms are disabled: every fp32 operation is a plain
# single-lane instruction.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-variable",
]


def _hipcc(sources, out, verbose):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = out + ".tmp"
    cmd = [hipcc, *FLAGS, "-I", os.path.join(ROOT, "include"), *srcs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so;
    # that line is expected and dropped.
    noise = "not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    _hipcc(PEAKS_SOURCES, PEAKS_LIB, verbose)
    return _hipcc(SOURCES, LIB, verbose)


# Host sanitizers for the C ABI's host code (argument checks, workspace
# carving): AddressSanitizer and UndefinedBehaviorSanitizer on the host pass
# only -- the device code is built as usual.  The resulting library is for the
# CPU-side ABI tests (transformer_attention_causal_amd/sanitize.sh); it needs
# the ASan runtime loaded first.
SAN_LIB = os.path.join(PKG, "libattn_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
             "-shared-libasan"]


def build_sanitized(verbose: bool = False) -> str:
    global FLAGS
    saved = FLAGS
    FLAGS = FLAGS + SAN_FLAGS
    try:
        return _hipcc(SOURCES, SAN_LIB, verbose)
    finally:
        FLAGS = saved


if __name__ == "__main__":
    import sys as _sys
    if "--sanitized" in _sys.argv:
        print(build_sanitized(verbose=True))
    else:
        print(build(verbose=True))
