"""Build libgdn.so for gfx950 with hipcc (in-tree, next to this file)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgdn.so")
# Microbenchmarks of the machine's limits (HBM streaming, MFMA issue rate): a
# library of their own, loaded only by the benchmark.
PEAKS_LIB = os.path.join(HERE, "libgdn_peaks.so")
PEAKS_SOURCES = ["peaks.hip"]
SOURCES = ["gdn_api.hip", "gdn_decode.hip", "gdn_prefill_f32.hip", "gdn_segment.hip", "gdn_profile.hip",
           "gdn_backward.hip", "gdn_conv.hip", "gdn_noalloc.hip"]
ARCH = "gfx950"

# Packed fp32 instructions are disabled for every HIP file (the compiler would
# otherwise pair ordinary float arithmetic into them).
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               # MFMA results in ordinary VGPRs (no accumulator-register copies on gfx950)
               "-mllvm", "-amdgpu-mfma-vgpr-form"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(verbose: bool = False) -> str:
    """Compile every kernel source into libgdn.so (and the microbenchmarks into
    libgdn_peaks.so); returns the path of libgdn.so."""
    _compile(SOURCES, LIB, verbose)
    _compile(PEAKS_SOURCES, PEAKS_LIB, verbose)
    return LIB


def _compile(sources, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIPCC_FLAGS + [os.path.join(CSRC, s) for s in sources] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, lib)


if __name__ == "__main__":
    print(build(verbose=True))
