"""Build the HIP library in-tree with hipcc for gfx950.

``python -m paged_kv_decode_07_amd.build`` compiles ``csrc/pa_decode.hip``
(BF16 pages; device kernels in ``csrc/pa_kernels.h``), ``csrc/pa_decode_q8.hip``
(INT8 pages; ``csrc/pa_kernels_q8.h``), ``csrc/pa_decode_balanced.hip`` (the balanced
launch over a host plan, every page format), ``csrc/pa_balance_plan.cpp`` (its host
planner), ``csrc/pa_measure.hip`` (streaming-read calibration) and
``csrc/pa_kvpool.cpp`` (host page allocator), against the
headers in ``include/``, into
``paged_kv_decode_07_amd/_lib/libpa_decode.so``.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", n)
        for n in ("pa_decode.hip", "pa_decode_q8.hip", "pa_decode_balanced.hip", "pa_measure.hip",
                  "pa_kvpool.cpp", "pa_balance_plan.cpp")]
OUT_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(OUT_DIR, "libpa_decode.so")
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden",
    # packed FP32 instructions stay off: plain FP32 VALU only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS,
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
           *SRCS, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("packed-fp32-ops", "--hip-link")
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines()
            if ln.strip() and not any(n in ln for n in noise)]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    missing = undefined_kernel_stubs(tmp)
    if missing:
        os.remove(tmp)
        raise RuntimeError("kernel launch stubs left undefined (a kernel template was not "
                           "instantiated on the host side):\n" + "\n".join(missing))
    os.replace(tmp, LIB)
    return LIB


CLIENT_SRC = os.path.join(ROOT, "tests", "c_client", "decode_client.cpp")
CLIENT = os.path.join(OUT_DIR, "decode_client")


def build_client(verbose: bool = False) -> str:
    """Build the C-ABI client used by the tests (a host program linked to the library)."""
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O2", "-std=c++17",
           "-I", os.path.join(ROOT, "include"), CLIENT_SRC, "-o", CLIENT + ".tmp",
           "-L", OUT_DIR, "-lpa_decode", "-Wl,-rpath,$ORIGIN"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed on the C client:\n" + res.stderr)
    os.replace(CLIENT + ".tmp", CLIENT)
    return CLIENT


def undefined_kernel_stubs(lib_path: str) -> list:
    """Host launch stubs referenced by the library but not defined in it."""
    nm = next((c for c in ("/opt/rocm/llvm/bin/llvm-nm", shutil.which("nm")) if c and os.path.exists(c)),
              None)
    if nm is None:
        return []
    out = subprocess.run([nm, "--undefined-only", lib_path], capture_output=True, text=True).stdout
    return [ln.split()[-1] for ln in out.splitlines() if "__device_stub__" in ln]


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_client(verbose="-v" in sys.argv))
