"""Build libattnfwd.so in-tree with hipcc for gfx950 (cross-compiles on a host without a GPU)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libattnfwd.so")
SOURCES = ["api.cpp", "prefill.hip", "prefill_fp8.hip", "decode.hip", "backward.hip", "probe.hip"]
HEADERS = ["attn_device.hpp", "fp8_device.hpp", "kernels.hpp", "plan.hpp"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the attention library)")


def compile_command(out: str) -> list[str]:
    return [
        hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
        # packed fp32 VALU forms stay off: the kernels get plain v_fma/v_mul/v_add
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", out,
    ]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = compile_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "unknown target feature"  # the host pass does not know the device-only feature flag
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l and "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    check_loadable(tmp)
    os.replace(tmp, LIB)
    return LIB


def check_loadable(path: str) -> None:
    """Refuse a library with unresolved symbols (e.g. a kernel whose host launch stub was not
    emitted): load it with every symbol bound now, as its first use on a GPU host would."""
    import ctypes
    try:
        ctypes.CDLL(path, mode=os.RTLD_NOW | os.RTLD_LOCAL)
    except OSError as e:
        os.unlink(path)
        raise RuntimeError(f"built library does not load: {e}") from None


if __name__ == "__main__":
    print(build(verbose=True))
