"""Build libmamba3.so in-tree with hipcc for gfx950.

    python -m mamba_selective_scan_amd.build          # compile (always)
    python -m mamba_selective_scan_amd.build --check  # compile + load + list exports
    python -m mamba_selective_scan_amd.build --debug  # the -DM3_DEBUG build: libmamba3_debug.so

Every translation unit is compiled in parallel to an object file under
``_build/`` and linked into ``mamba_selective_scan_amd/libmamba3.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmamba3.so")
DEBUG_LIB = os.path.join(HERE, "libmamba3_debug.so")
ARCH = os.environ.get("M3_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

# Packed fp32 instructions are disabled for all device code (the compiler would
# otherwise form v_pk_{add,mul,fma}_f32 from ordinary float code).
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-result", "-munsafe-fp-atomics"]

SOURCES = ["m3_scan_bf16_vec.hip", "m3_scan_bf16_gen.hip", "m3_scan_bf16_mimo.hip", "m3_scan_f32_vec.hip",
           "m3_scan_f32_gen.hip", "m3_scan.hip", "m3_state.hip", "m3_bwd.hip", "m3_perm.hip", "m3_api.cpp"]


def _compile(src: str, debug: bool = False) -> str:
    out = os.path.join(BUILD, "debug") if debug else BUILD
    obj = os.path.join(out, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *(["-DM3_DEBUG"] if debug else []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True, debug: bool = False) -> str:
    """Compile and link the library; ``debug`` builds libmamba3_debug.so with the device-side
    checks of -DM3_DEBUG (read back with m3_debug_checks)."""
    os.makedirs(os.path.join(BUILD, "debug") if debug else BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda f: _compile(f, debug), SOURCES))
    lib = DEBUG_LIB if debug else LIB
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(debug="--debug" in sys.argv)
    if "--check" in sys.argv:
        import ctypes
        lib = ctypes.CDLL(DEBUG_LIB if "--debug" in sys.argv else LIB)
        for name in ("m3_scan_siso", "m3_scan_mimo", "m3_step", "m3_scan_workspace_bytes",
                     "m3_status_str", "m3_version"):
            getattr(lib, name)
        print("exports ok")
