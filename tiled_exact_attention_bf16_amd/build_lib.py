"""Builds libfa_gfx950.so (the C-ABI library) in place with hipcc for gfx950, and its
check build libfa_gfx950_serial.so (every buffer->LDS load batch waited for as soon as
it is issued; the tests compare its results with the library's bit for bit).

    python -m tiled_exact_attention_bf16_amd.build_lib
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa_gfx950.so")
SERIAL_LIB = os.path.join(PKG, "libfa_gfx950_serial.so")
SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip"]
KERNEL_SOURCES = ["fa_fwd.hip", "fa_bwd.hip"]  # rebuilt with FA_SERIAL_LOADS for the check build
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
# Device code is compiled without packed-fp32 instructions.
DEVICE = ["-x", "hip", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def _compile(src: str, verbose: bool, serial: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ("_serial.o" if serial else ".o"))
    cmd = [HIPCC, *COMMON, *DEVICE, *(["-DFA_SERIAL_LOADS"] if serial else []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    noise = [l for l in r.stderr.splitlines()
             if l.strip() and "packed-fp32-ops" not in l and "ignoring feature" not in l]
    if noise and verbose:
        print("\n".join(noise), file=sys.stderr)
    return obj


def _link(objs, out: str, verbose: bool) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every source, link the library and its check build; returns the
    library's path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(s, False) for s in SOURCES] + [(s, True) for s in KERNEL_SOURCES]
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], verbose, j[1]), jobs))
    normal = objs[:len(SOURCES)]
    api = normal[SOURCES.index("fa_api.cpp")]
    _link(normal, LIB, verbose)
    _link([api, *objs[len(SOURCES):]], SERIAL_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
