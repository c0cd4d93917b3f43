"""Build libparo.so (HIP kernels + C-ABI) for gfx950 with hipcc, in-tree.

    python -m rotation_int4_weight_amd.build        # or build() from Python
    python -m rotation_int4_weight_amd.build --decode-timeline   # diagnostic tools
    python -m rotation_int4_weight_amd.build --prefill-timeline

Each source compiles to an object under _build/ (in parallel), then one link
produces rotation_int4_weight_amd/libparo.so.  Always rebuilds.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build", "paro")
LIB = os.path.join(PKG, "libparo.so")
ARCH = "gfx950"

SOURCES = ["paro_abi.cpp", "scale_rotate.hip", "unpack_dequant.hip", "decode.hip", "prefill.hip", "quantize.hip", "rotate_backward.hip", "mxfp4.hip", "noalloc.hip"]

# Packed-FP32 instructions are switched off for all device code: hipcc would
# otherwise form v_pk_{add,mul,fma}_f32 from scalar float code.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libparo)")


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    # the host pass warns that it does not know the packed-fp32 feature
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in (r.stderr or "").splitlines() if noise not in ln and ln.strip()]
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build(extra=(), verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra)), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    # A kernel template whose host pass fails quietly leaves its launch stub
    # undefined: the library would then not load.  Refuse such a link.
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [ln.split()[-1] for ln in nm.stdout.splitlines() if "__device_stub__" in ln]
    if missing:
        os.remove(tmp)
        raise RuntimeError(f"link left {len(missing)} kernel launch stubs undefined, e.g. {missing[0]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def _build_tool(name: str, define: str, verbose: bool) -> str:
    os.makedirs(BUILD, exist_ok=True)
    out = os.path.join(BUILD, name)
    cmd = [hipcc(), *[f for f in COMMON if f != "-fPIC"], f"-D{define}", os.path.join(CSRC, name + ".hip"),
           "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {name}.hip:\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {out}")
    return out


def build_decode_timeline(verbose: bool = False) -> str:
    """The per-wave decode timeline tool (csrc/decode_timeline.hip): decode.hip
    compiled with PARO_DECODE_TIMELINE into a standalone program under _build/."""
    return _build_tool("decode_timeline", "PARO_DECODE_TIMELINE", verbose)


def build_prefill_timeline(verbose: bool = False) -> str:
    """The per-wave prefill GEMM timeline tool (csrc/prefill_timeline.hip)."""
    return _build_tool("prefill_timeline", "PARO_PREFILL_TIMELINE", verbose)


if __name__ == "__main__":
    if "--decode-timeline" in sys.argv[1:]:
        build_decode_timeline(verbose=True)
    elif "--prefill-timeline" in sys.argv[1:]:
        build_prefill_timeline(verbose=True)
    else:
        build(verbose=True)
