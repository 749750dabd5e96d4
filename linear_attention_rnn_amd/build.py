"""Build libwkv7.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m linear_attention_rnn_amd.build

Compiles every source under csrc/ to an object in _build/ (in parallel) and
links linear_attention_rnn_amd/libwkv7.so; links the hardware-ceiling probes
under probe/ into libwkv7_probe.so, a library of their own that only
measurement code loads. Always rebuilds.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libwkv7.so")
PROBE_SRC = os.path.join(PKG, "probe")
PROBE_LIB = os.path.join(PKG, "libwkv7_probe.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc",
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libwkv7)")


COMMON = [
    "-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
    # code objects the HIP runtime bundled with torch loads as well
    "-mcode-object-version=5",
    # no packed fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


# Per-source options. The chunked prefill kernel is scheduled by LLVM's
# max-ILP machine scheduler instead of the default occupancy-driven one: its
# launch holds one 12-wavefront workgroup per CU whatever the register count,
# so the default scheduler's register savings buy nothing, while the
# interleaving of independent work shortens each pipeline step (the same
# instructions, so the same results bit for bit; measured 3-5% faster on the
# bf16 prefills and the mixed stack, no spills, at most 163 VGPRs of the 168
# that three wavefronts per SIMD allow).
PER_SOURCE = {
    "k2_chunk_p.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    extra = PER_SOURCE.get(os.path.basename(src), [])
    cmd = [hipcc(), *COMMON, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n"
                           f"{res.stderr}")
    return obj


def _sources(d: str) -> list:
    return sorted(os.path.join(d, f) for f in os.listdir(d)
                  if f.endswith((".hip", ".cpp")))


def _link(objs: list, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}",
           "-mcode-object-version=5", *objs,
           "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n"
                           f"{res.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = _sources(CSRC)
    probe_srcs = _sources(PROBE_SRC)
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(_compile, srcs + probe_srcs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], PROBE_LIB)
    if verbose:
        print(f"built {LIB}")
        print(f"built {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
