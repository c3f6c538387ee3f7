"""Build libmtla.so (the MTLA C-ABI library) in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmtla.so")
SOURCES = ["gemm.hip", "gemm_big.hip", "gemm_stream.hip", "decode.hip", "attention.hip", "append.hip", "heads.hip", "heads_f32.hip", "backward.hip", "backward_f32.hip", "rope.hip", "mtla_api.hip"]
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
# -amdgpu-mfma-vgpr-form: MFMA accumulators in ordinary VGPRs (gfx950 reads C
# and writes D there), instead of copying every accumulator through AGPRs
# around each product; the attention kernels keep their O accumulators live
# across VALU rescaling, which the copies otherwise make expensive.
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form=1",
         "-I", INCLUDE, "-I", CSRC]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


# Sources whose accumulators should live in AGPRs (a wave holding 256
# accumulator registers at one wave per SIMD): built without the VGPR form.
AGPR_SOURCES = {"gemm_big.hip"}


def _flags(src: str):
    if src not in AGPR_SOURCES:
        return FLAGS
    out, i = [], 0
    while i < len(FLAGS):
        if FLAGS[i] == "-mllvm" and FLAGS[i + 1].startswith("-amdgpu-mfma-vgpr-form"):
            i += 2
            continue
        out.append(FLAGS[i])
        i += 1
    return out


def _compile(src: str, obj: str, verbose: bool):
    cmd = [_hipcc(), *_flags(src), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libmtla.so next to this file."""
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, s.replace(".hip", ".o")) for s in SOURCES]
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        list(ex.map(lambda a: _compile(a[0], a[1], verbose), zip(SOURCES, objs)))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
