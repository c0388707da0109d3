"""Build the HIP library (gfx950) into gemm_decode_qgemm_amd/libqgemm.so.

Every translation unit is compiled with hipcc for gfx950 in parallel, then
linked into one shared library exporting the C ABI of include/qgemm.h.

Flags that matter for results:
  -ffp-contract=off                 no silent FMA contraction (the quantizers
                                    must match the CPU reference bit for bit)
  -fhip-fp32-correctly-rounded-divide-sqrt   IEEE binary32 division
  -fno-gpu-flush-denormals-to-zero  keep fp32 denormals
  -Xclang -target-feature -Xclang -packed-fp32-ops   no packed fp32 VALU ops
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqgemm.so")
OBJDIR = os.path.join(PKG, "_build")

SOURCES = ["api.hip", "quantize.hip", "gemv_w4a16.hip", "gemv_w8a16.hip", "gemv_w4a8.hip",
           "gemm_w4a16_mfma.hip", "gemv_w4a16_mx4.hip", "stream_read.hip",
           "gemm_w8a16_mfma.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-source flags.  The matrix-core kernel asks the backend to write MFMA
# results to ordinary VGPRs (the AGPR form costs a v_accvgpr_read per result
# element before the fp32 epilogue of every group).
SOURCE_FLAGS = {"gemm_w4a16_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "gemv_w4a16_mx4.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "gemv_w4a8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "gemm_w8a16_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, extra: list[str], objdir: str) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(out: str = LIB, extra: list[str] | None = None, objdir: str = OBJDIR,
          verbose: bool = False, link: list[str] | None = None) -> str:
    """Compile all sources (always; no staleness check) and link `out`.

    `extra` is added to every compile line; `link`, if given, replaces the
    default link driver (hipcc) with that command prefix (the objects, -shared
    and -o are appended)."""
    extra = list(extra or [])
    os.makedirs(objdir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, objdir), SOURCES))
    tmp = out + ".tmp"
    head = list(link) if link else [HIPCC, "--offload-arch=gfx950"]
    cmd = [*head, "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}", flush=True)
    return out


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
