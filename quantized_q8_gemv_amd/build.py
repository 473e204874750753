"""Build libq8l.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m quantized_q8_gemv_amd.build   (or call build()).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libq8l.so")
SOURCES = ["k_gemv.hip", "k_wgemv.hip", "k_xgemv.hip", "k_gemm.hip", "k_attn.hip", "k_misc.hip", "k_kquant.hip", "noalloc.hip", "runtime.cpp", "gguf.cpp"]
ARCH = os.environ.get("Q8L_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from forming packed FP32 instructions.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function",
          "-Wno-unused-variable"]


# MFMA kernels keep their results in VGPRs (no AGPR round trip before the
# per-block scale is applied in f32).
PER_FILE = {"k_gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
            "k_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, obj: str) -> None:
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + COMMON + PER_FILE.get(src, []) + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    subprocess.run(cmd, check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)


LLVM = os.environ.get("ROCM_LLVM", "/opt/rocm/llvm/bin")


def scratch_kernels(obj: str) -> list:
    """Kernels of a compiled .hip object (its gfx950 code object's metadata)
    that use scratch memory: a private segment or spilled VGPRs. A kernel of
    this library that does is a performance bug (its stack traffic goes to
    HBM), e.g. an argument struct grown past what stays in registers.
    Returns [] when the LLVM tools are not there."""
    objcopy, bundler, readelf = (os.path.join(LLVM, t) for t in
                                 ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf"))
    if not all(os.path.exists(t) for t in (objcopy, bundler, readelf)):
        return []
    fat, co = obj + ".fatbin", obj + ".co"
    subprocess.run([objcopy, f"--dump-section=.hip_fatbin={fat}", obj], check=True,
                   stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    subprocess.run([bundler, "--unbundle", "--type=o", f"--targets=hipv4-amdgcn-amd-amdhsa--{ARCH}",
                    f"--input={fat}", f"--output={co}"], check=True, stdout=subprocess.PIPE,
                   stderr=subprocess.STDOUT)
    notes = subprocess.run([readelf, "--notes", co], check=True, stdout=subprocess.PIPE,
                           stderr=subprocess.STDOUT).stdout.decode(errors="replace")
    bad, name = [], None
    for line in notes.splitlines():
        line = line.strip()
        if line.startswith(".name:"):
            name = line.split(":", 1)[1].strip()
        elif line.startswith((".private_segment_fixed_size:", ".vgpr_spill_count:")):
            if int(line.split(":", 1)[1]) > 0 and name and name not in bad:
                bad.append(name)
    return bad


def build(verbose: bool = False) -> str:
    """Compile every source and link libq8l.so; returns its path."""
    with tempfile.TemporaryDirectory(prefix="q8l_build_") as tmp:
        objs = [os.path.join(tmp, s + ".o") for s in SOURCES]
        with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
            futs = [ex.submit(_compile, s, o) for s, o in zip(SOURCES, objs)]
            for s, f in zip(SOURCES, futs):
                try:
                    f.result()
                except subprocess.CalledProcessError as e:
                    sys.stderr.write(e.stdout.decode(errors="replace"))
                    raise RuntimeError(f"hipcc failed on {s}") from None
        bad = [k for s, o in zip(SOURCES, objs) if s.endswith(".hip") for k in scratch_kernels(o)]
        if bad:
            raise RuntimeError("kernels using scratch memory (private segment or VGPR spills): " + ", ".join(bad))
        tmp_lib = LIB + ".tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib] + objs
        subprocess.run(cmd, check=True)
        os.replace(tmp_lib, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
