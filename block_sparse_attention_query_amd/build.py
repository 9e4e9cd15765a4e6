"""Build libsparse_attn.so for gfx950 in-tree (hipcc, one object per source, then link)."""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libsparse_attn.so")
SOURCES = ["api.cpp", "pool.hip", "select.hip", "attn_fwd.hip", "attn_bwd.hip", "patterns.hip", "probe.hip", "cluster.hip"]
# Per-source extra flags. The attention kernels assume finite-or-infinite inputs (NaN inputs give
# unspecified outputs), which lets fmaxf on MFMA results skip the NaN-quieting canonicalize.
# Matrix-core sources also take the VGPR form of every MFMA (results and accumulators in
# architectural VGPRs): by default the compiler places MFMA results in AGPRs, and kernels whose
# products feed vector arithmetic (the softmax of S, dS from dP) then spend one v_accvgpr_read per
# element, plus accumulator moves whenever the AGPR tuples fragment (160 of the 490 vector
# instructions of a dK/dV step on D = 128).
MFMA_VGPR = ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]
EXTRA = {"attn_fwd.hip": ["-fno-honor-nans", *MFMA_VGPR], "attn_bwd.hip": ["-fno-honor-nans", *MFMA_VGPR],
         "probe.hip": ["-fno-honor-nans", *MFMA_VGPR], "cluster.hip": ["-fno-honor-nans", *MFMA_VGPR]}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 VALU ops are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function"]


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, "-x", "hip", *COMMON, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


# Host-side sanitizer build of the C ABI's argument checks: api.cpp's host code compiled with
# AddressSanitizer and UndefinedBehaviorSanitizer (its device pass is unchanged), linked with the
# regular objects of the other sources. Run on the CPU only, with the sanitizer runtime preloaded
# (the CPU test suite does this for the host ABI tests).
CLANGXX = "/opt/rocm/lib/llvm/bin/clang++"
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    import glob
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise FileNotFoundError("clang AddressSanitizer runtime not found")
    return hits[-1]


def build_host_sanitized(out_dir: str) -> str:
    os.makedirs(out_dir, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, [s for s in SOURCES if s != "api.cpp"]))
    api_obj = os.path.join(out_dir, "api_san.o")
    cmd = [HIPCC, "-x", "hip", *COMMON, *DEVICE_FLAGS, *SANITIZE_HOST, "-g", "-c", os.path.join(CSRC, "api.cpp"),
           "-o", api_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stderr}")
    out = os.path.join(out_dir, "libsparse_attn_hostsan.so")
    cmd = [CLANGXX, "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libsan", api_obj, *objs,
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    return out


if __name__ == "__main__":
    build()
