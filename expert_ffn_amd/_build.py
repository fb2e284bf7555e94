"""Build of libexpert_ffn.so (hipcc for gfx950, in-tree)."""
from __future__ import annotations

import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_obj")
LIB = os.path.join(HERE, "libexpert_ffn.so")
# measurement kernels of the benchmark (achieved peaks): a library of their own
PEAKS_SRC = os.path.join(HERE, "measure", "peaks.hip")
PEAKS_LIB = os.path.join(HERE, "libpeaks.so")
ARCH = os.environ.get("EXPERT_FFN_ARCH", "gfx950")

HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else "hipcc"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 VALU instructions (v_pk_fma_f32 and the like): the compiler
    # would otherwise form them from ordinary float code; this library keeps them out
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: no v_accvgpr moves around each MFMA
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    deps = glob.glob(os.path.join(CSRC, "*.h")) + [os.path.join(HERE, "..", "include", "expert_ffn.h")]

    def compile_one(src):
        obj = os.path.join(OBJ, os.path.basename(src) + ".o")
        cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    del deps
    build_peaks()
    return LIB


def build_peaks() -> str:
    tmp = PEAKS_LIB + ".tmp%d" % os.getpid()
    r = subprocess.run([HIPCC, *FLAGS, "-shared", PEAKS_SRC, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {PEAKS_SRC}:\n{r.stderr}")
    os.replace(tmp, PEAKS_LIB)
    return PEAKS_LIB


if __name__ == "__main__":
    print(build(verbose=True))
