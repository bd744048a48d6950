"""Build the gfx950 shared library ``lib/libqlinear.so`` from ``csrc/`` with hipcc.

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction selection disabled,
then linked into one shared library whose exported symbols are the C ABI of include/qlinear.h.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libqlinear.so")
SOURCES = ["qlinear_api.cpp", "quantize.hip", "dequant.hip", "gemv.hip", "gemv_m1.hip", "gemv_m2.hip", "gemv_m4.hip",
           "gemv_m8.hip", "gemm.hip", "experts.hip", "experts_mx.hip",
           "experts_q8.hip", "experts_kq.hip", "gemv_stream.hip", "take.hip", "transcode.hip"]
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]
# Matrix-core kernels whose VALU reads the accumulators in the loop (to apply group scales) keep
# them in the architectural VGPRs (accumulation registers would need a move per element); the
# GEMM's accumulators are only read in its epilogue and may live in the accumulation registers.
FILE_FLAGS = {
    f: ["-mllvm", "-amdgpu-mfma-vgpr-form"]
    for f in ("gemv_m1.hip", "gemv_m2.hip", "gemv_m4.hip", "gemv_m8.hip")
}


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(verbose: bool = False, jobs: int = 8, extra_flags=(), out: str = LIB) -> str:
    """Compile every source and link `out` (default lib/libqlinear.so); `extra_flags` are added
    to each compile line (for example -D overrides of the launch tunables)."""
    hipcc = _hipcc()
    os.makedirs(os.path.dirname(out), exist_ok=True)
    with tempfile.TemporaryDirectory(prefix="qlinear_build_") as tmp:
        def compile_one(src: str) -> str:
            obj = os.path.join(tmp, src + ".o")
            lang = ["-x", "hip"] if src.endswith(".cpp") else []
            cmd = [hipcc, *FLAGS, *FILE_FLAGS.get(src, []), *extra_flags, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
            if verbose:
                errs = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln]
                if errs:
                    print("\n".join(errs))
            return obj

        with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        out_tmp = out + ".tmp"
        cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out_tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stderr}")
        os.replace(out_tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
