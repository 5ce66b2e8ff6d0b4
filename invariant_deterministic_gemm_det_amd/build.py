"""Build step for the det_gemm HIP library (gfx950).

Compiles the sources in ``csrc/`` with hipcc (one object per translation unit,
in parallel) and links ``libdet_gemm.so`` inside this package directory.

Device-code flags:
  * ``-Xclang -target-feature -Xclang -packed-fp32-ops``: no packed-fp32 VALU
    instructions (hipcc's host pass warns that it does not know the feature,
    which is harmless);
  * ``-Xclang -target-feature -Xclang -dot13-insts``: without the two-address
    v_dot2c_f32_bf16 the compiler emits the three-address v_dot2_f32_bf16 for
    the tree's bf16 adds, saving one move per add;
  * ``-mllvm -simplifycfg-sink-common=false``: keeps the optimizer from merging
    stores of different branches into one store through a pointer phi, which
    would force the kernels' register-resident tree nodes into scratch memory.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdet_gemm.so")
OBJDIR = os.path.join(HERE, "_build")

SOURCES = ["det_gemm.hip", "mfma_fwd_bf16.hip", "mfma_fwd_f32.hip", "mfma_kk_bf16.hip", "mfma_moe.hip", "fingerprint.hip", "rmsnorm.hip", "attention.hip",
           "mfma_nn_bf16.hip", "mfma_nn_bf16t.hip", "mfma_leaves.hip", "mfma_decode.hip"]
HEADERS = ["bf16_device.h", "device_check.h", "strict_kernel.h", "mfma_kernel.h", "mfma_fast.h", "mfma_wide.h",
           "mfma_launch.h"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Xclang", "-target-feature", "-Xclang", "-dot13-insts",
         "-mllvm", "-simplifycfg-sink-common=false",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _inputs():
    return [os.path.join(CSRC, f) for f in SOURCES + HEADERS] + \
        [os.path.join(ROOT, "include", h) for h in ("det_gemm.h", "det_moe.h", "det_fingerprint.h", "det_norm.h",
                                                       "det_attention.h")]


def _compile(src, extra):
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}{res.stderr}")
    return obj


def build(force: bool = True, extra=(), jobs: int = 0) -> str:
    """Compile and link the library; returns its path."""
    if not force and os.path.exists(LIB):
        mtime = os.path.getmtime(LIB)
        if all(os.path.getmtime(f) <= mtime for f in _inputs()):
            return LIB
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 16)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as pool:
        objs = list(pool.map(lambda s: _compile(s, list(extra)), SOURCES))
    tmp = LIB + ".tmp"
    res = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    args = [a for a in sys.argv[1:] if a != "--if-stale"]
    print(build(force="--if-stale" not in sys.argv, extra=args))
