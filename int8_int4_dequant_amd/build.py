"""Build libqw.so (the HIP kernels and the C ABI) in-tree for gfx950.

Every source is compiled by hipcc for gfx950 only, without fast-math and
without denormal flushing (bit-exact quantization needs IEEE fp32 division,
round-half-even and preserved fp32 subnormals), and with packed-fp32
instructions disabled.
"""

import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqw.so")
SOURCES = ["qw_api.hip", "quantize.hip", "gemv.hip", "gemm.hip", "gptq.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


# Flags of one source only.  gptq.hip: its fp64 MFMA GEMM keeps the
# accumulators in VGPRs (the VGPR form of v_mfma_f64_16x16x4f64); left to
# its heuristics the compiler put the 64-wide tiles' accumulators in AGPRs
# and copied them to and from VGPRs around every reduction stage, so every
# stage waited for the matrix pipeline to drain.
SOURCE_FLAGS = {
    "gptq.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def compile_objects(out_dir, extra=(), verbose=False):
    """Compiles every source into out_dir with FLAGS plus `extra`; returns
    the object paths."""
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    jobs = []
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        for src in SOURCES:
            obj = os.path.join(out_dir, src.replace(".hip", ".o"))
            objs.append(obj)
            cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), *extra, "-c",
                   os.path.join(CSRC, src), "-o", obj]
            jobs.append(ex.submit(_run, cmd))
        for j in jobs:
            msg = j.result()
            if verbose and msg:
                print(msg)
    return objs


def build(verbose=False, save_temps=False):
    objs = compile_objects(BUILD, ["--save-temps"] if save_temps else [], verbose)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
