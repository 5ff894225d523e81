"""Build linear_rnn_recurrent_amd/libssu.so (HIP for gfx950) in-tree.

    python -m linear_rnn_recurrent_amd.build        # or: python linear_rnn_recurrent_amd/build.py

Every HIP source is compiled with packed-FP32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops). The library links the HIP
runtime only.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libssu.so")
OBJDIR = os.path.join(HERE, "_build")

SOURCES = ["ssu_api.cpp", "ssu_decode.hip", "ssu_decode_f32.hip", "ssu_decode_f16.hip",
           "ssu_decode_bf16.hip", "ssu_prefill.hip", "ssu_prefill_f32.hip", "ssu_prefill_f16.hip",
           "ssu_prefill_bf16.hip", "ssu_replay.hip", "ssu_tree.hip", "ssu_tree_f32.hip",
           "ssu_tree_f16.hip", "ssu_tree_bf16.hip", "ssu_gdn.hip", "ssu_pool_kernels.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = ["-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
          "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src, extra, verbose):
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + CFLAGS + list(extra) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature: that warning is expected
    noise = [ln for ln in (r.stderr or "").splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln and "is not a recognized feature" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(noise))
    if noise and verbose:
        print("\n".join(noise))
    return obj


def build(verbose=False, extra=(), jobs=None):
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
