"""Compile librma.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m kv_cache_reads_amd.build_lib
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "librma.so")
OBJDIR = os.path.join(HERE, "_build")
SOURCES = ["rma_api.hip", "rma_build.hip", "rma_topk.hip", "rma_merge.hip", "rma_decode.hip",
           "rma_full.hip", "rma_phi_mlp.hip", "rma_stream.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# packed fp32 ops stay disabled: ordinary float code is compiled to unpacked VALU ops.
# The first kernel arguments are preloaded into SGPRs at wave launch (gfx950's
# kernarg preload; the code keeps a fallback that loads them when the launch
# does not), so a kernel's first loads need not wait for the argument segment.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-kernarg-preload-count=16",
         "-I", os.path.join(os.path.dirname(HERE), "include")]


def _compile(src):
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return obj, err


def build(verbose=True):
    os.makedirs(OBJDIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(_compile, SOURCES))
    for (_, err), src in zip(results, SOURCES):
        if verbose and err.strip():
            print(f"[{src}]\n{err}", file=sys.stderr)
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


def clean():
    shutil.rmtree(OBJDIR, ignore_errors=True)


if __name__ == "__main__":
    build()
