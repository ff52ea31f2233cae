"""Build libmsa.so (HIP, gfx950) in-tree: ``python -m block_sparse_gqa_amd.build``."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmsa.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["msa_api.hip", "index_topk.hip", "plan.hip", "attn_kv.hip", "attn_q.hip",
           "combine.hip", "select_tiles.hip", "backward.hip", "probe.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed-fp32 VALU ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"),
]


# Per-source extra flags. The index kernel's MFMA results feed VALU max-reductions directly,
# and the backward kernels' feed the softmax terms and the partial stores: the VGPR form of
# MFMA spares the accumulator-register moves the default form would need (proxy backward
# 6.61 -> 6.15 ms at the M3 shape).
EXTRA_FLAGS = {
    "index_topk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "backward.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libmsa.so next to this file."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max(1, min(len(SOURCES), os.cpu_count() or 1))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


ASAN_DIR = os.path.join(BUILD_DIR, "asan")


def asan_runtime() -> str | None:
    """The AddressSanitizer runtime of the compiler hipcc drives (to preload into a host)."""
    import glob
    hits = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(
        hipcc()))), "llvm", "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    hits += sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[0] if hits else None


def build_asan() -> str:
    """A copy of the library whose host code (argument checks, workspace plan, launchers) is
    built with AddressSanitizer; the device code is built as usual (no GPU sanitizer). For
    host-only tests: load it with the runtime from asan_runtime() preloaded."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    flags = [f for f in HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g", "-Xarch_host",
                                                       "-fsanitize=address", "-shared-libasan"]

    def one(src):
        obj = os.path.join(ASAN_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc(), *flags, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc (asan) failed on {src}:\n{r.stderr}")
        return obj
    with ThreadPoolExecutor(max(1, min(len(SOURCES), os.cpu_count() or 1))) as ex:
        objs = list(ex.map(one, SOURCES))
    out = os.path.join(ASAN_DIR, "libmsa_asan.so")
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-shared-libasan", *objs, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link (asan) failed:\n{r.stderr}")
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
