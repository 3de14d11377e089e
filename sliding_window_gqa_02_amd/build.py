"""Builds libswgqa.so (HIP, gfx950) in-tree with hipcc.

Every source is compiled for gfx950 only, with packed-FP32 instruction
selection turned off, and linked into one shared library next to this file.
"""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libswgqa.so")
SOURCES = ["swgqa_api.hip", "swgqa_attn_split.hip", "swgqa_attn_decode.hip",
           "swgqa_attn_decode_rot.hip", "swgqa_attn_decode_q8.hip", "swgqa_attn_decode_f8.hip",
           "swgqa_attn_chunk.hip", "swgqa_attn_chunk_q8.hip", "swgqa_attn_chunk_f8.hip", "swgqa_step_tail.hip", "swgqa_copy.hip",
           "swgqa_rotary.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compiles every source to an object and links libswgqa.so."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src: str) -> str:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        return obj

    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
