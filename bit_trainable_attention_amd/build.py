"""Build the gfx950 HIP library libsagebwd.so in-tree with hipcc.

Each .hip source under csrc/ is compiled to an object in _build/ (in
parallel), then linked into bit_trainable_attention_amd/libsagebwd.so.
Flags: gfx950 only, -O3, packed-FP32 VALU instructions disabled (the compiler
otherwise emits v_pk_*_f32 by itself), no fast-math (the quantizer's float32
divisions and roundings must be the IEEE ones the tests check bit for bit),
and no floating-point contraction: every fused multiply-add is written out,
so each template instantiation of a kernel (the debug ones that dump a tile
included) rounds exactly the same operations.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libsagebwd.so")
SOURCES = ["prepare.hip", "fwd.hip", "bwd.hip", "api.hip", "selftest.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in SOURCES]

    def compile_one(i):
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, SOURCES[i]), "-o", objs[i]]
        if verbose:
            print(" ".join(cmd), flush=True)
        _run(cmd)

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        list(ex.map(compile_one, range(len(SOURCES))))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
