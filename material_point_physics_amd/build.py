"""Build libmpm.so for gfx950 with hipcc (in-tree, no JIT cache).

Flags:
  --offload-arch=gfx950        CDNA4 only, no other target.
  -O3 -std=c++17 -fPIC -shared
  -munsafe-fp-atomics          float atomic add lowers to the native
                               global_atomic_add_f32 / ds_add_f32 instructions,
                               never to a compare-and-swap loop.
  -Xclang -target-feature -Xclang -packed-fp32-ops
                               no packed fp32 VALU instructions are generated.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc", "mpm.hip")
OUT = os.path.join(HERE, "libmpm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-munsafe-fp-atomics",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(out: str = OUT, extra=()) -> str:
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, SRC, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build_asm(out_dir: str) -> str:
    """Device assembly of our own gfx950 build, for inspecting the ISA."""
    os.makedirs(out_dir, exist_ok=True)
    cmd = [HIPCC, *[f for f in FLAGS if f not in ("-shared", "-fPIC")], "--cuda-device-only", "-S",
           SRC, "-o", os.path.join(out_dir, "mpm-gfx950.s")]
    subprocess.run(cmd, check=True)
    return os.path.join(out_dir, "mpm-gfx950.s")


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
