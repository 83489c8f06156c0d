"""Build the gfx950 HIP codec library in-tree (``libtq.so`` next to this file).

    python -m kv_cache_quantization_tq_amd.build

Always recompiles. Flags:
  -ffp-contract=off          products are rounded before they are added, as
                             the binary32 definition of every step requires;
  -packed-fp32-ops disabled  no v_pk_*_f32 instructions are generated.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "tq_codec.hip")
LIB = os.path.join(HERE, "libtq.so")
ARCH = os.environ.get("TQ_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-fconstexpr-steps=50000000",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
           "-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed building {SRC}")
    os.replace(tmp, LIB)
    return LIB


def build_asm(out: str) -> None:
    """Device assembly of the codec (for reading the generated ISA)."""
    cmd = [hipcc(), *[f for f in HIPCC_FLAGS if f not in ("-shared", "-fPIC")], "--cuda-device-only", "-S",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"), "-o", out, SRC]
    subprocess.run(cmd, check=True)


if __name__ == "__main__":
    print(build(verbose=True))
