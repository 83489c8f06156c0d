"""Build the gfx950 HIP codec library in-tree (``libtq.so`` next to this file).

    python -m kv_cache_quantization_tq_amd.build

Always recompiles. Each translation unit (the host API and one kernel unit
per head_dim) compiles in its own hipcc process, in parallel, then one link
step produces the shared library. Flags:
  -ffp-contract=off          products are rounded before they are added, as
                             the binary32 definition of every step requires;
  -packed-fp32-ops disabled  no v_pk_*_f32 instructions are generated.
Extra -D flags (compile-time tuning knobs of tq_device.h) may be passed
through the TQ_EXTRA_FLAGS environment variable.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import hashlib
import os
import shlex
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtq.so")
ARCH = os.environ.get("TQ_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-fconstexpr-steps=50000000",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


# Per-unit flags. The attention kernels keep their matrix-core accumulators
# in ordinary VGPRs: with accumulation registers the compiler copies every
# accumulator out and back on each tile around the (conditional) rescaling.
SOURCE_FLAGS = {"tq_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


# The sources each kind of kernel is built from (with include/tq.h); a
# measurement taken on a kernel stays valid while these files are unchanged.
BATCH_SOURCES = ("tq_batch.hip", "tq_host.h")
FIT_SOURCES = ("tq_fit.hip",)
ATTN_SOURCES = ("tq_attn.hip", "tq_device.h", "tq_host.h", "tq_tables.h")


def kernel_sources(kind: str = "all"):
    files = sorted(glob.glob(os.path.join(CSRC, "*")))
    if kind == "merge":
        files = [f for f in files if os.path.basename(f) in BATCH_SOURCES]
    elif kind == "fit":
        files = [f for f in files if os.path.basename(f) in FIT_SOURCES]
    elif kind == "attention":
        files = [f for f in files if os.path.basename(f) in ATTN_SOURCES]
    elif kind in ("encode", "decode", "unrotate", "codec"):
        files = [f for f in files if os.path.basename(f) not in ("tq_batch.hip", "tq_attn.hip") + FIT_SOURCES]
    return files + [os.path.join(ROOT, "include", "tq.h")]


def source_digest(kind: str = "all") -> str:
    """SHA-256 over the sources of one kind of kernel (all sources by default)
    and the public header."""
    h = hashlib.sha256()
    for p in kernel_sources(kind):
        h.update(os.path.basename(p).encode())
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def _flags(src: str = ""):
    return HIPCC_FLAGS + SOURCE_FLAGS.get(os.path.basename(src), []) + \
        shlex.split(os.environ.get("TQ_EXTRA_FLAGS", "")) + ["-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed: " + " ".join(cmd[-3:]))
    return r


def build(verbose: bool = False, out: str = LIB) -> str:
    with tempfile.TemporaryDirectory(prefix="tq_build_") as tmp:
        objs, cmds = [], []
        for src in sources():
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            objs.append(obj)
            cmds.append([hipcc(), *_flags(src), "-c", "-o", obj, src])
        workers = min(len(cmds), max(1, min(8, os.cpu_count() or 1)))
        with cf.ThreadPoolExecutor(workers) as ex:
            for cmd, _ in zip(cmds, ex.map(_run, cmds)):
                if verbose:
                    print(" ".join(cmd), flush=True)
        tmp_lib = out + ".tmp"
        link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib, *objs]
        if verbose:
            print(" ".join(link), flush=True)
        _run(link)
        os.replace(tmp_lib, out)
    return out


def build_asm(out_dir: str) -> None:
    """Device assembly of every kernel unit (for reading the generated ISA)."""
    os.makedirs(out_dir, exist_ok=True)
    cmds = [[hipcc(), *[f for f in _flags(s) if f != "-fPIC"], "--cuda-device-only", "-S",
             "-o", os.path.join(out_dir, os.path.basename(s) + ".s"), s] for s in sources()]
    with cf.ThreadPoolExecutor(8) as ex:
        list(ex.map(_run, cmds))


def kernel_resources(srcs=None) -> dict:
    """Per kernel of the device code: VGPRs (next free), LDS and scratch
    (private segment) bytes, read from the assembly hipcc produces with the
    build's flags. Scratch means register spills, which the kernels are
    written to avoid."""
    import re
    srcs = sources() if srcs is None else srcs
    res = {}
    with tempfile.TemporaryDirectory() as tmp:
        outs = [os.path.join(tmp, os.path.basename(s) + ".s") for s in srcs]
        cmds = [[hipcc(), *[f for f in _flags(s) if f != "-fPIC"], "--cuda-device-only", "-S", "-o", o, s]
                for s, o in zip(srcs, outs)]
        with cf.ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
            list(ex.map(_run, cmds))
        for o in outs:
            text = open(o).read()
            for m in re.finditer(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", text, re.S):
                body = m.group(2)
                field = lambda k: int(re.search(k + r" (\d+)", body).group(1))
                res[m.group(1)] = {"vgpr": field("next_free_vgpr"), "lds": field("group_segment_fixed_size"),
                                   "scratch": field("private_segment_fixed_size")}
    return res


if __name__ == "__main__":
    print(build(verbose=True))
