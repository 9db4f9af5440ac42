"""Build libmla_decode.so for gfx950 with hipcc (in-tree, no JIT cache)."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmla_decode.so")
SOURCES = ["mla_api.cpp", "mla_prep.hip", "mla_attn.hip", "mla_merge.hip", "mla_topk.hip", "mla_rope.hip",
           "mla_noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         # packed fp32 VALU ops stay off on this target
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops' is not a recognized" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        outs = list(ex.map(_run, cmds))
    tmp = LIB + ".tmp"
    outs.append(_run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]))
    os.replace(tmp, LIB)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
