"""Build libattn.so (the gfx950 attention library) in-tree with hipcc.

Every translation unit is compiled for gfx950 only, in parallel, and linked
into ``causal_self_attention_amd/libattn.so``.  Packed-fp32 instructions are
disabled for device code (``-packed-fp32-ops``); the host pass warns that it
does not know that feature, which is harmless.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libattn.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["attn_api.cpp", "attn_fwd.hip", "attn_bwd.hip", "attn_decode.hip", "attn_kv.hip", "attn_materialized.hip",
           "attn_prefill.hip", "attn_checks.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]


def build(verbose: bool = False) -> str:
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".", "_") + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([cc] + _flags() + lang + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        p = subprocess.run(cmd, capture_output=True, text=True)
        if p.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{p.stdout}\n{p.stderr}")
        return p.stderr

    with ThreadPoolExecutor(max_workers=min(len(cmds), 8)) as ex:
        for err in ex.map(run, cmds):
            if verbose and err.strip():
                print(err, file=sys.stderr)
    link = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", LIB + ".tmp"] + objs
    run(link)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
