"""Build libkvq.so in-tree with hipcc for gfx950.

    python -m decode_attention_streaming_amd.build
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libkvq.so")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# (source, object name, extra flags); the matrix-core kernels are built once per head_dim
SOURCES = [("kvq_runtime.cpp", "kvq_runtime", []), ("kvq_append.hip", "kvq_append", []),
           ("kvq_attention.hip", "kvq_attention", []), ("kvq_scratch.hip", "kvq_scratch", [])] + [
    ("kvq_attn_mfma.hip", "kvq_attn_mfma_d%d" % d, ["-DKVQ_D=%d" % d]) for d in (64, 128, 256)] + [
    ("kvq_attn_prefill.hip", "kvq_attn_prefill_d%d" % d, ["-DKVQ_D=%d" % d]) for d in (64, 128, 256)]
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # packed fp32 VALU instructions stay off: plain float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def _compile(item):
    src, name, extra = item
    obj = os.path.join(BUILD, name + ".o")
    cmd = [HIPCC] + FLAGS + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose=False):
    """Compile every source and link libkvq.so (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
