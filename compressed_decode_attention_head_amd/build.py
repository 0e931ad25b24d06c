"""Builds libaatc.so in-tree for gfx950 (hipcc for the kernels, g++ for the host solver).

Usage: python -m compressed_decode_attention_head_amd.build   (or build() from Python)
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libaatc.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17", "-I", INCLUDE, "-I", CSRC,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-result", "-munsafe-fp-atomics"]
# per-source extra flags: the codec's quantizer must not be contracted into FMAs
EXTRA = {"aatc_codec.hip": ["-ffp-contract=off"]}
CXX = shutil.which("g++") or "g++"
CXX_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-I", INCLUDE, "-I", CSRC, "-Wall"]

SOURCES = ["aatc_host.cpp", "aatc_tiers.cpp", "aatc_codec.hip", "aatc_attn.hip", "aatc_attn_np1.hip", "aatc_attn_np2.hip",
           "aatc_attn_np3.hip", "aatc_attn_np4.hip", "aatc_probe.hip"]


def _compile(src):
    path = os.path.join(CSRC, src)
    obj = os.path.join(OBJ, src + ".o")
    if src.endswith(".cpp"):
        cmd = [CXX] + CXX_FLAGS + ["-c", path, "-o", obj]
    else:
        cmd = [HIPCC] + HIP_FLAGS + EXTRA.get(src, []) + ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def build(verbose=False):
    os.makedirs(OBJ, exist_ok=True)
    if os.path.exists(LIB):
        os.remove(LIB)          # a failed build must not leave an older library behind
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
