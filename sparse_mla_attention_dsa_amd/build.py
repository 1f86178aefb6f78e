"""Compile the HIP sources into the in-tree shared library `libdsa.so` (gfx950).

Run as `python -m sparse_mla_attention_dsa_amd.build` or through
`__graft_entry__.build()`. Every call recompiles.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdsa.so")

SOURCES = ["dsa_api.cpp", "indexer.hip", "topk.hip", "sparse_mla.hip", "sparse_mla_fp8.hip", "quant.hip",
           "scratch.hip"]

ARCH = os.environ.get("DSA_OFFLOAD_ARCH", "gfx950")

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 instructions are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-source code generation options. The sparse attention kernel keeps its
# output accumulator in VGPRs (its rare rescale is VALU work on it) while q
# lives in AGPRs, and its LDS reads are scheduled as clauses ahead of the MFMAs.
# The indexer's MFMA results feed VALU epilogues directly from VGPRs.
SOURCE_FLAGS = {
    "sparse_mla.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1",
                       "-mllvm", "-amdgpu-sched-strategy=max-memory-clause"],
    "sparse_mla_fp8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1",
                           "-mllvm", "-amdgpu-sched-strategy=max-memory-clause"],
    "indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def _hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libdsa.so")
    return path


def _compile(src, extra):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = ([_hipcc()] + COMMON_FLAGS + SOURCE_FLAGS.get(src, []) + extra + lang +
           ["-c", os.path.join(CSRC, src), "-o", obj])
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj, res.stderr


def build(verbose=False, extra_flags=()):
    os.makedirs(BUILD, exist_ok=True)
    extra = list(extra_flags)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    objs = [r[0] for r in results]
    if verbose:
        for src, (_, err) in zip(SOURCES, results):
            if err.strip():
                print(f"[{src}]\n{err}", file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking libdsa.so failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


def source_digest():
    """Hash of the library sources (used to tell whether stored counter data is stale)."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
