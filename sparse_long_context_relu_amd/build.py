"""Builds libdsa.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree.

Run ``python -m sparse_long_context_relu_amd.build`` (or call ``build()``).
"""
from __future__ import annotations

import hashlib
import json
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libdsa.so")
SOURCES = ["dsa_api.hip", "indexer.hip", "indexer_decode.hip", "topk.hip", "sparse_mla.hip", "quantize.hip",
           "loss.hip", "sparse_bwd.hip", "ceiling.hip"]
HEADERS = ["common.h", "kernels.h", "indexer_common.h", "mla_tile.h"]

# Kernels whose machine code is fingerprinted at build time: a record measured
# on one build (profiles/traffic.json) stays valid while the fingerprint matches.
KERNEL_HASH_PATH = os.path.join(PKG, "kernel_isa.json")
# record name -> (source, symbol fragment of the instance)
HASHED_KERNELS = {"indexer_decode_kernel<bf16>": ("indexer_decode.hip", "indexer_decode_kernelILi1E")}

ARCH = "gfx950"
CXXFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # keep the compiler from emitting packed fp32 vector instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]
# Per-source flags.  The prefill indexer interleaves each group's MFMAs with the
# reduction of the previous group; machine sinking would move those MFMAs past
# the next branch, right in front of the instructions that read their results.
SOURCE_FLAGS = {"indexer.hip": ["-mllvm", "-disable-machine-sink"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the DSA library needs ROCm's hipcc to build")


# Host-side sanitizers for a checking build of the C ABI (the device code is
# compiled as usual): each flag applies to the host compilation only.
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def build(verbose: bool = False, jobs: int = 4, out_path: str = None, build_dir: str = None,
          sanitize_host: bool = False) -> str:
    """Compile every source for gfx950 and link libdsa.so next to this file (or
    at `out_path`; with `sanitize_host`, the host code under ASan and UBSan)."""
    build_dir = build_dir or BUILD_DIR
    out_path = out_path or LIB_PATH
    os.makedirs(build_dir, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    extra = SANITIZE_HOST if sanitize_host else []
    for src in SOURCES:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [cc, *CXXFLAGS, *SOURCE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _wait(procs.pop(0), verbose)
    for p in procs:
        _wait(p, verbose)
    tmp = out_path + ".tmp"
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if sanitize_host:
        link += ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan"]
    if verbose:
        print(" ".join(link), flush=True)
    res = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}")
    os.replace(tmp, out_path)
    if out_path == LIB_PATH:
        write_kernel_hashes(cc)
    return out_path


def kernel_isa_text(asm: str, kernel: str) -> str:
    """The instructions of every function in `asm` whose symbol names `kernel`
    (comments and the compilation-unit id dropped)."""
    keep, inside = [], False
    for line in asm.splitlines():
        if line.startswith("_Z") and kernel in line and line.split(";")[0].rstrip().endswith(":"):
            inside = True
        elif inside and line.lstrip().startswith(".Lfunc_end"):
            inside = False
        if inside and not line.lstrip().startswith(";"):
            keep.append(line.split(";")[0].rstrip())
    return "\n".join(keep)


def write_kernel_hashes(cc: str) -> dict:
    """SHA-256 of the gfx950 assembly of each fingerprinted kernel, to kernel_isa.json,
    with the compiler version line the library was built with."""
    out = {}
    ver = subprocess.run([cc, "--version"], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True).stdout
    out["hipcc_version"] = next((l.strip() for l in ver.splitlines() if "HIP version" in l), None)
    for name, (src, kernel) in HASHED_KERNELS.items():
        asm_path = os.path.join(BUILD_DIR, src + ".s")
        subprocess.run([cc, *CXXFLAGS, *SOURCE_FLAGS.get(src, []), "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", asm_path],
                       check=True, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
        with open(asm_path) as f:
            text = kernel_isa_text(f.read(), kernel)
        if not text:
            raise RuntimeError(f"{kernel} not found in the assembly of {src}")
        out[name] = hashlib.sha256(text.encode()).hexdigest()
    with open(KERNEL_HASH_PATH, "w") as f:
        json.dump(out, f, indent=1)
    return out


def _wait(item, verbose):
    src, p = item
    out, _ = p.communicate()
    text = out.decode(errors="replace")
    # hipcc's host pass does not know the packed-fp32 feature flag; that notice is harmless
    lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l]
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines))


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
