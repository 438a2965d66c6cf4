"""Build libkda.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Every source under csrc/ is compiled to its own object (in parallel), then
linked into gated_delta_rule_11_amd/libkda.so.  Cross-compiles without a GPU.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libkda.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-fp32 instructions are disabled for all device code: hipcc -O3 would
# otherwise form v_pk_* fp32 ops from scalar code.
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + ["-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC] + COMMON + ["-x", "hip", "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    # surface real warnings; the host pass warns that it does not know the fp32 feature flag
    msgs = [l for l in r.stderr.splitlines() if "warning" in l and "packed-fp32-ops" not in l]
    if msgs and verbose:
        print("\n".join(msgs), flush=True)
    return obj


def _write_build_info():
    """Record which commit the library was built from (and whether its sources had
    uncommitted changes) next to it; the benchmark reports it."""
    import json

    def git(*a):
        try:
            r = subprocess.run(["git", "-C", ROOT] + list(a), capture_output=True, text=True, timeout=20)
            return r.stdout.strip() if r.returncode == 0 else None
        except (OSError, subprocess.SubprocessError):
            return None
    head = git("rev-parse", "HEAD")
    try:
        r = subprocess.run([HIPCC, "--version"], capture_output=True, text=True, timeout=60)
        hv = next((l.strip() for l in r.stdout.splitlines() if "clang version" in l), None)
    except (OSError, subprocess.SubprocessError):
        hv = None
    dirty = git("status", "--porcelain", "--", "gated_delta_rule_11_amd/csrc", "include")
    info = {"commit": head, "sources_modified_since_commit": bool(dirty) if dirty is not None else None,
            "arch": ARCH, "hipcc": HIPCC, "hipcc_version": hv}
    with open(os.path.join(HERE, "build_info.json"), "w") as fh:
        json.dump(info, fh)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    _write_build_info()
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    deps = sources() + [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hpp")]
    deps.append(os.path.join(ROOT, "include", "kda.h"))
    return any(os.path.getmtime(d) > t for d in deps)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
