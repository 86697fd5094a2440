"""Build libdgmoe.so (HIP, gfx950) in place next to this file.

    python -m moe_denoise_forward_amd.build

Compiles every source under csrc/ with hipcc for gfx950 and links the shared
library; object files go to _build/ at the repository root.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build", "dgmoe")
LIB = os.path.join(PKG, "libdgmoe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CLANGXX = os.environ.get("DGMOE_CLANGXX", "/opt/rocm/llvm/bin/clang++")

SOURCES = ["dgmoe_api.cpp", "route.hip", "gemm.hip", "misc.hip", "head.hip", "attn.hip"]


def _runtime_link():
    """The HIP runtime, by its soname libamdhip64.so.7, found through the ROCm
    runpath when the library is used on its own.  In a PyTorch process the
    binding imports torch first; torch's bundled runtime carries the same soname,
    so the dynamic loader binds libdgmoe.so to that already-loaded copy and the
    process holds a single HIP runtime (a second one would see no device)."""
    return ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]


FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Wno-unused-function",
    # packed fp32 VALU ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # integer atomics stay single-lane as written: the wave-aggregating rewrite
    # reads the returned value right after the atomic, and that in-order wait
    # would also cover every load issued before it (the GEMM work-queue claims)
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    return r.returncode, out


def build(verbose=False):
    os.makedirs(OBJ, exist_ok=True)
    jobs = []
    for s in SOURCES:
        src = os.path.join(CSRC, s)
        obj = os.path.join(OBJ, s + ".o")
        lang = ["-x", "hip"] if s.endswith(".cpp") else []
        jobs.append((s, [HIPCC] + FLAGS + lang + ["-c", src, "-o", obj], obj))
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        results = list(ex.map(lambda j: (j[0], _run(j[1])), jobs))
    failed = False
    for name, (rc, out) in results:
        if out.strip() and (verbose or rc):
            print(f"--- {name}\n{out}", file=sys.stderr)
        failed |= rc != 0
    if failed:
        raise RuntimeError("libdgmoe: compilation failed")
    tmp = LIB + ".tmp"
    rc, out = _run([CLANGXX, "-shared", "-fPIC", "-o", tmp] + [j[2] for j in jobs] + _runtime_link())
    if rc:
        print(out, file=sys.stderr)
        raise RuntimeError("libdgmoe: link failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
