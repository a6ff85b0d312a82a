"""Build libkvpop.so (HIP, gfx950) in-tree with hipcc.

Each source compiles to its own object in parallel, then one link.  Every
HIP line carries ``-Xclang -target-feature -Xclang -packed-fp32-ops`` so the
device compiler emits no packed fp32 VALU instructions.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkvpop.so")
ARCH = os.environ.get("KVPOP_ARCH", "gfx950")

SOURCES = ["api.hip", "fwd_lse.hip", "future_target.hip", "select.hip", "decode.hip",
           "cache_step.hip", "decode_step.hip", "running_topk.hip", "mlstm.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-result", "-munsafe-fp-atomics"]


def _compile(src):
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    warn = "\n".join(ln for ln in (r.stderr or "").splitlines() if noise not in ln)
    return obj, warn.strip()


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        results = list(ex.map(_compile, SOURCES))
    for (obj, warn), src in zip(results, SOURCES):
        if verbose and warn:
            print(f"[{src}]\n{warn}", flush=True)
    objs = [o for o, _ in results]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(LIB, flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
