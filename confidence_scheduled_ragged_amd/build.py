"""Build libdspark.so (HIP, gfx950) in-tree with hipcc.

Every .hip source under csrc/ is compiled to an object in _build/ (in
parallel), then linked into confidence_scheduled_ragged_amd/libdspark.so.
The fused step (fused.hip) is compiled twice: once as is, once with
DSPARK_SLOTS32=1 (its kernels without 64-bit division, for steps whose slot
counts fit in 32 bits). Packed-fp32 instructions are disabled for device code.
"""
import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdspark.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-fvisibility=hidden",
          "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def units():
    """(source, extra flags, object name) of every object in the library."""
    out = [(src, [], os.path.basename(src) + ".o") for src in sources()]
    out.append((os.path.join(CSRC, "fused.hip"), ["-DDSPARK_SLOTS32=1"], "fused_slots32.o"))
    return out


def _compile(unit, verbose):
    src, extra, name = unit
    obj = os.path.join(BUILD, name)
    cmd = [HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    if verbose and r.stderr.strip():
        # the host pass does not know the packed-fp32 feature flag; that warning is harmless
        lines = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
        if lines:
            print("\n".join(lines), flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    todo = units()
    with ThreadPoolExecutor(max_workers=min(8, len(todo))) as ex:
        objs = list(ex.map(lambda u: _compile(u, verbose), todo))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
