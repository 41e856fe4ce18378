"""Builds libdory.so (the HIP kernels and the C ABI of include/dory.h) for gfx950.

Each .hip source compiles to an object in parallel, then they link into
looped_normalized_gpt_amd/libdory.so.  The q8_2f encoder is built with fp
contraction off so that its fp32 steps round exactly as written.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdory.so")
ARCH = os.environ.get("DORY_OFFLOAD_ARCH", "gfx950")

COMMON = ["hipcc", f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Wall", "-Wno-unused-parameter"]
PER_FILE = {"q8.hip": ["-ffp-contract=off"]}
SOURCES = ["api.hip", "gemv.hip", "rows.hip", "gemm.hip", "attn.hip", "q8.hip", "scratch.hip", "probe.hip"]


def _compile(src):
    obj = os.path.join(OUT, src.replace(".hip", ".o"))
    cmd = COMMON + PER_FILE.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature: that warning is noise
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode:
        raise RuntimeError(f"{' '.join(cmd)}\n{msgs}")
    return obj, msgs


def build(verbose: bool = False) -> str:
    os.makedirs(OUT, exist_ok=True)
    with cf.ThreadPoolExecutor(min(8, len(SOURCES))) as ex:
        results = list(ex.map(_compile, SOURCES))
    for obj, msgs in results:
        if verbose and msgs.strip():
            print(msgs)
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", LIB + ".tmp"] + [o for o, _ in results]
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
