"""Build libhd.so (the HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

``python -m latent_sequence_length_amd.build`` compiles every ``csrc/*.hip``
into ``_build/*.o`` in parallel and links ``latent_sequence_length_amd/libhd.so``.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libhd.so")
ARCH = os.environ.get("HD_OFFLOAD_ARCH", "gfx950")

# Packed-FP32 VALU ops are switched off for device code: hipcc would otherwise
# emit v_pk_{add,mul,fma}_f32 from ordinary float code.
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-fno-honor-nans",  # no NaNs by contract: max/min need no canonicalisation
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = ["hipcc", *CFLAGS, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines()
                     if "packed-fp32-ops" not in l and "reserved registers: m0" not in l)
    return obj, warn


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(lambda s: _compile(s, verbose), srcs))
    for _, warn in results:
        if warn.strip():
            print(warn, file=sys.stderr)
    objs = [o for o, _ in results]
    tmp = LIB + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
