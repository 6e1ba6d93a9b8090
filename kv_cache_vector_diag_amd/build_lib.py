"""Build libtq.so (host core + HIP kernels for gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["tq_host.cpp", "tq_abi.cpp", "tq_generic.hip", "tq_fast128.hip", "tq_score128.hip", "tq_split.hip", "tq_attend.hip", "tq_split256.hip", "tq_tiled.hip", "tq_wide.hip", "tq_decode.hip", "tq_haar256.hip", "tq_paged.hip", "tq_gram.hip", "tq_static.hip", "tq_score_lut.hip", "tq_decode_haar.hip"]

# Packed-FP32 VALU forms are disabled for every device pass; the host pass
# warns that it does not know the feature, which is harmless.  MFMA results
# are kept in ordinary VGPRs (gfx950 reads and writes them there directly):
# otherwise accumulators that also feed VALU code get copied through AGPRs
# around every matrix instruction.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form=1",
         "-Wall", "-Wno-unused-function"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def _check_symbols(lib: str) -> None:
    """Refuse a library that leaves one of its own symbols undefined.

    The host pass can skip a kernel template's launch stub without a
    diagnostic; the shared link then succeeds and the load fails later.
    """
    r = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True)
    if r.returncode != 0:
        return                      # no nm: nothing to check with
    own = [line.split()[-1] for line in r.stdout.splitlines() if line.split()[-1].startswith("_ZN2tq")]
    if own:
        os.remove(lib)
        raise RuntimeError("libtq.so leaves its own symbols undefined:\n  " + "\n  ".join(own))


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    _check_symbols(tmp)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
