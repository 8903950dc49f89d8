"""Build libpa.so (HIP kernels for gfx950 + the C ABI + the host allocator)
in-tree with hipcc. Run ``python -m paged_kv_cache_454_amd.build``.

Every source is compiled on each call (no staleness guesswork); objects go
to ``_build/`` next to this file and are linked into ``libpa.so`` here.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpa.so")
ROOT = os.path.dirname(HERE)

ARCH = "gfx950"
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIP_SOURCES = ["cache_write.hip", "copy_blocks.hip", "read_probe.hip", "decode.hip", "decode_tiled.hip", "decode_mfma.hip", "decode_balanced.hip", "decode_fp8.hip", "reduce.hip", "append.hip", "prefill.hip", "prefill_mfma.hip",
               "pa_api.hip"]
HOST_SOURCES = ["errors.cpp", "alloc.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I" + os.path.join(ROOT, "include")]
# gfx950 code is built without packed fp32 instructions (v_pk_*_f32).
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if src.endswith(".hip"):
        cmd = [hipcc()] + DEVICE + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
    else:
        cmd = [hipcc()] + COMMON + ["-x", "c++", "-D__HIP_PLATFORM_AMD__",
                                    "-I" + os.path.join(ROCM, "include"),
                                    "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the packed-fp32 feature; that warning is harmless.
    err = "\n".join(line for line in r.stderr.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    return obj, err.strip()


def build(verbose=False, jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    sources = HIP_SOURCES + HOST_SOURCES
    jobs = jobs or min(len(sources), max(1, (os.cpu_count() or 4)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_compile, sources))
    for obj, err in results:
        if verbose and err:
            print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + \
        [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
