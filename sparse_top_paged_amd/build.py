"""Build libstp.so (the HIP kernels and their C ABI) for gfx950, in-tree.

    python sparse_top_paged_amd/build.py

Compiles every csrc/*.hip with hipcc and links the shared library next to
this file; csrc/diag.hip (the measurement kernels of include/stp_diag.h)
goes into libstp_diag.so beside it, linked against libstp.so.  Always
rebuilds.
"""

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libstp.so")
DIAG_LIB = os.path.join(HERE, "libstp_diag.so")
DIAG_SOURCES = {"diag.hip"}
OBJ_DIR = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
    # never emit packed fp32 add/mul/fma
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Per-source extra flags.  dense.hip: its softmax takes maxima of finite
# scores and -inf masks only, so fmaxf needs no NaN handling; without it the
# extend kernel's VALU work shrinks (measured 13 % faster, identical output).
# dense.hip: MFMA results in VGPRs, so that accumulators stay in one register
# file instead of being moved between AGPRs and VGPRs.  Not decode.hip, whose
# output waves keep O^T in 256 AGPRs (the flag makes it 12 % slower).
_VGPR_MFMA = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
EXTRA_FLAGS = {"dense.hip": ["-fno-honor-nans", *_VGPR_MFMA]}


def _compile(src):
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs, out, extra=()):
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, *extra, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link of {out} failed:\n{res.stderr}")
    os.replace(tmp, out)


def build(verbose=True):
    os.makedirs(OBJ_DIR, exist_ok=True)
    sources = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        objs = list(ex.map(_compile, sources))
    is_diag = [os.path.basename(src) in DIAG_SOURCES for src in sources]
    _link([o for o, d in zip(objs, is_diag) if not d], LIB)
    _link([o for o, d in zip(objs, is_diag) if d], DIAG_LIB,
          [f"-L{HERE}", "-lstp", "-Wl,-rpath,$ORIGIN"])
    if verbose:
        print(f"built {LIB} from {len(sources) - sum(is_diag)} sources and {DIAG_LIB}")
    return LIB


if __name__ == "__main__":
    build()
