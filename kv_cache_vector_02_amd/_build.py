"""Build libtq.so (the HIP library behind include/tq.h) in-tree for gfx950.

Every .hip file under csrc/ is compiled to an object with hipcc (in parallel),
then linked into kv_cache_vector_02_amd/libtq.so.  Packed-FP32 instruction
selection is disabled for all device code.  csrc/tq_pycall.c, the CPython
argument marshalling of the per-step calls, is built with gcc into the
package's _tqcall extension module.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys
import sysconfig

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtq.so")
PYCALL_SRC = os.path.join(CSRC, "tq_pycall.c")
PYCALL = os.path.join(PKG, "_tqcall" + (sysconfig.get_config_var("EXT_SUFFIX") or ".so"))
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Per-file code generation options: the encoder's matrix-core transform keeps
# its accumulators in ordinary vector registers (no moves out of the
# accumulation registers before the quantizer reads them).
FILE_FLAGS = {"tq_encode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> tuple[str, str]:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile and link; returns the path of libtq.so.  Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = jobs or min(16, os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_compile, srcs))
    objs = [o for o, _ in results]
    if verbose:
        for o, err in results:
            noise = [ln for ln in err.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
            if noise:
                print(o, "\n".join(noise), file=sys.stderr)
    tmp = LIB + ".tmp"
    # --no-undefined: a symbol missing from every object fails here, not at load time
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    build_pycall()
    return LIB


def build_pycall() -> str:
    """The _tqcall extension (plain C against the CPython API; it does not link libtq)."""
    tmp = PYCALL + ".tmp"
    cmd = [os.environ.get("CC", "gcc"), "-O2", "-std=c11", "-Wall", "-Werror", "-shared", "-fPIC",
           f"-I{sysconfig.get_paths()['include']}", f"-I{INCLUDE}", PYCALL_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building {os.path.basename(PYCALL)} failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PYCALL)
    return PYCALL


if __name__ == "__main__":
    print(build(verbose=True))
