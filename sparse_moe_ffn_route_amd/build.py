"""Build the gfx950 HIP library ``libmoe_hip.so`` in-tree.

Every source under ``csrc/`` is compiled by hipcc for gfx950 only, in parallel,
then linked into one shared library next to this file.  Packed-FP32 VALU
instructions are disabled for all device code.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libmoe_hip.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the MoE library)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(hipcc, src, obj, extra):
    cmd = [hipcc, *COMMON_FLAGS, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{res.stderr}")
    # the host pass does not know the packed-fp32 feature; that warning is expected
    noise = [ln for ln in res.stderr.splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln and "warning generated" not in ln
             and "warnings generated" not in ln]
    return "\n".join(noise)


def _stale(src, obj):
    """True when obj is missing or older than src or any header it may include."""
    if not os.path.exists(obj):
        return True
    deps = [src] + [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hpp")] + \
        [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h")]
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(d) > t for d in deps)


def build(verbose: bool = False, extra_flags=(), incremental: bool = False) -> str:
    """Compile every source for gfx950 and link ``libmoe_hip.so``; returns its path.

    incremental: recompile only sources whose object is older than the source or a header.
    """
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(BUILD_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    todo = [(s, o) for s, o in zip(srcs, objs) if not incremental or _stale(s, o)]
    workers = max(1, min(len(srcs), os.cpu_count() or 1, 8))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        futs = [ex.submit(_compile, hipcc, s, o, list(extra_flags)) for s, o in todo]
        for f in futs:
            msg = f.result()
            if msg and verbose:
                print(msg, file=sys.stderr)
    tmp = LIB_PATH + ".tmp"
    # -z defs: a symbol left undefined (e.g. a kernel whose host stub was not emitted)
    # fails the link here instead of the library's load
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True, incremental="--incremental" in sys.argv))
