"""Build libpa.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m paged_kv_cache_138_amd.build [--verbose]

Every source under csrc/ is compiled with hipcc for gfx950 in parallel and
linked into paged_kv_cache_138_amd/libpa.so. Packed-fp32 instructions are
disabled for the device code.
"""

import argparse
import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpa.so")
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")

DEVICE_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]


# Per-source flags. The prefill instances assume no NaN operands: their max
# operations then need no quieting of signalling NaNs (two instructions per
# max of values the compiler cannot prove canonical); infinities, which the
# masks use, are still honoured.
FILE_FLAGS = {"pa_inst_prefill.hip": ["-fno-honor-nans"],
              "pa_inst_prefill_shared.hip": ["-fno-honor-nans"]}


def hipcc():
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found")
    return h


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
    if p.returncode != 0:
        raise RuntimeError("build failed: %s\n%s" % (" ".join(cmd), out))
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose=False, jobs=None, extra_flags=(), out=None):
    """Compile every csrc/*.hip and link libpa.so (or `out`). Always rebuilds."""
    out = out or LIB
    objdir = OBJDIR if out == LIB else out + ".objs"
    os.makedirs(objdir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no sources under %s" % CSRC)
    cc = hipcc()
    objs = []
    cmds = []
    for s in srcs:
        o = os.path.join(objdir, os.path.basename(s) + ".o")
        objs.append(o)
        cmds.append([cc] + DEVICE_FLAGS + FILE_FLAGS.get(os.path.basename(s), []) +
                    list(extra_flags) +
                    ["-I", INCLUDE, "-I", CSRC, "-c", s, "-o", o])
    jobs = jobs or min(8, len(cmds))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = out + ".tmp"
    _run([cc, "-shared", "-fPIC", "--offload-arch=" + ARCH] + objs + ["-o", tmp], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--out", default=None, help="library path (default: in-tree libpa.so)")
    ap.add_argument("-D", dest="defines", action="append", default=[],
                    help="extra preprocessor definition for a variant build")
    args = ap.parse_args()
    print(build(verbose=args.verbose, extra_flags=["-D" + d for d in args.defines], out=args.out))
    sys.exit(0)
