"""Build libtv.so (HIP for gfx950) in-tree with hipcc.

The library is one shared object compiled from the sources in ``csrc/``; it exports the
C ABI declared in ``include/tv.h``. Usage: ``python -m draft_tree_verification_tv_amd.build``.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(REPO_ROOT, "include")
LIB_DIR = os.path.join(PKG_DIR, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libtv.so")
SOURCES = ["tv_api.hip", "tv_attn.hip", "tv_argmax.hip", "tv_tree.hip", "tv_commit.hip", "tv_kvquant.hip"]
# Measurement probes the benchmark runs beside the library (not part of the verify step).
PROBE_LIB_PATH = os.path.join(LIB_DIR, "libtv_probe.so")
PROBE_SOURCES = ["tv_probe.hip"]
ARCH = "gfx950"
# Per-file extras. Attention never produces or consumes NaN on valid input (masking uses
# -inf, which stays honoured), so fmaxf needs no NaN canonicalisation there; the argmax
# keeps IEEE NaN semantics.
EXTRA = {"tv_attn.hip": ["-fno-honor-nans"]}

# Packed fp32 VALU ops are disabled for all device code: the kernels rely on plain
# scalar fp32 arithmetic only.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; a ROCm toolchain is required to build libtv")


def _run(cmd, verbose):
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in res.stderr.splitlines() if noise not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def _build_lib(cc, sources, lib_path, tmpdir, verbose):
    objs, procs = [], []
    for src in sources:
        obj = os.path.join(tmpdir, src + ".o")
        cmd = [cc, *FLAGS, *EXTRA.get(src, []), f"-I{INCLUDE}", "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    for cmd, pr in procs:
        _, err = pr.communicate()
        noise = "is not a recognized feature for this target"
        err = "\n".join(ln for ln in err.splitlines() if noise not in ln)
        if pr.returncode != 0:
            raise RuntimeError(f"hipcc failed ({pr.returncode}):\n{' '.join(cmd)}\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
    fd, tmp = tempfile.mkstemp(prefix=os.path.basename(lib_path) + ".", suffix=".so.tmp", dir=LIB_DIR)
    os.close(fd)
    try:
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
        os.replace(tmp, lib_path)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libtv.so and libtv_probe.so (always recompiles).
    Returns the path of libtv.so."""
    os.makedirs(LIB_DIR, exist_ok=True)
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="tvbuild.") as tmpdir:
        _build_lib(cc, SOURCES, LIB_PATH, tmpdir, verbose)
        _build_lib(cc, PROBE_SOURCES, PROBE_LIB_PATH, tmpdir, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
