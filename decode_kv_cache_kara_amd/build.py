"""Builds libkara.so (the HIP kernels for gfx950 and the C ABI front end) in
the package directory with hipcc.  Run as a script or via build_library()."""

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkara.so")
SOURCES = ["kara_api.cpp", "kara_score.hip", "kara_score_bf16_d128.hip", "kara_score_bf16_d64.hip",
           "kara_score_f32_d128.hip", "kara_score_f32_d64.hip", "kara_score_resident.hip", "kara_select.hip", "kara_compact.hip",
           "kara_decode.hip", "kara_policy.cpp", "kara_probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms stay disabled: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wno-unused-command-line-argument",
]
# roctx ranges of the C ABI calls (rocprofv3 --marker-trace)
LINK_LIBS = ["-L/opt/rocm/lib", "-lrocprofiler-sdk-roctx", "-Wl,-rpath,/opt/rocm/lib"]
# the host pass does not know the packed-fp32 feature name; that warning is expected
_NOISE = "is not a recognized feature for this target"


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(x for x in r.stderr.splitlines() if _NOISE not in x)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + err)
    return err


def build_library(verbose=False, extra_flags=(), out=None):
    """Compiles every source to an object (in parallel; each translation unit
    launches only its own kernels) and links libkara.so."""
    out = out or LIB
    objdir = tempfile.mkdtemp(prefix="kara_build_")
    try:
        objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [[HIPCC] + FLAGS + list(extra_flags) + ["-c", os.path.join(CSRC, s), "-o", o]
                for s, o in zip(SOURCES, objs)]
        workers = max(1, min(len(cmds), os.cpu_count() or 1))
        with concurrent.futures.ThreadPoolExecutor(workers) as pool:
            errs = list(pool.map(_run, cmds))
        tmp = out + ".tmp"
        errs.append(_run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + LINK_LIBS + ["-o", tmp]))
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
            for e in errs:
                if e.strip():
                    print(e, file=sys.stderr)
        os.replace(tmp, out)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True))
