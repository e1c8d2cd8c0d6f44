"""Builds libgdla.so (the GDLA C-ABI library) in-tree with hipcc for gfx950.

    python -m attention_gdla_prefill_decode_amd.build
"""

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libgdla.so")
CEILING_LIB = os.path.join(PKG, "libgdla_ceiling.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    # keep the compiler from forming packed fp32 instructions (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the disabled packed-fp32 feature: harmless.
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
    return r.returncode, msgs


def build(verbose=False, jobs=None):
    """Compiles every csrc/*.hip to an object in parallel (each kernel is launched from the file
    that defines it, so no relocatable device code is needed), then links libgdla.so."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(ROOT, "_build", "gdla")
    os.makedirs(objdir, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 1)
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    cmds, objs = [], []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src)[:-4] + ".o")
        objs.append(obj)
        cmds.append([hipcc] + compile_flags + ["-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj])
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    for cmd, (rc, msgs) in zip(cmds, results):
        if rc != 0:
            raise RuntimeError("hipcc failed (%d) on %s:\n%s" % (rc, cmd[-3], "\n".join(msgs)))
        if verbose and msgs:
            print("\n".join(msgs))
    tmp = LIB + ".tmp%d" % os.getpid()
    link = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    rc, msgs = _run(link)
    if rc != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc link failed (%d):\n%s" % (rc, "\n".join(msgs)))
    os.replace(tmp, LIB)
    # the benchmark's ceiling probes (measured MFMA and HBM rates), a library of their own
    tmp = CEILING_LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc] + HIPCC_FLAGS + [os.path.join(PKG, "ceiling", "ceiling.hip"), "-o", tmp]
    rc, msgs = _run(cmd)
    if rc != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed (%d) on ceiling.hip:\n%s" % (rc, "\n".join(msgs)))
    os.replace(tmp, CEILING_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
