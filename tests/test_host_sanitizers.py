"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Every csrc/*.hip file is compiled with its host code instrumented (the device code is built as
usual, without sanitizers), and linked with
tests/abi_sanitize.cpp, which drives the argument validation and workspace planning of every
entry point of include/gdla.h.  Any out-of-bounds access, use after free, signed overflow,
invalid shift or misaligned access in that code stops the run with a sanitizer report."""

import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# -Xarch_host puts the sanitizers (and -g) on the host pass only
FLAGS = ["--offload-arch=gfx950", "-O1", "-Xarch_host", "-g", "-std=c++17", "-fno-omit-frame-pointer",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         "-Xarch_host", "-fno-sanitize-recover=all",
         "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]


def _compile(args):
    r = subprocess.run(args, capture_output=True, text=True)
    return r.returncode, (r.stdout + r.stderr)[-4000:]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
@pytest.mark.timeout(600)
def test_abi_host_code_under_asan_ubsan(tmp_path):
    srcs = sorted(glob.glob(os.path.join(ROOT, "attention_gdla_prefill_decode_amd", "csrc", "*.hip")))
    srcs.append(os.path.join(ROOT, "tests", "abi_sanitize.cpp"))
    objs, cmds = [], []
    for s in srcs:
        o = str(tmp_path / (os.path.basename(s) + ".o"))
        objs.append(o)
        lang = ["-x", "hip"] if s.endswith(".hip") else []
        cmds.append([HIPCC] + FLAGS + lang + ["-c", s, "-o", o])
    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        for cmd, (rc, msg) in zip(cmds, ex.map(_compile, cmds)):
            assert rc == 0, f"compile failed: {cmd[-3]}\n{msg}"
    exe = str(tmp_path / "abi_sanitize")
    rc, msg = _compile([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                        "-pthread"] + objs + ["-o", exe])
    assert rc == 0, f"link failed\n{msg}"
    env = dict(os.environ)
    # the HIP runtime's own start-up allocations are not the library's: no leak report
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "all checks passed" in r.stdout, out[-6000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-6000:]
