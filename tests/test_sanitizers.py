"""AddressSanitizer / UndefinedBehaviorSanitizer builds of the host code, run on the CPU.

Two harnesses under tests/sanitizers/ are compiled with both sanitizers and run:
- host_checks.cpp drives every host-side argument check of the C ABI (the library's
  ffpa_api.hip and the backward's checks, compiled for the host only) with valid and invalid
  arguments, including the one check that reads memory (ffpa_check_cu_seqlens);
- oracle_calls.c drives the C oracle over every input kind it takes.
Any sanitizer report fails the run (-fno-sanitize-recover).  No GPU is involved.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitizers")
CSRC = os.path.join(ROOT, "exact_attention_head_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed:\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_calls")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "attn_oracle.c"), os.path.join(HERE, "oracle_calls.c"),
          "-o", exe, "-lm"])
    r = _run([exe], env=ENV, timeout=300)
    assert "0 failures" in r.stdout and "runtime error" not in r.stderr


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc is not installed")
def test_host_checks_under_sanitizers(tmp_path):
    # host-only objects: the sanitizers instrument host code (each flag after -Xarch_host)
    flags = ["-O1", "-g", "-std=c++17", "--offload-host-only", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all"]
    objs = []
    for src in (os.path.join(CSRC, "ffpa_api.hip"), os.path.join(CSRC, "ffpa_bwd.hip"),
                os.path.join(CSRC, "ffpa_dropout.hip"), os.path.join(HERE, "host_checks.cpp")):
        o = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, *flags, "-c", src, "-o", o])
        objs.append(o)
    exe = str(tmp_path / "host_checks")
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(HIPCC)))
    clang = os.path.join(rocm, "lib", "llvm", "bin", "clang++")
    # the kernel launchers live in the per-head-dim objects and are never reached by the checks
    _run([clang, "-fsanitize=address,undefined", *objs, "-o", exe, f"-L{rocm}/lib", "-lamdhip64",
          f"-Wl,-rpath,{rocm}/lib", "-Wl,--unresolved-symbols=ignore-all"])
    r = _run([exe], env=ENV, timeout=300)
    assert "0 failures" in r.stdout and "runtime error" not in r.stderr
