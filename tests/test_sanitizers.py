"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The host half of the C ABI (validation, workspace layout, cu_seqlens checks,
the allocation-free entry point's refusal) and the fp64 oracle are rebuilt
with the sanitizers (the device code is built as usual), and the CPU tests
that drive them run against those builds in a process of their own with the
sanitizer runtime preloaded. Any report fails the test.
"""
import os
import subprocess
import sys

import pytest

import mamba_ssd_sequence_fwd_amd.build as pkgbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang"
FILES = ["tests/test_abi_host.py", "tests/test_oracle_pins.py",
         "tests/test_chunk_log_decay_pins.py"]


def _runtime():
    r = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        rdir = subprocess.run([CLANG, "--print-runtime-dir"], capture_output=True,
                              text=True).stdout.strip()
        path = os.path.join(rdir, "libclang_rt.asan-x86_64.so")
    return path


def _build():
    os.makedirs(OUT, exist_ok=True)
    hipcc = pkgbuild._hipcc()
    flags = [f for f in pkgbuild.HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g"]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
    objs = []
    for src in pkgbuild.sources():
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        if not os.path.exists(obj) or os.path.getmtime(obj) < max(
                os.path.getmtime(p) for p in [src] + [os.path.join(pkgbuild.CSRC, h)
                                                     for h in os.listdir(pkgbuild.CSRC)]
                + [os.path.join(pkgbuild.INCLUDE, "ssd.h")]):
            subprocess.run([hipcc, *flags, *san, "-c", src, "-o", obj], check=True,
                           capture_output=True)
        objs.append(obj)
    lib = os.path.join(OUT, "libssd_san.so")
    subprocess.run([hipcc, "-shared", "-fPIC", "--offload-arch=%s" % pkgbuild.ARCH, "-o", lib,
                    *objs], check=True, capture_output=True)
    orc = os.path.join(OUT, "libssd_oracle_san.so")
    src = os.path.join(ROOT, "oracle", "ssd_oracle.c")
    subprocess.run([CLANG, "-O1", "-g", "-fPIC", "-shared", "-std=c99", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-o", orc, src, "-lm"], check=True, capture_output=True)
    return lib, orc


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang not installed")
def test_host_code_is_clean_under_asan_and_ubsan():
    lib, orc = _build()
    env = dict(os.environ)
    env["LD_PRELOAD"] = _runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitize_run.py"), lib, orc,
                        *FILES], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
