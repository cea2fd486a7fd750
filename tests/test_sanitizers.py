"""The host-side layers under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU needed).

- The C ABI's host layer (capi.cpp, selfcheck.cpp and the overlap analysis
  they include) built with g++ for the CPU, the kernel launchers and the few
  HIP runtime calls replaced by recording stubs (tests/host/capi_sanitize.cpp),
  and driven through every argument check and a valid call of each entry
  point.
- The CPU oracle (oracle/oracle.c) built with gcc under both sanitizers and
  run through every pin of _pins.py, the interpreter started with the ASan
  runtime preloaded.
Any sanitizer report aborts the program (-fno-sanitize-recover=all).
"""
import os
import subprocess
import sys

import oracle.build as obuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bf16_rope_geglu_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def test_capi_host_layer_sanitized(tmp_path):
    exe = os.path.join(tmp_path, "capi_sanitize")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", *SAN, "-D__HIP_PLATFORM_AMD__",
                    "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    os.path.join(CSRC, "capi.cpp"), os.path.join(CSRC, "selfcheck.cpp"),
                    os.path.join(ROOT, "tests", "host", "capi_sanitize.cpp"), "-o", exe],
                   check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "ok"


def test_oracle_pins_sanitized(tmp_path):
    lib = os.path.join(tmp_path, "liboracle_san.so")
    subprocess.run(["gcc", *obuild.CFLAGS, "-O1", "-g", *SAN, obuild.SOURCE, "-o", lib, "-lm"],
                   check=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "host", "oracle_pins_run.py"),
                        lib], capture_output=True, text=True, env=env, timeout=900)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert r.stdout.strip().endswith("ok")
