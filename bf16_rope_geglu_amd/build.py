"""Build lib/librgg.so: the HIP kernels and the C ABI, for gfx950 only.

    python -m bf16_rope_geglu_amd.build

build_capi_client() also compiles tests/host/capi_client.c, a plain C program
that drives the library through include/rgg.h with no Python in the way, and
build_stream_ref() the streaming reference kernel bench.py measures against
(lib/libstreamref.so, not part of the C ABI).

Flags: -ffp-contract=off keeps every multiply and add a separate IEEE op
(the bf16 rounding sits between them); packed-fp32 instructions are disabled;
symbols other than the C ABI are hidden.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(HERE, "lib")
LIBRARY = os.path.join(LIBDIR, "librgg.so")
SOURCES = [os.path.join(CSRC, "kernels.hip"), os.path.join(CSRC, "capi.cpp"),
           os.path.join(CSRC, "selfcheck.cpp"), os.path.join(CSRC, "noalloc.hip")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def build(out=LIBRARY, extra=()):
    """Compile the library to `out` (always recompiles); return its path."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, *SOURCES, "-o", tmp]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + proc.stdout + proc.stderr)
    os.replace(tmp, out)
    return out


STREAM_REF_SOURCE = os.path.join(CSRC, "stream_ref.hip")
STREAM_REF = os.path.join(LIBDIR, "libstreamref.so")


def build_stream_ref(out=STREAM_REF):
    """Compile the streaming reference that bench.py times beside each kernel."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    cmd = [HIPCC, *FLAGS, STREAM_REF_SOURCE, "-o", out + ".tmp"]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + proc.stdout + proc.stderr)
    os.replace(out + ".tmp", out)
    return out


CLIENT_SOURCE = os.path.join(ROOT, "tests", "host", "capi_client.c")
CLIENT = os.path.join(ROOT, "tests", "host", "_bin", "capi_client")
ROCM_LIB = "/opt/rocm/lib"


def build_capi_client(out=CLIENT, library=LIBRARY):
    """Compile the C client against `library` with gcc (C11, -Werror)."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    libdir = os.path.dirname(library)
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror",
           "-D__HIP_PLATFORM_AMD__", f"-I{INCLUDE}", "-I/opt/rocm/include",
           CLIENT_SOURCE, "-o", out + ".tmp",
           f"-L{libdir}", "-lrgg", f"-L{ROCM_LIB}", "-lamdhip64",
           f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{ROCM_LIB}"]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("gcc failed:\n" + proc.stdout + proc.stderr)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build())
    print(build_capi_client())
    print(build_stream_ref())
