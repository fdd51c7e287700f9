"""Sanitizer builds for the CPU tests (AddressSanitizer + UndefinedBehavior-
Sanitizer, host code only, g++):

  libkla_oracle_san.so  the fp64 oracle (oracle/kla_oracle.c), as
                        oracle/build.py builds it plus the sanitizers;
  libkla_host_san.so    the C-ABI layer (delta_rule_linear_amd/csrc/
                        kla_api.cpp) with stub launchers that report a HIP
                        error: argument validation, size queries and status
                        strings run under the sanitizers without a GPU.

    python tests/sanitize/build.py OUT_DIR
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g", "-O1"]


def build(out_dir):
    os.makedirs(out_dir, exist_ok=True)
    oracle_lib = os.path.join(out_dir, "libkla_oracle_san.so")
    subprocess.run(["gcc", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
                    "-fno-fast-math", "-ffp-contract=off"] + SAN +
                   [os.path.join(ROOT, "oracle", "kla_oracle.c"), "-o", oracle_lib], check=True)
    host_lib = os.path.join(out_dir, "libkla_host_san.so")
    subprocess.run(["g++", "-std=c++17", "-fPIC", "-shared", "-Wall", "-D__HIP_PLATFORM_AMD__",
                    "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include")] + SAN +
                   [os.path.join(ROOT, "delta_rule_linear_amd", "csrc", "kla_api.cpp"),
                    os.path.join(HERE, "stub_launch.cpp"), "-o", host_lib], check=True)
    return oracle_lib, host_lib


def runtime_preload():
    """The sanitizer runtimes to preload into an uninstrumented python."""
    libs = []
    for name in ("libasan.so", "libubsan.so"):
        p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                           check=True).stdout.strip()
        libs.append(os.path.realpath(p))
    return libs


if __name__ == "__main__":
    print(build(sys.argv[1] if len(sys.argv) > 1 else os.path.join(HERE, "_build")))
