"""Build libkdaconv.so in-tree with hipcc for gfx950.

    python -m packed_varlen_causal_depthwise_amd.build
"""

from __future__ import annotations

import os
import pathlib
import shutil
import subprocess

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
SOURCES = [PKG / "csrc" / "kdaconv.hip"]
HEADERS = [ROOT / "include" / "kdaconv.h", PKG / "csrc" / "kdaconv_device.h"]
LIBRARY = PKG / "libkdaconv.so"
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # Packed FP32 instructions stay off: the compiler must not form them.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Exact IEEE binary32 semantics: no contraction, no flushing of subnormals.
    "-ffp-contract=off",
    "-fno-fast-math",
    "-fno-gpu-flush-denormals-to-zero",
    "-Wall",
]


def hipcc() -> str:
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def build(output: pathlib.Path = LIBRARY, extra_flags=()) -> pathlib.Path:
    tmp = output.with_name(output.name + f".tmp{os.getpid()}")
    cmd = [hipcc(), *FLAGS, *extra_flags, "-I", str(ROOT / "include"), "-o", str(tmp),
           *map(str, SOURCES)]
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build())
