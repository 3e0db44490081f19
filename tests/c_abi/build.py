"""Build tests/c_abi/roundtrip: a C++ program that drives the C ABI directly and checks it
against the CPU oracle (test code; links oracle/liboracle.so and the product library)."""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "roundtrip.cpp")
EXE = os.path.join(HERE, "roundtrip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build() -> str:
    pkg = os.path.join(ROOT, "combine_topk_idx_expert_amd")
    orc = os.path.join(ROOT, "oracle")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-Wall",
           "-I", os.path.join(ROOT, "include"), "-I", orc, SRC, "-o", EXE + ".tmp",
           "-L", pkg, "-lep_mi355x", "-L", orc, "-loracle",
           "-Wl,-rpath,$ORIGIN/../../combine_topk_idx_expert_amd", "-Wl,-rpath,$ORIGIN/../../oracle"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build())
