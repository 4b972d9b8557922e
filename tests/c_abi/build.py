"""Build tests/c_abi/fused_from_c: a consumer of libce.so's C ABI with no
Python, checked against the oracle's C library (test infrastructure).

    python tests/c_abi/build.py

Needs libce.so (vocab_cross_entropy_amd/csrc/build.py) and libce_oracle.so
(oracle.build()) first; both are found at run time through the binary's rpath.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
OUT = os.path.join(HERE, "fused_from_c")


def build() -> str:
    pkg = os.path.join(ROOT, "vocab_cross_entropy_amd")
    orc = os.path.join(ROOT, "oracle")
    tmp = OUT + ".tmp"
    subprocess.run([HIPCC, "-O2", "-std=c++17", "-Wall", f"-I{ROOT}/include", f"-I{orc}",
                    os.path.join(HERE, "fused_from_c.cpp"), f"-L{pkg}", "-lce", f"-L{orc}", "-lce_oracle",
                    "-Wl,-rpath,$ORIGIN/../../vocab_cross_entropy_amd", "-Wl,-rpath,$ORIGIN/../../oracle",
                    "-Wl,-rpath,/opt/rocm/lib", "-o", tmp],
                   check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build())
