"""Runs the CPU test suite (pytest -m "not gpu") with the oracle and the host side of the C ABI
built under AddressSanitizer and UndefinedBehaviorSanitizer (g++, host code only).

- oracle/sage2_oracle.cpp -> an instrumented oracle library;
- quantized_exact_attention_token_amd/csrc/host.cpp (argument checks, workspace layout, dispatch)
  -> an instrumented ABI library whose kernel launchers are stubs that enqueue nothing (the CPU
  suite exercises only the host-side paths of the ABI, and no GPU is used).
Both are built into a temporary directory and loaded in place of the normal ones in a child
Python process started with the ASan runtime preloaded. Exit status: the suite's.

    python tests/run_sanitized_cpu_suite.py
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-fno-omit-frame-pointer",
       "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
STUB = """#include "sage2_internal.h"
namespace sage2 {
int launch_prepass(const KArgs&, void*) { return 0; }
int launch_attn(const KArgs&, void*) { return 0; }
int launch_attn_dump(const KArgs&, void*) { return 0; }
}
"""
CHILD = """import os, sys
sys.path.insert(0, {root!r})
import quantized_exact_attention_token_amd as s
s.LIB_PATH = {abi!r}
import oracle
oracle._LIB = {orc!r}
s.lib(); oracle.lib()
loaded = [l.split()[-1] for l in open("/proc/self/maps")]
assert {abi!r} in loaded and {orc!r} in loaded, "instrumented libraries not loaded"
import pytest
sys.exit(pytest.main(["-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider", os.path.join({root!r}, "tests")]))
"""


def asan_runtime() -> str:
    out = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True)
    return os.path.realpath(out.stdout.strip())


def main() -> int:
    with tempfile.TemporaryDirectory() as tmp:
        orc = os.path.join(tmp, "libsage2_oracle_san.so")
        abi = os.path.join(tmp, "libsage2_host_san.so")
        stub = os.path.join(tmp, "stub_launchers.cpp")
        with open(stub, "w") as fh:
            fh.write(STUB)
        subprocess.run(["g++", *SAN, "-ffp-contract=off", "-pthread",
                        os.path.join(ROOT, "oracle", "sage2_oracle.cpp"), "-o", orc], check=True)
        csrc = os.path.join(ROOT, "quantized_exact_attention_token_amd", "csrc")
        subprocess.run(["g++", *SAN, "-I", os.path.join(ROOT, "include"), "-I", csrc,
                        os.path.join(csrc, "host.cpp"), stub, "-o", abi], check=True)
        env = dict(os.environ, LD_PRELOAD=asan_runtime(), ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        code = CHILD.format(root=ROOT, abi=abi, orc=orc)
        return subprocess.run([sys.executable, "-c", code], env=env).returncode


if __name__ == "__main__":
    sys.exit(main())
