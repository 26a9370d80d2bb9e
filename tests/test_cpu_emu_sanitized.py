"""The kernels on the CPU execution harness built with AddressSanitizer (host code only:
the harness compiles the HIP sources as host C++): every MoE scheduler, split-K and decode
attention, with out-of-bounds accesses to any buffer (workspace, LDS arrays, operands)
reported."""

import os
import subprocess
import sys

from tests.cpu_emu import build_emu

HERE = os.path.dirname(os.path.abspath(__file__))


def test_kernels_under_address_sanitizer():
    lib = build_emu.build(sanitize="address")
    rt = subprocess.run([build_emu.CXX, "-print-file-name=libclang_rt.asan-x86_64.so"],
                        capture_output=True, text=True, check=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               ETC_EMU_CUS="4", ETC_EMU_STACK_KB="256")
    r = subprocess.run([sys.executable, os.path.join(HERE, "cpu_emu", "sanitized_run.py"), lib],
                       capture_output=True, text=True, env=env, timeout=900)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-6000:])
    assert "attention dynamic ok" in r.stdout
