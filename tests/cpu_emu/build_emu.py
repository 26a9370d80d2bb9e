"""Compile the library's HIP sources unchanged as host C++ against the CPU stand-in
headers in this directory: libetc_moe_emu.so runs every kernel on CPU threads (for
finding hangs, races and out-of-bounds accesses on the CPU; see hip/hip_runtime.h)."""

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "moe_layer_scheduling_amd", "csrc")
CXX = "/opt/rocm/lib/llvm/bin/clang++"


def build(out=None, sanitize=None, opt="-O1"):
    out = out or os.path.join(HERE, "libetc_moe_emu.so" if not sanitize else f"libetc_moe_emu_{sanitize}.so")
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    cmd = [CXX, "-std=c++17", opt, "-g", "-fPIC", "-shared", "-Wno-unused-command-line-argument",
           "-I", HERE, "-x", "c++", *srcs, "-x", "none", os.path.join(HERE, "emu_runtime.cpp"),
           "-o", out, "-lpthread"]
    if sanitize:
        cmd[1:1] = [f"-fsanitize={sanitize}", "-fno-omit-frame-pointer"]
    if sanitize == "thread":  # atomics carry the ordering the GPU's completion waits give
        cmd[1:1] = ["-DETC_EMU_SC_ATOMICS"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


if __name__ == "__main__":
    print(build())
