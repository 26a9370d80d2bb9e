"""Runs a few calls of every kernel on the CPU harness built with a sanitizer (run as a
child process, with the sanitizer's runtime preloaded).  Usage:
    sanitized_run.py <library>
Exit status 0 when every call completed, matched the oracle and the sanitizer reported
nothing (a report makes it exit non-zero)."""

import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402
import torch  # noqa: E402

from moe_layer_scheduling_amd import binding, synth  # noqa: E402
from oracle import splitk as osk  # noqa: E402
from tests import moe_check  # noqa: E402
from tests.cpu_emu import driver  # noqa: E402


def main(path):
    lib = binding.open_library(path)
    mid = synth.MoEConfig("mid", (300,), 512, 16, 6, 384, layers=2, zipf_s=0.5)
    cases = [("static", mid, 40), ("dynamic", synth.CONFIGS["tiny"], 16),
             ("dedicated", synth.CONFIGS["tiny"], 16)]
    for mode, cfg, T in cases:
        layers, x = synth.make_layers(cfg), synth.make_x(cfg, T)
        g = driver.moe(lib, cfg, x, layers, mode=mode, max_tokens=300)
        assert g["status"] == 0, (mode, cfg.name, g["status"])
        moe_check.compare(synth.as_numpy(x), synth.layers_as_numpy(layers), cfg.top_k, cfg.eps,
                          cfg.dtype, g)
        print(f"moe {mode} {cfg.name} T={T} ok", flush=True)
    M, N, K, S = 37, 256, 1024, 4
    A, B = synth.make_splitk(M=M, N=N, K=K, seed=2)
    n = lib.etc_splitk_workspace_size(M, N, S)
    ref = osk.splitk_gemm(synth.as_numpy(A), synth.as_numpy(B), S)
    for mode in ("static", "dynamic"):
        ws = torch.zeros(n + 256, dtype=torch.uint8)
        wptr = ws.data_ptr() + (-ws.data_ptr()) % 256
        C = torch.zeros(M, N, dtype=torch.float32)
        assert lib.etc_splitk_gemm(M, N, K, S, A.data_ptr(), B.data_ptr(), C.data_ptr(), wptr, n,
                                   binding.MODES[mode], 0, 0, None) == 0
        assert np.max(np.abs(C.numpy() - ref)) <= 1e-3 * np.max(np.abs(ref))
        print(f"splitk {mode} ok", flush=True)


if __name__ == "__main__":
    os.environ.setdefault("ETC_EMU_CUS", "4")
    os.environ.setdefault("ETC_EMU_STACK_KB", "256")
    main(sys.argv[1])
