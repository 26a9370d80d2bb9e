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
from oracle import attention as oa  # noqa: E402
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
    lens, HKV, G, D = [1, 257, 700], 2, 2, 128
    q, k, v, start = synth.make_attention(lens, HKV, G, seed=5)
    n = lib.etc_decode_attention_workspace_size(len(lens), HKV, G, D, int(np.sum(lens)))
    lens_t = torch.as_tensor(lens, dtype=torch.int32)
    kt = synth.as_numpy(k).transpose(1, 0, 2)
    vt = synth.as_numpy(v).transpose(1, 0, 2)
    ref = oa.decode_attention(synth.as_numpy(q), kt, vt, start.numpy(), np.asarray(lens), G, D ** -0.5)
    for mode in ("static", "dynamic"):
        ws = torch.zeros(n + 256, dtype=torch.uint8)
        wptr = ws.data_ptr() + (-ws.data_ptr()) % 256
        out = torch.zeros(len(lens), HKV * G, D, dtype=torch.float32)
        assert lib.etc_decode_attention(len(lens), HKV, G, D, lens_t.data_ptr(), start.data_ptr(),
                                        k.shape[1], D ** -0.5, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                        out.data_ptr(), wptr, n, len(lens), int(np.sum(lens)),
                                        binding.MODES[mode], 0, 0, None) == 0
        assert np.max(np.abs(out.numpy() - ref)) <= 1e-3 * np.max(np.abs(ref))
        print(f"attention {mode} ok", flush=True)


if __name__ == "__main__":
    os.environ.setdefault("ETC_EMU_CUS", "4")
    os.environ.setdefault("ETC_EMU_STACK_KB", "256")
    main(sys.argv[1])
