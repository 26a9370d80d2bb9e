"""One MoE call on the CPU harness with a dropped signal planted in the event tensor:
layer 0's ev_comb[0] starts far below zero, so the finalize task of routing tile 0 can
never see its target (static mode: its wait never completes; dynamic mode: the down task
whose signal should complete the counter never sees it complete, so the finalize task is
never queued).  Run as a script (its own process, so that the harness clock can run in
real time): prints one JSON line with the call's return code, the device status word, the
site of the wait that gave up and the seconds the call took, then clears the workspace
and runs the same call again to show that the workspace is usable afterwards."""

import ctypes
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from moe_layer_scheduling_amd import binding, synth  # noqa: E402
from tests.cpu_emu import driver  # noqa: E402

W_STATUS, W_AUX = 7, 8


def main(lib_path, mode):
    lib = binding.open_library(lib_path)
    cfg = synth.CONFIGS["tiny"]
    layers, x = synth.make_layers(cfg), synth.make_x(cfg, 16)
    T, H, E, k, F = 16, cfg.hidden, cfg.experts, cfg.top_k, cfg.ffn
    n = lib.etc_moe_workspace_size(T, H, E, k, F, 1, 0, 0)
    ws = torch.zeros(n + 256, dtype=torch.uint8)
    wptr = ws.data_ptr() + (-ws.data_ptr()) % 256
    lay = (ctypes.c_int64 * binding.LAYOUT_WORDS)()
    assert lib.etc_moe_workspace_layout(T, H, E, k, F, 1, 0, 0, 0, lay) == 0
    ctypes.c_int32.from_address(wptr + lay[3]).value = -(1 << 30)  # ev_comb[0] of layer 0
    t0 = time.time()
    g = driver.moe(lib, cfg, x, layers, mode=mode, ws=ws)
    took = time.time() - t0
    words = (ctypes.c_int32 * 16).from_address(wptr)
    res = {"status": int(words[W_STATUS]), "where": int(words[W_AUX]), "seconds": took}
    # afterwards: a cleared workspace serves the same call correctly
    assert lib.etc_workspace_init(wptr, n, None) == 0
    g2 = driver.moe(lib, cfg, x, layers, mode=mode, ws=ws)
    res["status_after_init"] = int(g2["status"])
    res["out_after_init"] = g2["outs"][-1].tolist()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main(sys.argv[1], sys.argv[2])
