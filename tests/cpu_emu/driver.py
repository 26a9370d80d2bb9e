"""Call the CPU build of the library (libetc_moe_emu.so) through the same C ABI,
with host tensors standing in for device memory."""

import ctypes

import numpy as np
import torch

from moe_layer_scheduling_amd import binding, synth

DT = {"bf16": 1, "f32": 0}


def moe(lib, cfg, x, layers, *, mode="dynamic", combine="atomic", workers=0, flags=0,
        max_tokens=None, ws=None):
    T, H = x.shape
    L, k, E, F = len(layers), cfg.top_k, cfg.experts, cfg.ffn
    maxT = max_tokens or max(T, 1)
    if ws is None:
        n = lib.etc_moe_workspace_size(maxT, H, E, k, F, L, DT[cfg.dtype], binding.COMBINES[combine])
        assert n > 0
        ws = torch.zeros(n + 256, dtype=torch.uint8)
    base = ws.data_ptr()
    wptr = base + (-base) % 256
    nbytes = ws.numel() - 256
    warr = (binding.MoeWeights * L)()
    keep = []
    for l, w in enumerate(layers):
        for name in ("gamma", "w_router", "router_bias", "w_gate", "w_up", "w_down"):
            t = w.get(name)
            if t is not None:
                t = t.contiguous()
                keep.append(t)
                setattr(warr[l], name, t.data_ptr())
    out = torch.zeros(T, H, dtype=x.dtype)
    lay = torch.zeros(max(L - 1, 1), T, H, dtype=x.dtype)
    idx = torch.zeros(L, T, k, dtype=torch.int32)
    gw = torch.zeros(L, T, k, dtype=torch.float32)
    cnt = torch.zeros(L, E, dtype=torch.int32)
    sa = torch.zeros(L, T * k, dtype=torch.int32)
    r = binding.MoeRouting(idx.data_ptr(), gw.data_ptr(), cnt.data_ptr(), sa.data_ptr())
    if mode == "dynamic":  # the harness runs the dynamic scheduler, which needs the opt-in
        flags |= binding.FLAG_ALLOW_DYNAMIC
    st = lib.etc_moe_layer(T, H, E, k, F, L, DT[cfg.dtype], cfg.eps, warr, x.contiguous().data_ptr(),
                           out.data_ptr(), lay.data_ptr() if L > 1 else None, ctypes.byref(r), wptr,
                           nbytes, maxT, binding.MODES[mode], binding.COMBINES[combine], flags,
                           workers, None)
    assert st == 0, st
    status = ctypes.c_int32.from_address(wptr + 7 * 4).value
    outs = [lay[l] for l in range(L - 1)] + [out]
    return {"idx": idx.numpy().astype(np.int64), "w": gw.numpy().astype(np.float64),
            "counts": cnt.numpy().astype(np.int64), "sa": sa.numpy().astype(np.int64),
            "outs": [synth.as_numpy(o) for o in outs], "status": status, "ws": ws, "wptr": wptr}
