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


def attention(lib, q, k, v, lens, kv_start, *, scale, mode="static", max_total=None, max_batch=None,
              workers=0, flags=0):
    """etc_decode_attention on host tensors.  Returns (out float64 array, status)."""
    B, HQ, D = q.shape
    HKV, rows, _ = k.shape
    G = HQ // HKV
    mb = max_batch or B
    mt = max_total or max(rows, 1)
    n = lib.etc_decode_attention_workspace_size(mb, HKV, G, D, mt)
    assert n > 0
    ws = torch.zeros(n + 256, dtype=torch.uint8)
    wptr = ws.data_ptr() + (-ws.data_ptr()) % 256
    out = torch.zeros(B, HQ, D, dtype=torch.float32)
    lens = torch.as_tensor(lens, dtype=torch.int32).contiguous()
    kv_start = torch.as_tensor(kv_start, dtype=torch.int32).contiguous()
    st = lib.etc_decode_attention(B, HKV, G, D, lens.data_ptr(), kv_start.data_ptr(), rows, scale,
                                  q.contiguous().data_ptr(), k.contiguous().data_ptr(),
                                  v.contiguous().data_ptr(), out.data_ptr(), wptr, n, mb, mt,
                                  binding.MODES[mode], flags, workers, None)
    assert st == 0, st
    status = ctypes.c_int32.from_address(wptr + 7 * 4).value
    return out.numpy().astype(np.float64), status
