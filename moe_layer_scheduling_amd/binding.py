"""ctypes binding of libetc_moe.so (the C ABI in include/etc_moe.h).

Argument marshalling only: torch supplies device memory and the current stream; every
step of the computation runs in the library's kernels.  A missing library raises
``EtcLibraryError`` -- there is no fallback.
"""

import ctypes
import os
import threading

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libetc_moe.so")
ABI_VERSION = 0x00010002

STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported shape", 3: "workspace",
          4: "HIP runtime error", 5: "device wait timed out", 6: "no gfx950 device"}
DTYPES = {torch.float32: 0, torch.bfloat16: 1}
MODES = {"static": 0, "dynamic": 1, "dedicated": 2}  # dedicated: etc_moe_layer only
COMBINES = {"atomic": 0, "ordered": 1}
FLAG_KEEP_COUNTERS = 0x1
FLAG_TRACE = 0x2
FLAG_ALLOW_DYNAMIC = 0x4
LAYOUT_WORDS = 17
W_TRACE_LAST = 10  # control word holding the last traced call's record count
CONTROL_WORDS = 416  # int32 control words at the start of every workspace
CONTROL_BYTES = -(-CONTROL_WORDS * 4 // 256) * 256  # the region after them starts here


class EtcError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} (status {status})")


class EtcLibraryError(ImportError):
    pass


class MoeWeights(ctypes.Structure):
    _fields_ = [("gamma", ctypes.c_void_p), ("w_router", ctypes.c_void_p),
                ("router_bias", ctypes.c_void_p), ("w_gate", ctypes.c_void_p),
                ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p)]


class MoeRouting(ctypes.Structure):
    _fields_ = [("topk_idx", ctypes.c_void_p), ("topk_w", ctypes.c_void_p),
                ("expert_counts", ctypes.c_void_p), ("sorted_assign", ctypes.c_void_p)]


_lib = None
_lock = threading.Lock()


def library_path():
    return LIB_PATH


def open_library(path):
    """Open and type a build of the C ABI at `path` (no caching)."""
    if not os.path.exists(path):
        raise EtcLibraryError(
            f"{path} is missing: build it with `python -m moe_layer_scheduling_amd.build`")
    try:
        lib = ctypes.CDLL(path)
    except OSError as exc:
        raise EtcLibraryError(f"cannot load {path}: {exc}") from exc
    c_i32, c_u32, c_sz, c_p = ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t, ctypes.c_void_p
    lib.etc_abi_version.restype = c_i32
    lib.etc_status_string.restype = ctypes.c_char_p
    lib.etc_status_string.argtypes = [ctypes.c_int]
    lib.etc_moe_layer.restype = ctypes.c_int
    lib.etc_moe_layer.argtypes = [c_i32] * 6 + [ctypes.c_int, ctypes.c_float,
                                                ctypes.POINTER(MoeWeights), c_p, c_p, c_p,
                                                ctypes.POINTER(MoeRouting), c_p, c_sz, c_i32,
                                                ctypes.c_int, ctypes.c_int, c_u32, c_i32, c_p]
    lib.etc_moe_workspace_size.restype = c_sz
    lib.etc_moe_workspace_size.argtypes = [c_i32] * 6 + [ctypes.c_int, ctypes.c_int]
    lib.etc_moe_workspace_layout.restype = ctypes.c_int
    lib.etc_moe_workspace_layout.argtypes = [c_i32] * 6 + [ctypes.c_int, ctypes.c_int, c_i32,
                                                           ctypes.POINTER(ctypes.c_int64)]
    lib.etc_splitk_gemm.restype = ctypes.c_int
    lib.etc_splitk_gemm.argtypes = [c_i32] * 4 + [c_p, c_p, c_p, c_p, c_sz, ctypes.c_int, c_u32,
                                                  c_i32, c_p]
    lib.etc_splitk_gemm_noalloc.restype = ctypes.c_int
    lib.etc_splitk_gemm_noalloc.argtypes = [c_i32] * 4 + [c_p, c_p, c_p, c_p, ctypes.c_int, c_u32, c_i32, c_p]
    lib.etc_splitk_workspace_size.restype = c_sz
    lib.etc_splitk_workspace_size.argtypes = [c_i32] * 3
    lib.etc_workspace_init.restype = ctypes.c_int
    lib.etc_workspace_init.argtypes = [c_p, c_sz, c_p]
    lib.etc_query_device_status.restype = ctypes.c_int
    lib.etc_query_device_status.argtypes = [c_p, c_p]
    lib.etc_decode_attention.restype = ctypes.c_int
    lib.etc_decode_attention.argtypes = [c_i32] * 4 + [c_p, c_p, c_i32, ctypes.c_float, c_p, c_p, c_p,
                                                       c_p, c_p, c_sz, c_i32, ctypes.c_int64,
                                                       ctypes.c_int, c_u32, c_i32, c_p]
    lib.etc_decode_attention_workspace_size.restype = c_sz
    lib.etc_decode_attention_workspace_size.argtypes = [c_i32] * 4 + [ctypes.c_int64]
    lib.etc_default_workers.restype = c_i32
    lib.etc_default_workers.argtypes = [c_i32, ctypes.c_int]
    if lib.etc_abi_version() != ABI_VERSION:
        raise EtcLibraryError(f"{path} has ABI {lib.etc_abi_version():#x}, expected {ABI_VERSION:#x}")
    return lib


def load_library(path=None):
    """Load (once) the in-tree library; raise EtcLibraryError if it is absent."""
    global _lib
    with _lock:
        if _lib is None:
            _lib = open_library(path or LIB_PATH)
        return _lib


def _check(status, where):
    if status != 0:
        raise EtcError(status, where)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev_ptr(t, name, dtype=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


class Workspace:
    """Device scratch owned by the caller; cleared once at creation."""

    def __init__(self, nbytes, device=None):
        lib = load_library()
        self.nbytes = int(nbytes)
        # 256 bytes of slack so the start can be aligned to 256
        self.buffer = torch.empty(self.nbytes + 256, dtype=torch.uint8, device=device or "cuda")
        base = self.buffer.data_ptr()
        self.offset = (-base) % 256
        self.ptr = base + self.offset
        _check(lib.etc_workspace_init(self.ptr, self.nbytes, _stream()), "etc_workspace_init")

    def reset(self):
        _check(load_library().etc_workspace_init(self.ptr, self.nbytes, _stream()), "etc_workspace_init")

    def status(self):
        return load_library().etc_query_device_status(self.ptr, _stream())

    def view(self, offset, count, dtype):
        """Tensor view of workspace bytes [offset, offset + count * itemsize)."""
        itemsize = torch.empty((), dtype=dtype).element_size()
        start = self.offset + offset
        return self.buffer[start:start + count * itemsize].view(dtype)


class MoEWorkspace(Workspace):
    def __init__(self, max_tokens, hidden, experts, top_k, ffn, num_layers, dtype,
                 combine="atomic", device=None):
        lib = load_library()
        self.shape = (int(max_tokens), hidden, experts, top_k, ffn, num_layers)
        self.dtype = dtype
        self.combine = combine
        n = lib.etc_moe_workspace_size(*self.shape, DTYPES[dtype], COMBINES[combine])
        if n == 0:
            raise EtcError(2, "etc_moe_workspace_size")
        super().__init__(n, device)

    def layout(self, layer):
        lib = load_library()
        out = (ctypes.c_int64 * LAYOUT_WORDS)()
        _check(lib.etc_moe_workspace_layout(*self.shape, DTYPES[self.dtype], COMBINES[self.combine],
                                            layer, out), "etc_moe_workspace_layout")
        return list(out)

    def read_trace(self):
        """Records of the last call made with FLAG_TRACE, as a (n, 4) uint64 host array
        (decode with moe_layer_scheduling_amd.trace)."""
        torch.cuda.synchronize()
        lay = self.layout(0)
        n = int(self.view(4 * W_TRACE_LAST, 1, torch.int32).item())
        n = min(n, lay[14])
        return self.view(lay[13], 4 * n, torch.int64).cpu().numpy().view("u8").reshape(n, 4)


class SplitKWorkspace(Workspace):
    def __init__(self, M, N, split_k, device=None):
        n = load_library().etc_splitk_workspace_size(M, N, split_k)
        if n == 0:
            raise EtcError(2, "etc_splitk_workspace_size")
        self.shape = (M, N, split_k)
        super().__init__(n, device)


def moe_layer(x, layers, top_k, *, eps=1e-6, mode="static", combine="atomic", workspace=None,
              max_tokens=None, return_routing=False, return_layer_outputs=False, workers=0,
              flags=0, check=False):
    """Run len(layers) chained MoE layers on x [T][H] (float32 or bfloat16 device tensor).

    layers: list of dicts of device tensors gamma [H] f32, w_router [E][H], optional
    router_bias [E] f32, w_gate [E][F][H], w_up [E][F][H], w_down [E][H][F] (x's dtype).
    Returns out, or (out, info) when routing or layer outputs are requested.

    Device-side timeouts: when the binding allocates the workspace itself (workspace is
    None) or check is True, it synchronises the stream after the call and raises
    EtcError on a device timeout; otherwise the caller reads workspace.status().
    """
    lib = load_library()
    if x.dim() != 2:
        raise ValueError("x must be [T][H]")
    T, H = x.shape
    dtype = x.dtype
    if dtype not in DTYPES:
        raise ValueError(f"unsupported dtype {dtype}")
    L = len(layers)
    E, F = layers[0]["w_gate"].shape[0], layers[0]["w_gate"].shape[1]
    own = workspace is None
    if own:
        workspace = MoEWorkspace(max_tokens or max(T, 1), H, E, top_k, F, L, dtype, combine,
                                 device=x.device)
    if workspace.shape[1:] != (H, E, top_k, F, L) or workspace.dtype != dtype:
        raise ValueError("workspace was sized for another shape")
    if workspace.combine != combine and combine == "ordered":
        raise ValueError("the ordered combine needs a workspace sized for it")
    ws_max = workspace.shape[0]

    warr = (MoeWeights * L)()
    for l, w in enumerate(layers):
        warr[l].gamma = _dev_ptr(w["gamma"], "gamma", torch.float32)
        warr[l].w_router = _dev_ptr(w["w_router"], "w_router", dtype)
        warr[l].router_bias = _dev_ptr(w.get("router_bias"), "router_bias", torch.float32)
        warr[l].w_gate = _dev_ptr(w["w_gate"], "w_gate", dtype)
        warr[l].w_up = _dev_ptr(w["w_up"], "w_up", dtype)
        warr[l].w_down = _dev_ptr(w["w_down"], "w_down", dtype)

    out = torch.empty(T, H, dtype=dtype, device=x.device)
    layer_out = torch.empty(max(L - 1, 0), T, H, dtype=dtype, device=x.device) \
        if (return_layer_outputs and L > 1) else None
    routing = None
    info = {}
    if return_routing:
        info = {
            "topk_idx": torch.empty(L, T, top_k, dtype=torch.int32, device=x.device),
            "topk_w": torch.empty(L, T, top_k, dtype=torch.float32, device=x.device),
            "expert_counts": torch.empty(L, E, dtype=torch.int32, device=x.device),
            "sorted_assign": torch.empty(L, T * top_k, dtype=torch.int32, device=x.device),
        }
        routing = MoeRouting(*(info[k].data_ptr() for k in
                               ("topk_idx", "topk_w", "expert_counts", "sorted_assign")))
    st = lib.etc_moe_layer(T, H, E, top_k, F, L, DTYPES[dtype], float(eps), warr,
                           _dev_ptr(x, "x", dtype), out.data_ptr(),
                           layer_out.data_ptr() if layer_out is not None else None,
                           ctypes.byref(routing) if routing is not None else None,
                           workspace.ptr, workspace.nbytes, ws_max, MODES[mode],
                           COMBINES[combine], int(flags), int(workers), _stream())
    _check(st, "etc_moe_layer")
    if (own or check) and T > 0:
        _check(workspace.status(), "etc_moe_layer (device)")
    if layer_out is not None:
        info["layer_outputs"] = layer_out
    if return_routing or return_layer_outputs:
        return out, info
    return out


def splitk_gemm(A, B, split_k=8, *, mode="static", workspace=None, workers=0, flags=0,
                check=False):
    """C = A @ B (bfloat16 in, float32 out) through split_k event-counted partials.
    Device-side timeouts are raised as for moe_layer."""
    lib = load_library()
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    own = workspace is None
    if own:
        workspace = SplitKWorkspace(M, N, split_k, device=A.device)
    C = torch.empty(M, N, dtype=torch.float32, device=A.device)
    st = lib.etc_splitk_gemm(M, N, K, split_k, _dev_ptr(A, "A", torch.bfloat16),
                             _dev_ptr(B, "B", torch.bfloat16), C.data_ptr(), workspace.ptr,
                             workspace.nbytes, MODES[mode], int(flags), int(workers), _stream())
    _check(st, "etc_splitk_gemm")
    if own or check:
        _check(workspace.status(), "etc_splitk_gemm (device)")
    return C


class AttnWorkspace(Workspace):
    """Workspace of etc_decode_attention for up to max_batch requests whose context
    lengths sum to at most max_total_tokens."""

    def __init__(self, max_batch, kv_heads, group, max_total_tokens, head_dim=128, device=None):
        n = load_library().etc_decode_attention_workspace_size(max_batch, kv_heads, group, head_dim,
                                                               int(max_total_tokens))
        if n == 0:
            raise EtcError(2, "etc_decode_attention_workspace_size")
        self.shape = (int(max_batch), kv_heads, group, head_dim, int(max_total_tokens))
        super().__init__(n, device)


def decode_attention(q, k_cache, v_cache, context_lens, kv_start, *, scale=None, mode="static",
                     workspace=None, max_total_tokens=None, workers=0, flags=0, check=False):
    """out[b, h] = softmax(scale * q[b,h] K_b^T) V_b for one query token per request.

    q [B][H_kv*G][128] bfloat16; k_cache, v_cache [H_kv][rows][128] bfloat16; context_lens
    and kv_start device int32 [B] (request b's tokens are cache rows kv_start[b] ..
    kv_start[b] + L_b - 1).  Returns out [B][H_kv*G][128] float32.  Device-side errors
    (lengths out of range, too little workspace, timeouts) are raised as for moe_layer
    when the binding owns the workspace or check is True.
    """
    lib = load_library()
    B, HQ, D = q.shape
    HKV, rows, D2 = k_cache.shape
    if D2 != D or tuple(v_cache.shape) != (HKV, rows, D) or HQ % HKV:
        raise ValueError("q, k_cache and v_cache shapes disagree")
    G = HQ // HKV
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    own = workspace is None
    if own:
        workspace = AttnWorkspace(B, HKV, G, max_total_tokens or rows, D, device=q.device)
    mb, whkv, wg, wd, mt = workspace.shape
    if (whkv, wg, wd) != (HKV, G, D) or B > mb:
        raise ValueError("workspace was sized for another shape")
    out = torch.empty(B, HQ, D, dtype=torch.float32, device=q.device)
    st = lib.etc_decode_attention(B, HKV, G, D, _dev_ptr(context_lens, "context_lens", torch.int32),
                                  _dev_ptr(kv_start, "kv_start", torch.int32), rows, float(scale),
                                  _dev_ptr(q, "q", torch.bfloat16), _dev_ptr(k_cache, "k_cache", torch.bfloat16),
                                  _dev_ptr(v_cache, "v_cache", torch.bfloat16), out.data_ptr(),
                                  workspace.ptr, workspace.nbytes, mb, mt, MODES[mode], int(flags),
                                  int(workers), _stream())
    _check(st, "etc_decode_attention")
    if own or check:
        _check(workspace.status(), "etc_decode_attention (device)")
    return out


def splitk_gemm_noalloc(A, B, split_k=8, *, mode="static", out=None, status=None, workers=0, flags=0):
    """C = A @ B like splitk_gemm, through the library's allocation-free entry point (its
    partials live in a static device array; no workspace is passed).  out: optional
    preallocated float32 [M][N]; status: optional device int32 [1] that receives the
    kernel's device status."""
    lib = load_library()
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    C = out if out is not None else torch.empty(M, N, dtype=torch.float32, device=A.device)
    st = lib.etc_splitk_gemm_noalloc(M, N, K, split_k, _dev_ptr(A, "A", torch.bfloat16),
                                     _dev_ptr(B, "B", torch.bfloat16), _dev_ptr(C, "out", torch.float32),
                                     _dev_ptr(status, "status", torch.int32), MODES[mode], int(flags),
                                     int(workers), _stream())
    _check(st, "etc_splitk_gemm_noalloc")
    return C


def default_workers(kind="moe", dtype=torch.bfloat16):
    return load_library().etc_default_workers(0 if kind == "moe" else 1, DTYPES[dtype])
