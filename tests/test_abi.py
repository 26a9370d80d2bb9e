"""The C ABI on the CPU: the library loads, exports every entry point the header
declares, sizes workspaces consistently, and rejects bad arguments before any HIP call
(no compute call is made here: there may be no GPU)."""

import ctypes
import os
import re
import subprocess

import pytest

from moe_layer_scheduling_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "etc_moe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from moe_layer_scheduling_amd import build

        build.build()
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(etc_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert "etc_moe_layer" in names and "etc_splitk_gemm" in names
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (etc_[a-z_0-9]+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(lib, n)
    # nothing beyond the header leaks out
    assert exported <= set(names), exported - set(names)


def test_version_and_status_strings(lib):
    assert lib.etc_abi_version() == binding.ABI_VERSION
    for code in range(7):
        assert lib.etc_status_string(code).decode()
    assert lib.etc_status_string(99).decode() == "unknown status"


def _moe_ws(lib, T, H=4096, E=64, k=6, F=1408, L=2, dt=1, comb=0):
    return lib.etc_moe_workspace_size(T, H, E, k, F, L, dt, comb)


def test_workspace_sizes(lib):
    sizes = [_moe_ws(lib, T) for T in (1, 16, 17, 4096, 8192)]
    assert all(s > 0 for s in sizes)
    assert sizes == sorted(sizes)  # monotone in max_tokens
    assert _moe_ws(lib, 4096, comb=1) > _moe_ws(lib, 4096)  # ordered keeps y rows
    assert _moe_ws(lib, 4096, dt=0) > _moe_ws(lib, 4096)  # float32 activations
    assert _moe_ws(lib, 16, H=100) == 0  # hidden not a multiple of 128
    assert _moe_ws(lib, 16, F=100) == 0  # ffn not a multiple of 64
    assert _moe_ws(lib, 16, H=384, F=320) > 0  # ragged tiles along H and F are masked
    assert _moe_ws(lib, 16, E=300, k=2) == 0
    assert _moe_ws(lib, 16, E=4, k=5) == 0
    assert _moe_ws(lib, 16, L=5) == 0
    assert lib.etc_splitk_workspace_size(64, 4096, 8) >= 32 * 8 * 64 * 128 * 4
    assert lib.etc_splitk_workspace_size(64, 100, 8) == 0
    assert lib.etc_splitk_workspace_size(64, 4096, 65) == 0


def test_layout_offsets_inside_workspace(lib):
    n = _moe_ws(lib, 4096)
    out = (ctypes.c_int64 * binding.LAYOUT_WORDS)()
    for layer in range(2):
        assert lib.etc_moe_workspace_layout(4096, 4096, 64, 6, 1408, 2, 1, 0, layer, out) == 0
        offs = list(out)
        assert all(0 < o < n and o % 4 == 0 for o in offs[:6] + [offs[13], offs[15]])
        assert offs[14] > 0 and offs[13] + 32 * offs[14] <= n
        assert offs[6] == 4096 * 6 // 128 + 64  # row-tile capacity
        bn1 = offs[11]
        assert offs[7] == (1408 + bn1 - 1) // bn1 and offs[8] == 4096 // offs[9]
    assert lib.etc_moe_workspace_layout(4096, 4096, 64, 6, 1408, 2, 1, 0, 2, out) == 1
    # the control words come first; layer 0's first counter follows them
    assert lib.etc_moe_workspace_layout(4096, 4096, 64, 6, 1408, 2, 1, 0, 0, out) == 0
    assert out[0] == binding.CONTROL_BYTES


def _call_moe(lib, **over):
    a = dict(T=16, H=128, E=4, k=2, F=256, L=1, dt=0, eps=1e-6, weights=None, x=8 * 1024,
             out=16 * 1024, layer_out=None, routing=None, ws=256 * 1024, wsb=1 << 30, maxT=16,
             mode=0, comb=0, flags=0, workers=0, stream=None)
    a.update(over)
    w = a["weights"]
    if w is None:
        w = (binding.MoeWeights * 1)()
        w[0].gamma, w[0].w_router, w[0].w_gate, w[0].w_up, w[0].w_down = 16, 32, 48, 64, 80
    return lib.etc_moe_layer(a["T"], a["H"], a["E"], a["k"], a["F"], a["L"], a["dt"], a["eps"], w,
                             a["x"], a["out"], a["layer_out"], a["routing"], a["ws"], a["wsb"],
                             a["maxT"], a["mode"], a["comb"], a["flags"], a["workers"], a["stream"])


def test_moe_argument_errors_before_any_hip_call(lib):
    INVALID, UNSUP, WS = 1, 2, 3
    assert _call_moe(lib, T=17) == INVALID  # T > max_tokens
    assert _call_moe(lib, T=-1) == INVALID
    assert _call_moe(lib, k=5) == INVALID  # top_k > experts
    assert _call_moe(lib, H=100) == UNSUP
    assert _call_moe(lib, F=96) == UNSUP
    assert _call_moe(lib, L=5) == UNSUP
    assert _call_moe(lib, mode=7) == INVALID
    assert _call_moe(lib, comb=3) == INVALID
    assert _call_moe(lib, dt=5) == INVALID
    assert _call_moe(lib, x=None) == INVALID
    assert _call_moe(lib, x=8 * 1024 + 2) == INVALID  # misaligned
    assert _call_moe(lib, eps=float("nan")) == INVALID
    bad = (binding.MoeWeights * 1)()
    assert _call_moe(lib, weights=bad) == INVALID  # null weight pointers
    assert _call_moe(lib, ws=None) == WS
    assert _call_moe(lib, ws=256 * 1024 + 16) == WS  # not 256-byte aligned
    assert _call_moe(lib, wsb=1024) == WS
    assert _call_moe(lib, mode=2, workers=1) == INVALID  # dedicated: a scheduler and a worker


def test_dynamic_moe_refused_without_the_flag(lib):
    """The dynamic MoE scheduler is refused unless the call sets ETC_FLAG_ALLOW_DYNAMIC
    (host check, before any HIP call); the library reads no environment variables."""
    assert _call_moe(lib, mode=1) == 2
    import subprocess
    strings = subprocess.run(["strings", binding.library_path()], capture_output=True, text=True).stdout
    assert "getenv" not in strings and "ETC_ENABLE" not in strings


def test_splitk_argument_errors_before_any_hip_call(lib):
    f = lib.etc_splitk_gemm
    ok = dict(M=64, N=4096, K=14336, S=8, A=1 << 20, B=2 << 20, C=3 << 20, ws=4 << 20, wsb=1 << 30)

    def call(**over):
        a = dict(ok, **over)
        return f(a["M"], a["N"], a["K"], a["S"], a["A"], a["B"], a["C"], a["ws"], a["wsb"], 0, 0, 0, None)

    assert call(M=0) == 1
    assert call(A=None) == 1
    assert call(B=(2 << 20) + 8) == 1
    assert call(N=100) == 2
    assert call(K=14336 + 64) == 2  # K not a multiple of 64 * split_k
    assert call(S=65) == 2
    assert call(wsb=100) == 3
    assert f(64, 4096, 14336, 8, 1 << 20, 2 << 20, 3 << 20, 4 << 20, 1 << 30, 2, 0, 0, None) == 1  # no dedicated mode


def test_no_cpu_fallback_without_library(tmp_path, monkeypatch):
    """The binding refuses to run when the library is absent."""
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(binding.EtcLibraryError):
        binding.load_library(str(tmp_path / "missing.so"))


def test_decode_attention_arguments_before_any_hip_call(lib):
    """Host-side validation of etc_decode_attention: sizes, pointers, alignment and the
    workspace, all before any HIP call (no GPU needed)."""
    f = lib.etc_decode_attention
    ws_n = lib.etc_decode_attention_workspace_size(32, 8, 4, 128, 200000)
    assert ws_n > 0
    assert lib.etc_decode_attention_workspace_size(32, 8, 4, 64, 200000) == 0  # head_dim != 128
    assert lib.etc_decode_attention_workspace_size(32, 8, 9, 128, 200000) == 0  # group > 8
    assert lib.etc_decode_attention_workspace_size(4096, 8, 4, 128, 200000) == 0  # batch > 2048
    assert lib.etc_decode_attention_workspace_size(0, 8, 4, 128, 200000) == 0
    # more tokens need more partial records
    assert lib.etc_decode_attention_workspace_size(32, 8, 4, 128, 400000) > ws_n
    ok = dict(B=32, HKV=8, G=4, D=128, lens=1 << 20, start=2 << 20, rows=200000, scale=0.088,
              q=3 << 20, k=4 << 20, v=5 << 20, out=6 << 20, ws=1 << 30, wsb=ws_n, mb=32, mt=200000,
              mode=0, flags=0, workers=0)

    def call(**over):
        a = dict(ok, **over)
        return f(a["B"], a["HKV"], a["G"], a["D"], a["lens"], a["start"], a["rows"], a["scale"],
                 a["q"], a["k"], a["v"], a["out"], a["ws"], a["wsb"], a["mb"], a["mt"], a["mode"],
                 a["flags"], a["workers"], None)

    assert call(B=0) == 1
    assert call(B=33) == 1  # more requests than the workspace holds
    assert call(D=64) == 2
    assert call(G=9) == 2
    assert call(lens=None) == 1
    assert call(lens=(1 << 20) + 2) == 1  # int32 array misaligned
    assert call(q=(3 << 20) + 8) == 1
    assert call(rows=0) == 1
    assert call(scale=float("nan")) == 1
    assert call(mode=3) == 1
    assert call(mode=2) == 1  # the dedicated scheduler is the MoE layer's only
    assert call(ws=None) == 3
    assert call(wsb=ws_n - 1) == 3
