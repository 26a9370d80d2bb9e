"""The allocation-free split-K entry point (etc_splitk_gemm_noalloc) on the GPU, through
the C ABI: its output equals the workspace entry point's (etc_splitk_gemm) bit for bit and
the oracle within the split-K rule, on two calls in a row -- the second with a smaller
input -- in both schedulers; shapes beyond its static scratch are refused before any HIP
call."""

import ctypes

import numpy as np
import pytest
import torch

from moe_layer_scheduling_amd import binding, synth
from oracle import splitk as osk
from tests.gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _pair(M, N, K, S, seed, mode):
    A, B = synth.make_splitk(M=M, N=N, K=K, seed=seed)
    Ad, Bd = A.cuda(), B.cuda()
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    c_free = binding.splitk_gemm_noalloc(Ad, Bd, S, mode=mode, status=status)
    c_ws = binding.splitk_gemm(Ad, Bd, S, mode=mode, check=True)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(c_free, c_ws), float((c_free - c_ws).abs().max())
    ref = osk.splitk_gemm(synth.as_numpy(A), synth.as_numpy(B), S)
    err = float(np.max(np.abs(c_free.cpu().numpy().astype(np.float64) - ref)))
    assert err <= 1e-3 * float(np.max(np.abs(ref))), err
    return err


@pytest.mark.parametrize("mode", ["static", "dynamic"])
def test_two_calls_match_the_workspace_entry_point(mode):
    cfg = synth.SPLITK
    say(f"no-alloc {mode}: full size, then a smaller shape")
    e1 = _pair(cfg["M"], cfg["N"], cfg["K"], cfg["split_k"], 0, mode)
    e2 = _pair(37, 256, 1024, 4, 3, mode)
    say(e1, e2)


def test_shapes_beyond_the_scratch_are_refused():
    lib = binding.load_library()
    # 64 x 4096 tiles with 64 slices: 64 MiB of partials > 16 MiB
    assert lib.etc_splitk_workspace_size(64, 4096, 64) > 16 << 20
    st = lib.etc_splitk_gemm_noalloc(64, 4096, 64 * 64, 64, 1 << 20, 2 << 20, 3 << 20, None, 0, 0, 0, None)
    assert st == 3
