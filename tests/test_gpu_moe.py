"""The persistent MoE kernel on the GPU, against the oracle (parity rules in
tests/moe_check.py), for every workload shape, both schedulers and both combines, plus
edge cases (T = 0, T = 1, routing-tile boundaries, a single worker, reuse of one
workspace across token counts) and the final state of the event tensor."""

import numpy as np
import pytest
import torch

from moe_layer_scheduling_amd import binding, synth
from tests import moe_check
from tests.gpu_util import layers_to_device, require_gpu, run_moe, say

pytestmark = pytest.mark.gpu

# The dynamic (ready-queue) MoE scheduler is disabled on the GPU: its first GPU run did
# not terminate and the cause is not identified; the library refuses the mode unless the
# caller passes ETC_FLAG_ALLOW_DYNAMIC.  It is covered on the CPU execution harness
# instead (tests/test_cpu_emu.py).
DYN_SKIP = pytest.mark.skip(reason="dynamic MoE scheduler disabled on the GPU pending the "
                                   "cause of a non-terminating run; covered by the CPU harness")
# the schedulers that run on the GPU: static tickets and the dedicated scheduler workgroup
GPU_MODES = ("static", "dedicated")
MODES = ["static", pytest.param("dynamic", marks=DYN_SKIP), "dedicated"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _setup(cfg, T, call=0):
    layers = synth.make_layers(cfg)
    x = synth.make_x(cfg, T, call=call)
    return x, layers, layers_to_device(layers), synth.layers_as_numpy(layers)


def _compare(cfg, x, layers_np, gpu):
    return moe_check.compare(synth.as_numpy(x), layers_np, cfg.top_k, cfg.eps, cfg.dtype, gpu)


MID = synth.MoEConfig("mid", (300,), 512, 16, 6, 384, layers=2, zipf_s=0.5)


@pytest.mark.parametrize("mode", MODES)
def test_tiny_fp32(mode):
    cfg = synth.CONFIGS["tiny"]
    x, layers, ld, lnp = _setup(cfg, 16)
    say(f"tiny fp32 mode={mode}")
    gpu = run_moe(x.cuda(), ld, cfg.top_k, mode=mode)
    st = _compare(cfg, x, lnp, gpu)
    say(st)


@pytest.mark.parametrize("mode,combine", [("static", "atomic"),
                                          pytest.param("dynamic", "atomic", marks=DYN_SKIP),
                                          ("static", "ordered"),
                                          pytest.param("dynamic", "ordered", marks=DYN_SKIP),
                                          ("dedicated", "atomic"), ("dedicated", "ordered")])
def test_mid_two_layers(mode, combine):
    """300 tokens (ragged last routing tile), 16 experts (ragged row tiles), 2 layers."""
    cfg = MID
    x, layers, ld, lnp = _setup(cfg, 300)
    say(f"mid mode={mode} combine={combine}")
    ws = binding.MoEWorkspace(300, cfg.hidden, cfg.experts, cfg.top_k, cfg.ffn, cfg.layers,
                              torch.bfloat16, combine)
    gpu = run_moe(x.cuda(), ld, cfg.top_k, mode=mode, combine=combine, workspace=ws)
    say(_compare(cfg, x, lnp, gpu))


EDGE = synth.MoEConfig("edge", (70,), 384, 6, 2, 320, layers=2, zipf_s=0.3)


@pytest.mark.parametrize("combine", ["atomic", "ordered"])
def test_ragged_hidden_and_ffn_tiles(combine):
    """H = 384 and F = 320 end inside a column tile of both GEMMs."""
    cfg = EDGE
    x, layers, ld, lnp = _setup(cfg, 70)
    say(f"edge H=384 F=320 combine={combine}")
    gpu = run_moe(x.cuda(), ld, cfg.top_k, mode="static", combine=combine)
    say(_compare(cfg, x, lnp, gpu))


def test_ordered_combine_is_bit_reproducible():
    """Ordered combine: three calls give bit-identical outputs."""
    cfg = MID
    x, layers, ld, lnp = _setup(cfg, 300, call=1)
    ws = binding.MoEWorkspace(300, cfg.hidden, cfg.experts, cfg.top_k, cfg.ffn, cfg.layers,
                              torch.bfloat16, "ordered")
    xd = x.cuda()
    outs = [run_moe(xd, ld, cfg.top_k, mode="static", combine="ordered", workspace=ws)["out_tensor"].clone()
            for _ in range(3)]
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


@pytest.mark.parametrize("T", [1, 15, 16, 17, 33, 300])
def test_token_counts_share_one_workspace(T):
    """Edge token counts (one token, a routing tile +-1) through one workspace sized for
    300 tokens: no recompilation, the same kernel for every T."""
    cfg = MID.with_(layers=1)
    x, layers, ld, lnp = _setup(cfg, T, call=T)
    ws = _shared_ws(cfg)
    for mode in GPU_MODES:
        gpu = run_moe(x.cuda(), ld, cfg.top_k, mode=mode, workspace=ws)
        _compare(cfg, x, lnp, gpu)


_WS = {}


def _shared_ws(cfg):
    key = (cfg.hidden, cfg.experts, cfg.top_k, cfg.ffn, cfg.layers)
    if key not in _WS:
        _WS[key] = binding.MoEWorkspace(300, *key, torch.bfloat16)
    return _WS[key]


def test_zero_tokens_is_a_noop():
    cfg = MID.with_(layers=1)
    _, layers, ld, _ = _setup(cfg, 1)
    x = torch.empty(0, cfg.hidden, dtype=torch.bfloat16, device="cuda")
    out = binding.moe_layer(x, ld, cfg.top_k, workspace=_shared_ws(cfg))
    assert out.shape == (0, cfg.hidden)


@pytest.mark.parametrize("mode", MODES)
def test_single_worker(mode):
    """One workgroup runs the whole task graph alone (no deadlock in any mode); in
    dedicated mode one worker beside the scheduler workgroup."""
    cfg = MID.with_(layers=2)
    x, layers, ld, lnp = _setup(cfg, 40, call=7)
    gpu = run_moe(x.cuda(), ld, cfg.top_k, mode=mode, workers=2 if mode == "dedicated" else 1)
    _compare(cfg, x, lnp, gpu)


@pytest.mark.parametrize("mode", MODES)
def test_event_tensor_final_state(mode):
    """With the counters kept, every counter of the event tensor ends exactly at the
    value the scheduler model derives from the GPU's own routing and split."""
    cfg = MID
    T = 300
    x, layers, ld, lnp = _setup(cfg, T, call=3)
    ws = binding.MoEWorkspace(T, cfg.hidden, cfg.experts, cfg.top_k, cfg.ffn, cfg.layers,
                              torch.bfloat16)
    gpu = run_moe(x.cuda(), ld, cfg.top_k, mode=mode, workspace=ws,
                  flags=binding.FLAG_KEEP_COUNTERS)
    moe_check.check_event_tensor(lambda off, n: ws.view(off, n, torch.int32).cpu().numpy(),
                                 ws.layout, T, cfg.hidden, cfg.ffn, cfg.top_k, cfg.experts, gpu,
                                 cfg.layers)
    ws.reset()


def _trace_check(cfg, T, ws, gpu):
    rec = ws.read_trace()

    def read(off, cnt):
        return ws.view(off, cnt, torch.int32).cpu().numpy()

    checked = moe_check.check_trace_causality(rec, T, cfg.hidden, cfg.ffn, cfg.top_k, cfg.experts,
                                              gpu, ws.layout, read, cfg.layers)
    # the same trace against the data each task reads (independent of the counters)
    pairs = moe_check.check_data_dependencies(rec, T, cfg.hidden, cfg.top_k, cfg.experts, gpu,
                                              ws.layout, read, cfg.layers)
    assert pairs > 100
    return checked


@pytest.mark.parametrize("mode", GPU_MODES)
@pytest.mark.parametrize("which", ["mid", "decode"])
def test_trace_respects_every_dependency(which, mode):
    """On the device clock (a trace of one call): every task of the scheduler model ran
    exactly once, and none began before every task whose signals it waits for had
    signalled -- the event tensor's true dependencies hold on the hardware."""
    cfg, T = (MID, 300) if which == "mid" else (synth.CONFIGS["decode"], 64)
    x, layers, ld, lnp = _setup(cfg, T, call=13)
    ws = binding.MoEWorkspace(T, cfg.hidden, cfg.experts, cfg.top_k, cfg.ffn, cfg.layers,
                              torch.bfloat16)
    say(f"trace {which} T={T} mode={mode}")
    gpu = run_moe(x.cuda(), ld, cfg.top_k, mode=mode, workspace=ws, flags=binding.FLAG_TRACE)
    _compare(cfg, x, lnp, gpu)
    checked = _trace_check(cfg, T, ws, gpu)
    say(f"{checked} dependencies checked")
    assert checked > 100


LIMITS = synth.MoEConfig("limits", (200,), 256, 256, 16, 128, layers=1, zipf_s=0.5)
DEEP = synth.MoEConfig("deep", (40,), 256, 8, 2, 128, layers=4)


@pytest.mark.parametrize("combine", ["atomic", "ordered"])
@pytest.mark.parametrize("T", [40, 200])
def test_most_experts_and_top_k(T, combine):
    """256 experts and top-16 (the largest the library accepts), with the permutation
    scattered inside the scan (3 routing tiles) and by P tasks (13), through one
    workspace sized for 200 tokens."""
    cfg = LIMITS
    x, layers, ld, lnp = _setup(cfg, T, call=T)
    ws = binding.MoEWorkspace(200, cfg.hidden, cfg.experts, cfg.top_k, cfg.ffn, 1,
                              torch.bfloat16, combine)
    say(f"limits T={T} combine={combine}")
    gpu = run_moe(x.cuda(), ld, cfg.top_k, mode="static", combine=combine, workspace=ws)
    say(_compare(cfg, x, lnp, gpu))


@pytest.mark.parametrize("which", sorted(moe_check.DEGENERATE))
def test_degenerate_cases(which):
    """One expert with top-1, top-k equal to the expert count, identical experts (the
    output must not depend on the routing)."""
    cfg, layers, x = moe_check.degenerate_case(which)
    say(f"degenerate {which}")
    gpu = run_moe(x.cuda(), layers_to_device(layers), cfg.top_k, mode="static")
    say(moe_check.check_degenerate(which, cfg, x, layers, gpu))


# One expert with top-1: T sets the rows of the row tiles (see the CPU harness test of
# the same name): the layout boundaries 16 / 17, 32 / 33, 64 / 65 and a one-row tile
# after a full one, bf16 and float32.
ONE = synth.MoEConfig("one", (129,), 256, 1, 1, 128, layers=1)


@pytest.mark.parametrize("T", [1, 16, 17, 32, 33, 64, 65, 129])
def test_tile_layout_boundaries(T):
    for cfg in (ONE, ONE.with_(dtype="f32")):
        x, layers, ld, lnp = _setup(cfg, T, call=T)
        say(f"layout boundary T={T} {cfg.dtype}")
        gpu = run_moe(x.cuda(), ld, cfg.top_k, mode="static")
        _compare(cfg, x, lnp, gpu)


def test_four_chained_layers():
    """Four layers (the most one call chains) of a small shape."""
    cfg = DEEP
    x, layers, ld, lnp = _setup(cfg, 40)
    say("four layers")
    gpu = run_moe(x.cuda(), ld, cfg.top_k, mode="static")
    say(_compare(cfg, x, lnp, gpu))


# ------------------------------------------------------------------ workload shapes


def test_decode_sequence_one_kernel():
    """Decode shape (H=4096, E=8, k=2, F=14336): token counts 1, 4, 16, 64 drawn per call
    through one workspace sized for 64 -- the same compiled kernel serves them all."""
    cfg = synth.CONFIGS["decode"]
    layers = synth.make_layers(cfg)
    ld = layers_to_device(layers)
    lnp = synth.layers_as_numpy(layers)
    ws = binding.MoEWorkspace(64, cfg.hidden, cfg.experts, cfg.top_k, cfg.ffn, 1, torch.bfloat16)
    seq = [64, 1, 16, 4]  # every size once, largest first
    for i, T in enumerate(seq):
        x = synth.make_x(cfg, T, call=i)
        for mode in GPU_MODES:
            say(f"decode T={T} mode={mode}")
            gpu = run_moe(x.cuda(), ld, cfg.top_k, mode=mode, workspace=ws)
            say(_compare(cfg, x, lnp, gpu))


@pytest.mark.timeout(400)
def test_decode_32_calls_drawn_token_counts():
    """The decode workload as defined: 32 calls whose token counts are drawn from
    {1, 4, 16, 64} (seeded, every count at least once) through one workspace and the one
    compiled kernel, each call checked against the oracle."""
    cfg = synth.CONFIGS["decode"]
    layers = synth.make_layers(cfg)
    ld = layers_to_device(layers)
    lnp = synth.layers_as_numpy(layers)
    ws = binding.MoEWorkspace(64, cfg.hidden, cfg.experts, cfg.top_k, cfg.ffn, 1, torch.bfloat16)
    rng = np.random.default_rng(0)
    seq = [int(t) for t in rng.choice([1, 4, 16, 64], size=32)]
    for i, T in enumerate((1, 4, 16, 64)):  # every count at least once
        if T not in seq:
            seq[i] = T
    for i, T in enumerate(seq):
        x = synth.make_x(cfg, T, call=100 + i)
        say(f"decode call {i}: T={T}")
        gpu = run_moe(x.cuda(), ld, cfg.top_k, mode="static", workspace=ws)
        _compare(cfg, x, lnp, gpu)


def test_finegrained_zipf():
    cfg = synth.CONFIGS["finegrained"]
    x, layers, ld, lnp = _setup(cfg, 256)
    for mode in GPU_MODES:
        say(f"finegrained mode={mode}")
        gpu = run_moe(x.cuda(), ld, cfg.top_k, mode=mode)
        say(_compare(cfg, x, lnp, gpu))
    counts = gpu["counts"][0]
    assert counts[0] == counts.max() and (counts > 0).sum() < cfg.experts  # skewed


@pytest.mark.timeout(300)
def test_prefill_two_layers():
    """Full prefill shape (T=4096, H=4096, E=64, k=6, F=1408, two layers): routing,
    gates, counts, permutation and outputs of every token in both layers, each layer on
    the GPU's own input, plus the end-to-end chain."""
    cfg = synth.CONFIGS["prefill"]
    say("prefill: drawing inputs")
    x, layers, ld, lnp = _setup(cfg, 4096)
    for mode in GPU_MODES:
        say(f"prefill mode={mode}")
        gpu = run_moe(x.cuda(), ld, cfg.top_k, mode=mode)
        say(_compare(cfg, x, lnp, gpu))
