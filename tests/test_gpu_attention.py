"""Variable-context decode attention on the GPU (csrc/attn.hip through the C ABI)
against the oracle's plain definition (oracle/attention.py), both schedulers.

Tolerance: max |gpu - ref| <= 1e-3 * max |ref|, the split-K rule for partials merged
through counters against a float64 reference.  The error budget: float32 accumulation of
bf16 products over head_dim 128 in the scores (relative ~1e-6), exp on the vector ALUs
(a few ulp), float32 sums of up to 256 weighted value rows per chunk and a float32 merge
of at most 128 chunks -- well under 1e-4 of the largest output."""

import numpy as np
import pytest
import torch

from moe_layer_scheduling_amd import binding, synth
from oracle import attention as oa
from tests.gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu
TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _case(lens, HKV, G, seed):
    q, k, v, start = synth.make_attention(lens, HKV, G, seed=seed)
    return q, k, v, start


def _ref(q, k, v, start, lens, G, scale):
    # the library's caches are head-major [H_kv][rows][D]; the oracle takes [rows][H_kv][D]
    kt = synth.as_numpy(k).transpose(1, 0, 2)
    vt = synth.as_numpy(v).transpose(1, 0, 2)
    return oa.decode_attention(synth.as_numpy(q), kt, vt, start.numpy(), np.asarray(lens), G, scale)


def _run(q, k, v, lens, start, mode, ws=None, workers=0, flags=0):
    lens_d = torch.as_tensor(lens, dtype=torch.int32).cuda()
    out = binding.decode_attention(q.cuda(), k.cuda(), v.cuda(), lens_d, start.cuda(), mode=mode,
                                   workspace=ws, workers=workers, flags=flags, check=True)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _assert_close(out, ref):
    err = float(np.max(np.abs(out - ref)))
    mx = float(np.max(np.abs(ref)))
    assert err <= TOL * mx, (err, mx)
    return err, mx


@pytest.mark.parametrize("mode", ["static", "dynamic"])
def test_ragged_lengths(mode):
    """One token, a chunk +-1, several chunks, in one call."""
    lens = [1, 255, 256, 257, 600, 1000, 3]
    q, k, v, start = _case(lens, 2, 4, seed=1)
    ref = _ref(q, k, v, start, lens, 4, 1 / np.sqrt(128))
    say(f"ragged {mode}:", _assert_close(_run(q, k, v, lens, start, mode), ref))


@pytest.mark.parametrize("G", [1, 2, 8])
def test_group_sizes(G):
    lens = [700, 90, 256]
    q, k, v, start = _case(lens, 4, G, seed=G)
    ref = _ref(q, k, v, start, lens, G, 1 / np.sqrt(128))
    _assert_close(_run(q, k, v, lens, start, "dynamic"), ref)


@pytest.mark.parametrize("mode", ["static", "dynamic"])
def test_serving_batch_full_size(mode):
    """The benchmarked workload: 32 requests, 32 query heads on 8 KV heads, context
    lengths drawn log-uniformly from [64, 32768] -- every output compared."""
    cfg = synth.ATTN
    lens = synth.draw_context_lens(cfg["batch"], cfg["min_len"], cfg["max_len"], cfg["seed"])
    q, k, v, start = _case(lens, cfg["kv_heads"], cfg["group"], seed=cfg["seed"])
    say(f"serving batch {mode}: {int(lens.sum())} tokens")
    ref = _ref(q, k, v, start, lens.numpy(), cfg["group"], 1 / np.sqrt(128))
    say(_assert_close(_run(q, k, v, lens, start, mode), ref))


def test_one_workspace_many_length_mixes():
    """One workspace and one compiled kernel for calls whose lengths differ in every
    call (the counter targets follow the lengths), including a 32768-token context."""
    HKV, G = 8, 4
    ws = binding.AttnWorkspace(16, HKV, G, 40000)
    rng = np.random.default_rng(0)
    mixes = [[32768], [1] * 16, [4096, 1, 17, 256, 257], list(rng.integers(1, 2500, size=16))]
    for i, lens in enumerate(mixes):
        q, k, v, start = _case(lens, HKV, G, seed=10 + i)
        say(f"mix {i}: {len(lens)} requests, {int(np.sum(lens))} tokens")
        ref = _ref(q, k, v, start, lens, G, 1 / np.sqrt(128))
        for mode in ("static", "dynamic"):
            _assert_close(_run(q, k, v, lens, start, mode, ws=ws), ref)


@pytest.mark.parametrize("mode", ["static", "dynamic"])
def test_counters_reach_their_length_dependent_targets(mode):
    """With the counters kept, ev[b][g] ends at ceil(L_b / 256) for every request and KV
    head: the targets the kernel derived from the lengths on the GPU."""
    lens = [1, 256, 257, 2000, 513]
    HKV, G = 3, 2
    q, k, v, start = _case(lens, HKV, G, seed=5)
    ws = binding.AttnWorkspace(len(lens), HKV, G, int(np.sum(lens)))
    ref = _ref(q, k, v, start, lens, G, 1 / np.sqrt(128))
    _assert_close(_run(q, k, v, lens, start, mode, ws=ws, flags=binding.FLAG_KEEP_COUNTERS), ref)
    # the counters follow the block of control words, one per 128-byte line
    words = ws.view(binding.CONTROL_BYTES, len(lens) * HKV * 32, torch.int32).cpu().numpy()
    ev = words[::32].reshape(len(lens), HKV)
    want = np.array([oa.split_count(L, 256) for L in lens])
    assert np.array_equal(ev, np.repeat(want[:, None], HKV, axis=1)), ev
    assert np.all(np.delete(words, np.arange(0, words.size, 32)) == 0)
    ws.reset()


@pytest.mark.parametrize("mode", ["static", "dynamic"])
def test_single_worker(mode):
    lens = [300, 5, 600]
    q, k, v, start = _case(lens, 2, 4, seed=7)
    ref = _ref(q, k, v, start, lens, 4, 1 / np.sqrt(128))
    _assert_close(_run(q, k, v, lens, start, mode, workers=1), ref)


def test_device_side_length_checks():
    """A zero length or rows past the cache: the kernel runs no task and reports
    ETC_ERR_INVALID_ARG in the device status; out is not written."""
    lens = [40, 60]
    q, k, v, start = _case(lens, 2, 4, seed=9)
    ws = binding.AttnWorkspace(2, 2, 4, 100)
    for bad in ([40, 0], [40, 61]):
        with pytest.raises(binding.EtcError) as ei:
            _run(q, k, v, bad, start, "static", ws=ws)
        assert ei.value.status == 1
        ws.reset()
