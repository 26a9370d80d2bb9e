"""Pins of the MoE-layer oracle (CPU only).

Each oracle step is checked against something other than itself: the hand-worked case
in ``tests/golden/moe_hand_case.json``, closed forms, invariants the layer must keep
(counts sum to T*k, the permutation is a bijection, gates sum to 1), library routines
(stable argsort, bincount, scipy softmax, fp64 matmul), brute force over every k-subset
and over every (token, expert) pair, and special cases (identical experts, E = 1,
k = E, prefix invariance).
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit, softmax

from oracle import moe as om
from oracle.numerics import round_bf16


def _load_hand(golden_dir):
    with open(os.path.join(golden_dir, "moe_hand_case.json")) as f:
        case = json.load(f)
    layer = {k: np.array(case[k], dtype=np.float64)
             for k in ("gamma", "w_router", "w_gate", "w_up", "w_down")}
    return case, layer


def _rand_layer(rng, H, E, F, sigma=0.3, bias=False):
    layer = {
        "gamma": 1.0 + 0.1 * rng.standard_normal(H),
        "w_router": sigma * rng.standard_normal((E, H)),
        "w_gate": sigma * rng.standard_normal((E, F, H)),
        "w_up": sigma * rng.standard_normal((E, F, H)),
        "w_down": sigma * rng.standard_normal((E, H, F)),
    }
    if bias:
        layer["router_bias"] = rng.standard_normal(E)
    return layer


# ------------------------------------------------------------------ hand-worked case


def test_hand_case_every_stage(golden_dir):
    case, layer = _load_hand(golden_dir)
    x = np.array(case["x"])
    exp = case["expect"]
    r, out = om.moe_layer(x, layer, case["top_k"], case["eps"], act="f64")
    np.testing.assert_allclose(r.xn, exp["xn"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(r.logits, exp["logits"], rtol=0, atol=1e-15)
    np.testing.assert_array_equal(r.idx, exp["idx"])
    np.testing.assert_allclose(r.gates, exp["gates"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(om.topk_gap(r.logits, case["top_k"]), exp["gap"], atol=1e-15)
    np.testing.assert_array_equal(r.counts, exp["counts"])
    np.testing.assert_array_equal(r.offsets, exp["offsets"])
    np.testing.assert_array_equal(r.sorted_assign, exp["sorted_assign"])
    np.testing.assert_array_equal(r.pos, exp["pos"])
    np.testing.assert_allclose(out, exp["out"], rtol=0, atol=1e-15)
    dense = om.moe_dense_bruteforce(x, layer, case["top_k"], case["eps"], act="f64")
    np.testing.assert_allclose(dense, exp["out"], rtol=0, atol=1e-15)


# ------------------------------------------------------------------ RMSNorm


def test_rmsnorm_closed_forms():
    c = np.array([[2.0] * 8, [-0.5] * 8, [1e-3] * 8])
    eps = 1e-6
    xn = om.rmsnorm(c, np.ones(8), eps)
    want = c / np.sqrt(c * c + eps)
    np.testing.assert_allclose(xn, want, rtol=1e-15)
    # eps = 0: unit mean square, invariant to positive scaling, odd in x
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 64))
    xn0 = om.rmsnorm(x, np.ones(64), 0.0)
    np.testing.assert_allclose(np.mean(xn0 ** 2, axis=1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(om.rmsnorm(7.5 * x, np.ones(64), 0.0), xn0, rtol=1e-13)
    np.testing.assert_allclose(om.rmsnorm(-x, np.ones(64), 0.0), -xn0, rtol=1e-15)
    g = rng.standard_normal(64)
    np.testing.assert_allclose(om.rmsnorm(x, g, 0.0), xn0 * g, rtol=1e-13)
    # 3-4-5: mean square 12.5
    np.testing.assert_allclose(om.rmsnorm(np.array([[3.0, 4.0]]), np.ones(2), 0.0),
                               [[3 / math.sqrt(12.5), 4 / math.sqrt(12.5)]], rtol=1e-15)


# ------------------------------------------------------------------ router


def test_router_bruteforce_and_onehot():
    rng = np.random.default_rng(1)
    xn = rng.standard_normal((3, 5))
    W = rng.standard_normal((4, 5))
    b = rng.standard_normal(4)
    got = om.router_logits(xn, W, b)
    for t in range(3):
        for e in range(4):
            s = b[e]
            for h in range(5):
                s += xn[t, h] * W[e, h]
            assert abs(got[t, e] - s) < 1e-13
    onehot = np.eye(5)[[2]]
    np.testing.assert_array_equal(om.router_logits(onehot, W), W[:, 2][None, :])


# ------------------------------------------------------------------ top-k and gates


def test_topk_bruteforce_subsets():
    rng = np.random.default_rng(2)
    for trial in range(200):
        E = int(rng.integers(1, 9))
        k = int(rng.integers(1, E + 1))
        # small integer logits force many ties
        logits = rng.integers(-3, 4, size=(1, E)).astype(np.float64)
        idx = om.topk_experts(logits, k)[0]
        l = logits[0]
        # brute force over every k-subset: a valid top-k set has no chosen logit below
        # an unchosen one; among the valid sets the tie rule picks the lowest indices
        best = None
        for S in itertools.combinations(range(E), k):
            rest = [e for e in range(E) if e not in S]
            if rest and min(l[list(S)]) < max(l[rest]):
                continue
            key = sorted(S)
            if best is None or key < best:
                best = key
        assert sorted(idx.tolist()) == best
        # slot order: descending value, ascending index on ties; equals lexsort
        want_order = np.lexsort((np.arange(E), -l))[:k]
        np.testing.assert_array_equal(idx, want_order)


def test_gate_weights():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((50, 8)) * 3
    idx = om.topk_experts(logits, 3)
    g = om.gate_weights(logits, idx)
    np.testing.assert_allclose(g.sum(axis=1), 1.0, rtol=1e-15)
    assert np.all(np.diff(g, axis=1) <= 0)  # slot order is descending logit
    # k = E reduces to the full softmax (library routine), permuted to slot order
    idxE = om.topk_experts(logits, 8)
    gE = om.gate_weights(logits, idxE)
    np.testing.assert_allclose(gE, np.take_along_axis(softmax(logits, axis=1), idxE, 1), rtol=1e-13)
    # shift invariance and the two-expert closed form sigma(l0 - l1)
    np.testing.assert_allclose(om.gate_weights(logits + 100.0, idx), g, rtol=1e-12)
    two = om.gate_weights(np.array([[1.0, 0.0]]), np.array([[0, 1]]))
    np.testing.assert_allclose(two, [[expit(1.0), expit(-1.0)]], rtol=1e-15)
    # renormalised top-k of the full softmax equals the softmax of the selected logits
    p = softmax(logits, axis=1)
    sel = np.take_along_axis(p, idx, 1)
    np.testing.assert_allclose(sel / sel.sum(1, keepdims=True), g, rtol=1e-13)


# ------------------------------------------------------------------ counts, scan, permutation


def test_counts_scan_permutation_invariants():
    rng = np.random.default_rng(4)
    for T, E, k in [(1, 4, 2), (37, 8, 2), (200, 16, 6), (64, 128, 8), (5, 3, 3)]:
        logits = rng.standard_normal((T, E))
        idx = om.topk_experts(logits, k)
        for t in range(T):
            assert len(set(idx[t].tolist())) == k  # distinct experts per token
        counts = om.expert_counts(idx, E)
        assert counts.sum() == T * k
        np.testing.assert_array_equal(counts, np.bincount(idx.reshape(-1), minlength=E))
        offsets = om.exclusive_scan(counts)
        np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
        sa, pos = om.permutation(idx, E)
        # bijection on [0, T*k)
        np.testing.assert_array_equal(np.sort(sa), np.arange(T * k))
        # equals a stable argsort of the flat expert ids (library routine)
        np.testing.assert_array_equal(sa, np.argsort(idx.reshape(-1), kind="stable"))
        # pos is its inverse
        np.testing.assert_array_equal(sa[pos.reshape(-1)], np.arange(T * k))
        # each expert's segment holds exactly its pairs, tokens ascending
        for e in range(E):
            seg = sa[offsets[e]:offsets[e + 1]]
            assert np.all(idx.reshape(-1)[seg] == e)
            assert np.all(np.diff(seg // k) > 0)


def test_k_equals_E_and_bias_forcing():
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((9, 4))
    idx = om.topk_experts(logits, 4)
    np.testing.assert_array_equal(om.expert_counts(idx, 4), [9, 9, 9, 9])
    assert np.all(np.isinf(om.topk_gap(logits, 4)))
    # a large router bias puts expert 3 in every token's top-2 at slot 0
    xn = rng.standard_normal((9, 6))
    W = rng.standard_normal((4, 6))
    l = om.router_logits(xn, W, np.array([0.0, 0.0, 0.0, 1e3]))
    assert np.all(om.topk_experts(l, 2)[:, 0] == 3)


# ------------------------------------------------------------------ experts


def test_silu():
    assert om.silu(0.0) == 0.0
    assert abs(om.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    z = np.linspace(-20, 20, 401)
    np.testing.assert_allclose(om.silu(z), z * expit(z), rtol=1e-14, atol=1e-300)
    assert abs(om.silu(-50.0)) < 1e-19
    assert abs(om.silu(50.0) - 50.0) < 1e-15


def test_expert_ffn_bruteforce():
    rng = np.random.default_rng(6)
    H, F = 4, 3
    x = rng.standard_normal((2, H))
    wg, wu, wd = rng.standard_normal((F, H)), rng.standard_normal((F, H)), rng.standard_normal((H, F))
    got = om.expert_ffn(x, wg, wu, wd, act="f64")
    for t in range(2):
        h = []
        for f in range(F):
            g = sum(x[t, i] * wg[f, i] for i in range(H))
            u = sum(x[t, i] * wu[f, i] for i in range(H))
            h.append(g / (1 + math.exp(-g)) * u)
        for o in range(H):
            assert abs(got[t, o] - sum(h[f] * wd[o, f] for f in range(F))) < 1e-12


# ------------------------------------------------------------------ whole layer


@pytest.mark.parametrize("T,H,E,k,F,bias", [(7, 8, 4, 2, 6, False), (23, 16, 8, 3, 8, True),
                                             (40, 8, 16, 6, 4, True), (3, 4, 5, 5, 2, False)])
def test_sparse_equals_dense_bruteforce(T, H, E, k, F, bias):
    rng = np.random.default_rng(T * 100 + E)
    layer = _rand_layer(rng, H, E, F, bias=bias)
    x = rng.standard_normal((T, H))
    _, sparse = om.moe_layer(x, layer, k, 1e-6, act="f64")
    dense = om.moe_dense_bruteforce(x, layer, k, 1e-6, act="f64")
    np.testing.assert_allclose(sparse, dense, rtol=1e-12, atol=1e-14)
    # with bfloat16 storage the two may only differ by the final rounding of a sum
    # taken in another order: at most one bfloat16 spacing
    _, s16 = om.moe_layer(x, layer, k, 1e-6, act="bf16")
    d16 = om.moe_dense_bruteforce(x, layer, k, 1e-6, act="bf16")
    spacing = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(d16), 1e-30))) - 7)
    assert np.all(np.abs(s16 - d16) <= spacing + 1e-300)


def test_identical_experts_and_single_expert():
    rng = np.random.default_rng(7)
    H, E, F, T = 8, 6, 5, 11
    layer = _rand_layer(rng, H, E, F, bias=True)
    for name in ("w_gate", "w_up", "w_down"):
        layer[name][:] = layer[name][0]
    x = rng.standard_normal((T, H))
    _, out = om.moe_layer(x, layer, 3, 1e-6, act="f64")
    xq = om.rmsnorm(x, layer["gamma"], 1e-6)
    ffn = om.expert_ffn(xq, layer["w_gate"][0], layer["w_up"][0], layer["w_down"][0], act="f64")
    np.testing.assert_allclose(out, ffn, rtol=1e-12, atol=1e-14)  # gates sum to 1
    one = _rand_layer(rng, H, 1, F)
    r, out1 = om.moe_layer(x, one, 1, 1e-6, act="f64")
    np.testing.assert_array_equal(r.gates, 1.0)
    xq1 = om.rmsnorm(x, one["gamma"], 1e-6)
    np.testing.assert_allclose(out1, om.expert_ffn(xq1, one["w_gate"][0], one["w_up"][0],
                                                   one["w_down"][0], act="f64"), rtol=1e-13)


def test_prefix_invariance_and_token_subset():
    rng = np.random.default_rng(8)
    layer = _rand_layer(rng, 16, 8, 8, bias=True)
    x = rng.standard_normal((30, 16))
    _, full = om.moe_layer(x, layer, 2, 1e-6, act="bf16")
    _, pre = om.moe_layer(x[:13], layer, 2, 1e-6, act="bf16")
    np.testing.assert_array_equal(pre, full[:13])
    _, sub = om.moe_layer(x, layer, 2, 1e-6, act="bf16", tokens=[0, 7, 29])
    np.testing.assert_array_equal(sub[[0, 7, 29]], full[[0, 7, 29]])
    assert np.all(np.isnan(sub[1]))


def test_chain_feeds_rounded_output():
    rng = np.random.default_rng(9)
    layers = [_rand_layer(rng, 8, 4, 4) for _ in range(2)]
    x = rng.standard_normal((6, 8))
    routings, outs = om.moe_forward(x, layers, 2, 1e-6, act="bf16")
    _, second = om.moe_layer(outs[0], layers[1], 2, 1e-6, act="bf16")
    np.testing.assert_array_equal(outs[1], second)
    np.testing.assert_array_equal(round_bf16(outs[0]), outs[0])


def test_valid_sets_and_token_output():
    l = np.array([1.0, 0.5, 0.5 + 1e-7, -1.0])
    sets = om.valid_topk_sets(l, 2, 1e-5)
    assert sorted(sorted(s) for s in sets) == [[0, 1], [0, 2]]
    assert om.valid_topk_sets(l, 2, 0.0) == [frozenset({0, 2})]
    rng = np.random.default_rng(10)
    layer = _rand_layer(rng, 8, 4, 4)
    x = rng.standard_normal((5, 8))
    r, out = om.moe_layer(x, layer, 2, 1e-6, act="bf16")
    for t in range(5):
        got = om.token_output_for_set(x[t], layer, set(r.idx[t].tolist()), 1e-6, act="bf16")
        np.testing.assert_array_equal(got, out[t])
