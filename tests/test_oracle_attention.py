"""Pins of the decode-attention oracle (oracle/attention.py) against what the
mathematics fixes: a case worked by hand, closed forms, a library softmax, brute-force
loops, the invariance of the output under any split of the context, and the
query-head to KV-head mapping.  CPU only."""

import json
import os

import numpy as np
import pytest
import scipy.special

from oracle import attention as oa

HERE = os.path.dirname(os.path.abspath(__file__))


def _rand_case(rng, B=3, HKV=2, G=2, D=8, lens=(5, 1, 12), spread=1.0):
    lens = np.asarray(lens)
    start = np.concatenate([[0], np.cumsum(lens)[:-1]])
    rows = int(lens.sum())
    q = rng.standard_normal((B, HKV * G, D))
    k = rng.standard_normal((rows, HKV, D)) * spread
    v = rng.standard_normal((rows, HKV, D))
    return q, k, v, start, lens


def test_hand_case():
    with open(os.path.join(HERE, "golden", "attn_hand_case.json")) as f:
        h = json.load(f)
    q, k, v = np.array(h["q"]), np.array(h["k"]), np.array(h["v"])
    out = oa.decode_attention(q, k, v, h["kv_start"], h["lens"], h["group"], h["scale"])
    assert np.allclose(out, h["out"], rtol=0, atol=1e-12)
    parts = [oa.chunk_partial(q[0, 0], k[t0:t1, 0], v[t0:t1, 0], h["scale"])
             for t0, t1 in oa.chunk_bounds(3, h["chunk"])]
    for (m, l, o), (mw, lw, ow) in zip(parts, h["partials"]):
        assert abs(m - mw) < 1e-12 and abs(l - lw) < 1e-12 and np.allclose(o, ow, atol=1e-12)
    assert np.allclose(oa.merge_partials(parts), h["out"][0][0], atol=1e-12)
    split, n = oa.decode_attention_split(q, k, v, h["kv_start"], h["lens"], 1, h["scale"], h["chunk"])
    assert list(n) == [2] and np.allclose(split, h["out"], atol=1e-12)


def test_one_token_returns_its_value_row():
    rng = np.random.default_rng(1)
    q, k, v, start, lens = _rand_case(rng, lens=(1, 1, 1))
    out = oa.decode_attention(q, k, v, start, lens, 2, 0.3)
    for b in range(3):
        for h in range(4):
            assert np.array_equal(out[b, h], v[start[b], h // 2])


def test_equal_keys_average_the_values():
    rng = np.random.default_rng(2)
    q, k, v, start, lens = _rand_case(rng, lens=(6, 3, 9))
    k[:] = k[0:1]  # every key the same: uniform weights
    out = oa.decode_attention(q, k, v, start, lens, 2, 0.7)
    for b in range(3):
        rows = slice(start[b], start[b] + lens[b])
        for h in range(4):
            assert np.allclose(out[b, h], v[rows, h // 2].mean(axis=0), atol=1e-12)


def test_softmax_matches_scipy():
    rng = np.random.default_rng(3)
    for n in (1, 2, 17, 300):
        s = rng.standard_normal(n) * 10
        assert np.allclose(oa.softmax(s), scipy.special.softmax(s), rtol=1e-13, atol=0)


def test_against_brute_force_loops():
    rng = np.random.default_rng(4)
    q, k, v, start, lens = _rand_case(rng, B=2, HKV=2, G=3, D=4, lens=(4, 7))
    scale = 0.37
    out = oa.decode_attention(q, k, v, start, lens, 3, scale)
    for b in range(2):
        for h in range(6):
            g = h // 3
            s = []
            for t in range(lens[b]):
                acc = 0.0
                for d in range(4):
                    acc += q[b, h, d] * k[start[b] + t, g, d]
                s.append(scale * acc)
            w = [np.exp(x - max(s)) for x in s]
            z = sum(w)
            for d in range(4):
                ref = sum(w[t] * v[start[b] + t, g, d] for t in range(lens[b])) / z
                assert abs(out[b, h, d] - ref) < 1e-12


@pytest.mark.parametrize("chunk", [1, 2, 3, 5, 12, 64])
def test_any_split_merges_to_the_unsplit_output(chunk):
    rng = np.random.default_rng(5)
    q, k, v, start, lens = _rand_case(rng, lens=(5, 1, 12), spread=4.0)
    ref = oa.decode_attention(q, k, v, start, lens, 2, 0.5)
    out, n = oa.decode_attention_split(q, k, v, start, lens, 2, 0.5, chunk)
    assert list(n) == [oa.split_count(L, chunk) for L in lens]
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_query_heads_share_their_own_kv_head():
    """Query head h reads KV head h // G: with one KV head's values all +1 and the
    other's all -1, heads 0..G-1 give +1 and G..2G-1 give -1 (a transposed mapping,
    h % H_kv, would mix them)."""
    rng = np.random.default_rng(6)
    q, k, v, start, lens = _rand_case(rng, B=1, HKV=2, G=3, D=4, lens=(7,))
    v[:, 0, :] = 1.0
    v[:, 1, :] = -1.0
    out = oa.decode_attention(q, k, v, start, lens, 3, 1.0)
    assert np.allclose(out[0, :3], 1.0) and np.allclose(out[0, 3:], -1.0)


def test_token_order_does_not_matter():
    rng = np.random.default_rng(7)
    q, k, v, start, lens = _rand_case(rng, B=1, lens=(11,))
    perm = rng.permutation(11)
    a = oa.decode_attention(q, k, v, start, lens, 2, 0.4)
    b = oa.decode_attention(q, k[perm], v[perm], start, lens, 2, 0.4)
    assert np.allclose(a, b, atol=1e-12)


def test_chunk_bounds_cover_the_context():
    for L in (1, 2, 255, 256, 257, 1000):
        for C in (1, 64, 256):
            b = oa.chunk_bounds(L, C)
            assert len(b) == oa.split_count(L, C) == -(-L // C)
            assert b[0][0] == 0 and b[-1][1] == L
            assert all(e > s for s, e in b) and all(b[i][1] == b[i + 1][0] for i in range(len(b) - 1))
