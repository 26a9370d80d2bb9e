"""Pins of the split-K oracle (CPU only): the hand-worked case, exact special cases
(one-hot rows, ones), split invariance against a brute-force triple loop, and the
slice bounds."""

import json
import os

import numpy as np
import pytest

from oracle import splitk as osk


def test_hand_case(golden_dir):
    with open(os.path.join(golden_dir, "splitk_hand_case.json")) as f:
        case = json.load(f)
    A, B = np.array(case["A"]), np.array(case["B"])
    parts = osk.splitk_partials(A, B, case["split_k"])
    np.testing.assert_array_equal(np.array(parts), case["expect"]["partials"])
    np.testing.assert_array_equal(osk.splitk_gemm(A, B, case["split_k"]), case["expect"]["C"])


def test_onehot_and_ones():
    rng = np.random.default_rng(0)
    K, N = 96, 7
    B = np.round(rng.standard_normal((K, N)) * 64) / 64
    A = np.zeros((3, K))
    A[0, 5] = 1.0
    A[1, 95] = 1.0
    A[2, 40] = 1.0
    C = osk.splitk_gemm(A, B, 8)
    np.testing.assert_array_equal(C, B[[5, 95, 40]])  # one-hot rows copy rows of B exactly
    Aw = rng.standard_normal((4, K))
    np.testing.assert_allclose(osk.splitk_gemm(Aw, np.ones((K, 3)), 8),
                               np.repeat(Aw.sum(1, keepdims=True), 3, 1), rtol=1e-13)


@pytest.mark.parametrize("M,N,K,S", [(2, 3, 8, 1), (3, 2, 16, 4), (2, 2, 13, 3), (1, 4, 9, 9)])
def test_split_invariance_bruteforce(M, N, K, S):
    rng = np.random.default_rng(M * N * K * S)
    A, B = rng.standard_normal((M, K)), rng.standard_normal((K, N))
    C = osk.splitk_gemm(A, B, S)
    for i in range(M):
        for j in range(N):
            assert abs(C[i, j] - sum(A[i, kk] * B[kk, j] for kk in range(K))) < 1e-12


def test_bounds():
    assert osk.split_bounds(14336, 8) == [(s * 1792, (s + 1) * 1792) for s in range(8)]
    assert osk.split_bounds(13, 3) == [(0, 5), (5, 10), (10, 13)]
    with pytest.raises(ValueError):
        osk.split_bounds(4, 3)  # ceil(4/3) = 2 leaves the third slice empty
