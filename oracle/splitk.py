"""Oracle for the split-K summation GEMM (test infrastructure only).

The podcast episode page "Prompt Boundary-Aware Scheduling with Event Tensors for
Dynamic Kernels" uses a split-K summation to illustrate waiting on true data
dependencies: the K range of C = A B is cut into S slices, each slice produces a
partial tile, and the tile's sum is formed once all S partials exist.  The sum is
taken in slice order s = 0..S-1.

reading: A is [M][K] and B is [K][N], both row-major; C is float32 (a bfloat16 result
alone would carry 2**-9 relative error); slice s covers columns
[s*ceil(K/S), min(K, (s+1)*ceil(K/S))) of A.
"""

import numpy as np


def split_bounds(K, split_k):
    """[(k_begin, k_end)] of each slice; the last may be shorter, none is empty."""
    step = -(-K // split_k)
    bounds = [(s * step, min(K, (s + 1) * step)) for s in range(split_k)]
    if any(b >= e for b, e in bounds):
        raise ValueError("split_k leaves an empty slice")
    return bounds


def splitk_partials(A, B, split_k):
    """The S partial tiles P_s = A[:, slice s] @ B[slice s, :] in float64."""
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    return [A[:, b:e] @ B[b:e, :] for b, e in split_bounds(A.shape[1], split_k)]


def splitk_gemm(A, B, split_k):
    """C = sum of the partial tiles in slice order (float64)."""
    parts = splitk_partials(A, B, split_k)
    C = np.zeros_like(parts[0])
    for p in parts:
        C = C + p
    return C
