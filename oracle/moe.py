"""Oracle for one Mixture-of-Experts layer and a chain of them (test infrastructure).

The layer, in the order its stages run:

  1. RMSNorm          xn[t] = x[t] / sqrt(mean_h x[t,h]^2 + eps) * gamma
  2. router           logits[t,e] = sum_h xn[t,h] * W_r[e,h] (+ b[e])
  3. top-k            S_t = the k experts with the largest logits
  4. softmax          gates over the k selected logits (they sum to 1)
  5. counts           c_e = number of (token, slot) pairs routed to expert e
  6. exclusive scan   o_e = c_0 + ... + c_{e-1}
  7. permutation      the (token, slot) pairs grouped by expert, tokens ascending
  8. gate/up          G = X_e W_g[e]^T, U = X_e W_u[e]^T for the rows X_e of expert e
  9. SwiGLU           h = silu(G) * U, silu(z) = z / (1 + exp(-z))
 10. down             Y_e = h W_d[e]^T
 11. combine          out[t] = sum_j g[t,j] * Y[pos[t,j]]

Steps 5-7 are what the podcast episode page "Prompt Boundary-Aware Scheduling with
Event Tensors for Dynamic Kernels" describes as MoE dependencies known only at run
time: the per-expert counts are the data-dependent targets of the event counters that
release expert work (chapter "5 · Event Tensor et le dynamisme", §5.5 Obstacle 1:
targets are computed on the GPU from the routing before anyone waits on them).
The pages do not define the arithmetic of any stage; every reading taken here is
marked "reading:" and listed with the others in the design notes.

Precision: everything is float64.  Activations are rounded to the storage type at
three points only -- the expert input X (= rounded xn), the SwiGLU output h, and the
layer output -- by ``oracle.numerics.rounder(act)``.  The router works on the
*unrounded* normalised input (reading: the router is an fp32-accumulate GEMV on fp32
activations, so routing decisions do not depend on the bfloat16 rounding of xn).
"""

from dataclasses import dataclass

import numpy as np

from .numerics import rounder


# --------------------------------------------------------------------------- routing


def rmsnorm(x, gamma, eps):
    """RMSNorm of every row of ``x``: x * gamma / sqrt(mean(x^2) + eps).

    reading: gamma multiplies after normalisation (the usual RMSNorm form); no bias.
    """
    x = np.asarray(x, dtype=np.float64)
    mean_sq = np.mean(x * x, axis=1, keepdims=True)
    return x / np.sqrt(mean_sq + eps) * np.asarray(gamma, dtype=np.float64)[None, :]


def router_logits(xn, w_router, bias=None):
    """logits[t, e] = sum_h xn[t, h] * w_router[e, h] (+ bias[e]).

    reading: the router weight is stored [experts][hidden] (nn.Linear layout).
    """
    logits = np.asarray(xn, np.float64) @ np.asarray(w_router, np.float64).T
    if bias is not None:
        logits = logits + np.asarray(bias, np.float64)[None, :]
    return logits


def topk_experts(logits, k):
    """The k experts of each token in slot order: larger logit first, and on equal
    logits the lower expert index first.

    reading: ties break towards the lower expert index; slot j holds the j-th largest.
    """
    logits = np.asarray(logits, np.float64)
    T, E = logits.shape
    idx = np.empty((T, k), dtype=np.int64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-logits[t, e], e))
        idx[t] = order[:k]
    return idx


def gate_weights(logits, idx):
    """Softmax over each token's k selected logits, in slot order.

    Softmax over all E logits followed by renormalising the k selected probabilities
    gives the same numbers (the common factor cancels); the gates sum to 1.
    """
    sel = np.take_along_axis(np.asarray(logits, np.float64), idx, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def expert_counts(idx, num_experts):
    """c_e = number of (token, slot) pairs routed to expert e."""
    counts = np.zeros(num_experts, dtype=np.int64)
    for e in np.asarray(idx).reshape(-1):
        counts[e] += 1
    return counts


def exclusive_scan(counts):
    """offsets[e] = counts[0] + ... + counts[e-1]; offsets[E] = total."""
    offsets = np.zeros(len(counts) + 1, dtype=np.int64)
    running = 0
    for e, c in enumerate(counts):
        offsets[e] = running
        running += int(c)
    offsets[len(counts)] = running
    return offsets


def permutation(idx, num_experts):
    """Group the (token, slot) pairs by expert.

    Returns ``sorted_assign`` (length T*k) where entry ``offsets[e] + r`` holds
    ``t*k + j`` for the r-th pair routed to expert e, and ``pos`` [T][k] with
    ``sorted_assign[pos[t, j]] == t*k + j``.

    reading: within one expert the pairs are ordered by token index (stable), so the
    permutation is deterministic.  A token never picks one expert twice, so the slot
    index never decides the order.
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    buckets = [[] for _ in range(num_experts)]
    for t in range(T):
        for j in range(k):
            buckets[int(idx[t, j])].append(t * k + j)
    sorted_assign = np.array([a for b in buckets for a in b], dtype=np.int64)
    pos = np.empty((T, k), dtype=np.int64)
    for p, a in enumerate(sorted_assign):
        pos[a // k, a % k] = p
    return sorted_assign, pos


@dataclass
class Routing:
    xn: np.ndarray  # [T][H] float64, unrounded normalised input
    logits: np.ndarray  # [T][E]
    idx: np.ndarray  # [T][k] experts in slot order
    gates: np.ndarray  # [T][k]
    counts: np.ndarray  # [E]
    offsets: np.ndarray  # [E+1]
    sorted_assign: np.ndarray  # [T*k]
    pos: np.ndarray  # [T][k]


def route(x, layer, top_k, eps):
    """Steps 1-7 for every token of ``x`` (layer = dict of weights, see ``moe_layer``)."""
    xn = rmsnorm(x, layer["gamma"], eps)
    logits = router_logits(xn, layer["w_router"], layer.get("router_bias"))
    idx = topk_experts(logits, top_k)
    gates = gate_weights(logits, idx)
    E = logits.shape[1]
    counts = expert_counts(idx, E)
    offsets = exclusive_scan(counts)
    sorted_assign, pos = permutation(idx, E)
    return Routing(xn, logits, idx, gates, counts, offsets, sorted_assign, pos)


def topk_gap(logits, k):
    """l_(k) - l_(k+1) per token: how far the k-th selected logit is above the best
    unselected one (infinity when k equals the number of experts)."""
    s = -np.sort(-np.asarray(logits, np.float64), axis=1)
    if k >= s.shape[1]:
        return np.full(s.shape[0], np.inf)
    return s[:, k - 1] - s[:, k]


# --------------------------------------------------------------------------- experts


def silu(z):
    """silu(z) = z / (1 + exp(-z)), the SwiGLU gate activation."""
    z = np.asarray(z, np.float64)
    return z / (1.0 + np.exp(-z))


def expert_ffn(xq, w_gate, w_up, w_down, act="bf16"):
    """One SwiGLU expert on rows ``xq`` (already in storage precision).

    G = xq W_g^T, U = xq W_u^T, h = silu(G) * U rounded to storage precision, y = h W_d^T.
    reading: weights use the nn.Linear [out][in] layout, gate and up are separate
    matrices [F][H], down is [H][F]; h is rounded to the activation type before the
    down projection (it is stored between the two GEMMs).
    """
    rnd = rounder(act)
    xq = np.asarray(xq, np.float64)
    g = xq @ np.asarray(w_gate, np.float64).T
    u = xq @ np.asarray(w_up, np.float64).T
    h = rnd(silu(g) * u)
    return h @ np.asarray(w_down, np.float64).T


def moe_layer(x, layer, top_k, eps, act="bf16", tokens=None):
    """One MoE layer (steps 1-11).  ``layer`` holds float arrays:
    gamma[H], w_router[E][H], optional router_bias[E], w_gate[E][F][H], w_up[E][F][H],
    w_down[E][H][F].

    ``tokens``: optional sorted list of token indices whose outputs are wanted; routing
    is always computed for every token (the counts and permutation are global), the
    experts only for the rows of the wanted tokens.  Returns (Routing, out) where out
    is [T][H] float64 with NaN in rows that were not computed.

    reading: no residual connection and no shared expert; the layer output is the
    combine result rounded to the activation type.
    """
    rnd = rounder(act)
    r = route(x, layer, top_k, eps)
    T, H = r.xn.shape
    xq = rnd(r.xn)  # expert input in storage precision
    want = np.ones(T, dtype=bool) if tokens is None else np.isin(np.arange(T), tokens)
    Y = np.full((T * top_k, H), np.nan)
    E = len(r.counts)
    for e in range(E):
        rows = np.arange(r.offsets[e], r.offsets[e + 1])
        toks = r.sorted_assign[rows] // top_k
        keep = want[toks]
        rows, toks = rows[keep], toks[keep]
        if len(rows) == 0:
            continue
        Y[rows] = expert_ffn(xq[toks], layer["w_gate"][e], layer["w_up"][e],
                             layer["w_down"][e], act)
    out = np.full((T, H), np.nan)
    for t in np.nonzero(want)[0]:
        acc = np.zeros(H)
        for j in range(top_k):  # slot order
            acc = acc + r.gates[t, j] * Y[r.pos[t, j]]
        out[t] = acc
    return r, rnd(out)


def moe_dense_bruteforce(x, layer, top_k, eps, act="bf16"):
    """The same layer evaluated densely: every expert on every token, masked by the
    routing.  out[t] = sum_e mask[t,e] * gate[t,e] * FFN_e(xq[t]).

    Shares only steps 1-4 with ``moe_layer`` (no counts, scan, permutation, gather or
    scatter), so agreement pins the sparse machinery.
    """
    rnd = rounder(act)
    xn = rmsnorm(x, layer["gamma"], eps)
    logits = router_logits(xn, layer["w_router"], layer.get("router_bias"))
    idx = topk_experts(logits, top_k)
    gates = gate_weights(logits, idx)
    T, E = logits.shape
    dense_gate = np.zeros((T, E))
    for t in range(T):
        for j in range(top_k):
            dense_gate[t, idx[t, j]] = gates[t, j]
    xq = rnd(xn)
    out = np.zeros((T, xq.shape[1]))
    for e in range(E):
        y = expert_ffn(xq, layer["w_gate"][e], layer["w_up"][e], layer["w_down"][e], act)
        out += dense_gate[:, e:e + 1] * y
    return rnd(out)


def moe_forward(x, layers, top_k, eps, act="bf16", tokens=None):
    """A chain of MoE layers: the (rounded) output of layer l is the input of layer
    l+1, which applies its own RMSNorm first.  reading: nothing else sits between the
    layers (no residual, no shared expert).

    With ``tokens`` given, every layer computes routing for all tokens only in the
    first layer; later layers need every token's input to route globally, so a
    subset is supported only for a single layer.  Returns (list of Routing, list of
    layer outputs).
    """
    if tokens is not None and len(layers) > 1:
        raise ValueError("a token subset needs the full previous layer output")
    routings, outs = [], []
    h = np.asarray(x, np.float64)
    for layer in layers:
        r, h = moe_layer(h, layer, top_k, eps, act, tokens)
        routings.append(r)
        outs.append(h)
    return routings, outs


# ------------------------------------------------------------- near-tie alternatives


def valid_topk_sets(logits_row, k, delta):
    """Every expert set a correct top-k may return for one token when logits closer
    than ``delta`` to the k-th value count as ties.  Experts clearly above the
    boundary are always in; the rest are filled from the ones within ``delta`` of it.
    """
    from itertools import combinations

    l = np.asarray(logits_row, np.float64)
    kth = np.sort(l)[::-1][k - 1]
    sure = [e for e in range(len(l)) if l[e] > kth + delta]
    near = [e for e in range(len(l)) if abs(l[e] - kth) <= delta]
    need = k - len(sure)
    return [frozenset(sure) | frozenset(c) for c in combinations(near, need)]


def token_output_for_set(x_row, layer, expert_set, eps, act="bf16"):
    """Layer output of one token for a given expert set (gates = softmax over that
    set's logits), in the same precision as ``moe_layer``."""
    rnd = rounder(act)
    x_row = np.asarray(x_row, np.float64)[None, :]
    xn = rmsnorm(x_row, layer["gamma"], eps)
    logits = router_logits(xn, layer["w_router"], layer.get("router_bias"))[0]
    experts = sorted(expert_set, key=lambda e: (-logits[e], e))
    sel = np.array([logits[e] for e in experts])
    g = np.exp(sel - sel.max())
    g = g / g.sum()
    xq = rnd(xn)
    acc = np.zeros(x_row.shape[1])
    for gj, e in zip(g, experts):
        acc = acc + gj * expert_ffn(xq, layer["w_gate"][e], layer["w_up"][e],
                                    layer["w_down"][e], act)[0]
    return rnd(acc)
