"""Oracle for variable-context decode attention with split-KV partials merged once a
per-head counter reaches its target (test infrastructure only).

Why this workload.  The tutorial chapter "5 · Event Tensor et le dynamisme" lists the
context length of each request as a source of shape dynamism (§5.1, its table of
dynamism sources), and notes that when the number of producer tasks depends on such a
length, the counter targets must be computed at run time on the GPU before anyone waits
(§5.5 Obstacle 1).  The podcast episode page "Prompt Boundary-Aware Scheduling with
Event Tensors for Dynamic Kernels" (summary) uses split-K summation as its example of
waiting on true data dependencies.  Decode attention over a key/value cache of ragged
length is that pattern: the cache of request b is cut into ceil(L_b / C) chunks, each
chunk yields a partial result, and the head's output is formed once all of its chunks
have reported -- a count that depends on L_b.

Definition (reading: the pages give no formula; this is standard scaled dot-product
attention for one query token per request, grouped-query form):
  for request b with context length L_b, KV head g and query head h = g*G + i
  (G query heads share one KV head; G = 1 is plain multi-head attention):
      s_t = scale * q[b,h] . K[b,t,g]          t = 0 .. L_b - 1
      p   = softmax(s)                          over t
      out[b,h] = sum_t p_t V[b,t,g]
Layouts: q [B][H_kv*G][D]; the caches hold rows [rows][H_kv][D], request b's token t
at row kv_start[b] + t; out [B][H_kv*G][D].

Split form (reading: the partial of a chunk is the usual (max, sum, weighted sum)
triple, merged with the log-sum-exp identity; the chunks are [c*C, min(L_b, (c+1)*C))):
  partial of chunk c:  m_c = max_t s_t,  l_c = sum_t exp(s_t - m_c),
                       o_c = sum_t exp(s_t - m_c) V_t
  merge:               M = max_c m_c,  L = sum_c l_c exp(m_c - M),
                       out = sum_c o_c exp(m_c - M) / L
Everything is float64; q, K and V are taken exactly as given (bfloat16 values).
A request with L_b = 0 has no defined softmax; such requests are out of the domain.
"""

import numpy as np


def split_count(length, chunk):
    """Chunks of a context of `length` tokens: the target of its counter."""
    return -(-int(length) // int(chunk))


def chunk_bounds(length, chunk):
    """[(t_begin, t_end)] of every chunk; the last may be shorter, none is empty."""
    n = split_count(length, chunk)
    return [(c * chunk, min(length, (c + 1) * chunk)) for c in range(n)]


def head_scores(q_row, k_rows, scale):
    """s_t = scale * q . k_t for the rows of one request and KV head (float64)."""
    return scale * (np.asarray(k_rows, np.float64) @ np.asarray(q_row, np.float64))


def softmax(s):
    """p_t = exp(s_t - max s) / sum exp(s - max s)."""
    s = np.asarray(s, np.float64)
    e = np.exp(s - s.max())
    return e / e.sum()


def decode_attention(q, k_cache, v_cache, kv_start, lens, group, scale):
    """out[b, h] = softmax(scale * q[b,h] K_b^T) V_b for every request and query head,
    in float64 (the plain definition, no splitting)."""
    q = np.asarray(q, np.float64)
    B, HQ, D = q.shape
    out = np.zeros((B, HQ, D))
    for b in range(B):
        L = int(lens[b])
        rows = slice(int(kv_start[b]), int(kv_start[b]) + L)
        for h in range(HQ):
            g = h // group
            K = np.asarray(k_cache[rows, g, :], np.float64)
            V = np.asarray(v_cache[rows, g, :], np.float64)
            p = softmax(head_scores(q[b, h], K, scale))
            out[b, h] = p @ V
    return out


def chunk_partial(q_row, k_rows, v_rows, scale):
    """(m, l, o) of one chunk: its largest score, the sum of exp(s - m) and the
    exp(s - m)-weighted sum of its value rows."""
    s = head_scores(q_row, k_rows, scale)
    m = float(s.max())
    w = np.exp(s - m)
    return m, float(w.sum()), w @ np.asarray(v_rows, np.float64)


def merge_partials(partials):
    """Combine chunk partials [(m, l, o)] into the attention output of the head."""
    M = max(m for m, _, _ in partials)
    L = sum(l * np.exp(m - M) for m, l, _ in partials)
    O = sum(o * np.exp(m - M) for m, _, o in partials)
    return O / L


def decode_attention_split(q, k_cache, v_cache, kv_start, lens, group, scale, chunk):
    """The same output through chunk partials and their merge (the split form the
    kernel computes), float64.  Returns (out, n_split per request)."""
    q = np.asarray(q, np.float64)
    B, HQ, D = q.shape
    out = np.zeros((B, HQ, D))
    n_split = np.zeros(B, dtype=np.int64)
    for b in range(B):
        L = int(lens[b])
        base = int(kv_start[b])
        bounds = chunk_bounds(L, chunk)
        n_split[b] = len(bounds)
        for h in range(HQ):
            g = h // group
            parts = [chunk_partial(q[b, h], k_cache[base + t0:base + t1, g, :],
                                   v_cache[base + t0:base + t1, g, :], scale)
                     for t0, t1 in bounds]
            out[b, h] = merge_partials(parts)
    return out, n_split
