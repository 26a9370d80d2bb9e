"""Seeded synthetic inputs for the MoE layer and the split-K GEMM.

This is the only module that both the HIP path's callers and the CPU oracle's tests
use.  It draws random numbers and rounds them to the storage type; it contains none
of the layer's arithmetic.  Everything is drawn on the host with a seeded
``torch.Generator`` (fast, deterministic) and returned as CPU tensors in the storage
dtype; ``as_numpy`` gives the exact float values for the oracle.

Workloads (the pages name no dataset; these synthetic draws stand in for real
activations and trained weights):

  tiny        T=16, H=128, E=4, k=2, F=256, float32, x~N(0,1), weights ~N(0,0.05)
  decode      H=4096, E=8, k=2, F=14336, bfloat16, weights ~N(0,0.02), x~N(0,1),
              T per call drawn from {1, 4, 16, 64}
  finegrained H=2048, E=128, k=8, F=768, T=256, bfloat16, router logits offset by
              the log of a Zipf(s=1.1) popularity per expert (expert 0 most popular)
  prefill     T=4096, H=4096, E=64, k=6, F=1408, bfloat16, two layers chained
  splitk      C[64x4096] = A[64x14336] B[14336x4096], bfloat16 ~N(0,0.02), split 8

RMSNorm gamma is 1 and eps is 1e-6 everywhere.
"""

from dataclasses import dataclass, replace
import math

import numpy as np
import torch


@dataclass(frozen=True)
class MoEConfig:
    name: str
    tokens: tuple  # token counts the workload uses
    hidden: int
    experts: int
    top_k: int
    ffn: int
    layers: int = 1
    dtype: str = "bf16"  # storage type of x, weights and activations: "bf16" | "f32"
    sigma_router: float = 0.02
    sigma_expert: float = 0.02
    zipf_s: float = 0.0  # > 0: router bias b_e = -zipf_s * ln(e + 1)
    eps: float = 1e-6
    seed: int = 0

    def with_(self, **kw):
        return replace(self, **kw)


CONFIGS = {
    "tiny": MoEConfig("tiny", (16,), 128, 4, 2, 256, dtype="f32",
                      sigma_router=0.05, sigma_expert=0.05),
    "decode": MoEConfig("decode", (1, 4, 16, 64), 4096, 8, 2, 14336),
    "finegrained": MoEConfig("finegrained", (256,), 2048, 128, 8, 768, zipf_s=1.1),
    "prefill": MoEConfig("prefill", (4096,), 4096, 64, 6, 1408, layers=2),
}

SPLITK = dict(M=64, N=4096, K=14336, split_k=8, sigma=0.02, seed=0)


def torch_dtype(name):
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def _normal(gen, shape, sigma, dtype):
    t = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if sigma != 1.0:
        t.mul_(sigma)
    return t.to(dtype)


def make_layers(cfg, seed=None):
    """Weights of every layer: list of dicts of CPU tensors.

    Draw order per layer: router weight, then per expert gate, up, down.
    gamma and router_bias are float32; the rest use the config's storage type.
    """
    seed = cfg.seed if seed is None else seed
    gen = torch.Generator().manual_seed(1_000_003 * seed + 17)
    dt = torch_dtype(cfg.dtype)
    H, E, F = cfg.hidden, cfg.experts, cfg.ffn
    layers = []
    for _ in range(cfg.layers):
        layer = {"gamma": torch.ones(H, dtype=torch.float32),
                 "w_router": _normal(gen, (E, H), cfg.sigma_router, dt)}
        if cfg.zipf_s > 0:
            layer["router_bias"] = torch.tensor(
                [-cfg.zipf_s * math.log(e + 1) for e in range(E)], dtype=torch.float32)
        wg = torch.empty(E, F, H, dtype=dt)
        wu = torch.empty(E, F, H, dtype=dt)
        wd = torch.empty(E, H, F, dtype=dt)
        for e in range(E):
            wg[e] = _normal(gen, (F, H), cfg.sigma_expert, dt)
            wu[e] = _normal(gen, (F, H), cfg.sigma_expert, dt)
            wd[e] = _normal(gen, (H, F), cfg.sigma_expert, dt)
        layer.update(w_gate=wg, w_up=wu, w_down=wd)
        layers.append(layer)
    return layers


def make_x(cfg, T, seed=None, call=0):
    """Layer input x [T][H] ~ N(0, 1) in the storage type."""
    seed = cfg.seed if seed is None else seed
    gen = torch.Generator().manual_seed(2_000_029 * seed + 7919 * call + T)
    return _normal(gen, (T, cfg.hidden), 1.0, torch_dtype(cfg.dtype))


def decode_sequence(n=32, seed=0, choices=(1, 4, 16, 64)):
    """Token counts of a decode run: n draws from ``choices``, each at least once."""
    rng = np.random.default_rng(seed)
    seq = list(rng.choice(choices, size=n))
    for i, c in enumerate(choices):  # force every size to appear
        if c not in seq:
            seq[i] = c
    return [int(v) for v in seq]


def make_splitk(M=None, N=None, K=None, sigma=None, seed=None):
    """A [M][K] and B [K][N], bfloat16 ~ N(0, sigma)."""
    M = SPLITK["M"] if M is None else M
    N = SPLITK["N"] if N is None else N
    K = SPLITK["K"] if K is None else K
    sigma = SPLITK["sigma"] if sigma is None else sigma
    seed = SPLITK["seed"] if seed is None else seed
    gen = torch.Generator().manual_seed(3_000_017 * seed + 5)
    A = _normal(gen, (M, K), sigma, torch.bfloat16)
    B = _normal(gen, (K, N), sigma, torch.bfloat16)
    return A, B


def as_numpy(t):
    """Exact values of a tensor as a float32 array (bfloat16 and float32 values are all
    exact in float32; the oracle widens to float64 where it computes)."""
    if t is None:
        return None
    return t.detach().to("cpu", torch.float32).numpy()


def layers_as_numpy(layers):
    return [{k: as_numpy(v) for k, v in layer.items()} for layer in layers]


# ------------------------------------------------------------------ decode attention

# The decode-attention workload: a batch of 32 requests, 32 query heads sharing 8 KV
# heads (4 per KV head), head dimension 128, bfloat16 caches; context lengths per request
# drawn log-uniformly from [64, 32768] (the pages name no model or trace; the mix of
# short and long contexts stands in for a serving batch).  q, K and V ~ N(0, 1).
ATTN = dict(batch=32, kv_heads=8, group=4, head_dim=128, min_len=64, max_len=32768, seed=0)


def draw_context_lens(batch, lo, hi, seed=0):
    """Per-request context lengths, log-uniform in [lo, hi] (int32 CPU tensor)."""
    gen = torch.Generator().manual_seed(7_919 * seed + 29)
    u = torch.rand(batch, generator=gen, dtype=torch.float64)
    lens = torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo))).round().to(torch.int64)
    return lens.clamp(lo, hi).to(torch.int32)


def make_attention(lens, kv_heads, group, head_dim=128, seed=0):
    """(q, k_cache, v_cache, kv_start) for requests of the given context lengths: the
    caches hold the requests' rows one after another (kv_start = exclusive scan of the
    lengths), head-major [kv_heads][rows][head_dim]; q is [B][kv_heads*group][head_dim];
    all bfloat16 CPU tensors ~N(0, 1) (kv_start int32)."""
    lens = torch.as_tensor(lens, dtype=torch.int64)
    B = lens.numel()
    rows = int(lens.sum())
    gen = torch.Generator().manual_seed(104_729 * seed + 31)
    q = _normal(gen, (B, kv_heads * group, head_dim), 1.0, torch.bfloat16)
    k = _normal(gen, (kv_heads, rows, head_dim), 1.0, torch.bfloat16)
    v = _normal(gen, (kv_heads, rows, head_dim), 1.0, torch.bfloat16)
    start = torch.cumsum(lens, 0) - lens
    return q, k, v, start.to(torch.int32)
