"""Seeded synthetic KV-cache workloads.

This module only draws random numbers. It holds none of the quantization or
attention arithmetic, so both the GPU library's tests and the CPU oracle can be
fed from it without sharing any of the method's code.

The shapes of the draws follow what the KIVI explainer page ("ICML 2024論文解説:
KIVI — チューニング不要のKVキャッシュ2bit非対称量子化") says about the cache, in its
section on the KV-cache distribution (KVキャッシュの分布特性):

* Keys: a few channels carry large values across every token, so each channel
  gets its own spread. Here sigma[h, c] ~ LogNormal(0, 1) per (KV head,
  channel), shared by all batch rows and tokens, and 4 channels per KV head,
  picked by a seeded permutation, are multiplied by 8 (the outlier channels).
  K[b, h, t, c] = N(0, 1) * sigma[h, c].
* Values: large values sit on particular tokens, in particular the first tokens
  of the sequence (attention sinks). Here V[b, h, t, c] = N(0, 1), times 5 for
  absolute token positions 0..3.
* Queries: q ~ N(0, 1).

Everything is stored as fp16 (queries as fp16 or bf16).

Draw order, for a workload with seed S and layer L:
  1. generator seeded with S * 1_000_003 + L: sigma = exp(randn(Hkv, d)); then,
     for h = 0..Hkv-1, randperm(d)[:4] picks that head's outlier channels.
  2. token chunk [t0, t0 + n): generator seeded with
     hash(S, L, t0, 1): randn(B, Hkv, n, d) for K, then randn(B, Hkv, n, d) for V.
  3. query for decode step i: generator seeded with hash(S, L, i, 2):
     randn(B, Hq, d).
Chunks are drawn independently, so a prefill of T tokens followed by decode
tokens T, T+1, ... is reproducible from (S, L) and the positions alone.

Batches whose sequences differ in length (a serving batch) draw one length per
batch row, uniform over the integers [T_min, T_max], from a generator seeded
with hash(S, 3); row b then holds tokens [0, len[b]) of its chunk draws. A
paged cache's block table takes the pages in a random order: a permutation of
the pool drawn from a generator seeded with hash(S, 4).
"""

from __future__ import annotations

import torch

N_OUTLIER_CHANNELS = 4
OUTLIER_FACTOR = 8.0
SINK_TOKENS = 4
SINK_FACTOR = 5.0


def _mix(*parts: int) -> int:
    """Deterministic 63-bit seed from integers (splitmix64 finaliser)."""
    x = 0x9E3779B97F4A7C15
    for p in parts:
        x ^= (int(p) + 0x9E3779B97F4A7C15 + ((x << 6) & 0xFFFFFFFFFFFFFFFF) + (x >> 2)) & 0xFFFFFFFFFFFFFFFF
        z = x
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
        x = z ^ (z >> 31)
    return x & 0x7FFFFFFFFFFFFFFF


class KVWorkload:
    """Seeded K/V/q generator for one layer of a cache."""

    def __init__(self, batch: int, n_kv_heads: int, head_dim: int, seed: int,
                 layer: int = 0, device="cpu"):
        self.batch = batch
        self.n_kv_heads = n_kv_heads
        self.head_dim = head_dim
        self.seed = seed
        self.layer = layer
        self.device = torch.device(device)
        g = torch.Generator(device=self.device)
        g.manual_seed(seed * 1_000_003 + layer)
        sigma = torch.exp(torch.randn(n_kv_heads, head_dim, generator=g,
                                      device=self.device, dtype=torch.float32))
        for h in range(n_kv_heads):
            idx = torch.randperm(head_dim, generator=g, device=self.device)[:N_OUTLIER_CHANNELS]
            sigma[h, idx] *= OUTLIER_FACTOR
        self.sigma = sigma  # [Hkv, d] float32

    def kv(self, t0: int, ntok: int):
        """K, V for absolute token positions [t0, t0 + ntok): fp16 [B, Hkv, ntok, d]."""
        g = torch.Generator(device=self.device)
        g.manual_seed(_mix(self.seed, self.layer, t0, 1))
        shape = (self.batch, self.n_kv_heads, ntok, self.head_dim)
        k = torch.randn(shape, generator=g, device=self.device, dtype=torch.float32)
        v = torch.randn(shape, generator=g, device=self.device, dtype=torch.float32)
        k.mul_(self.sigma[None, :, None, :])
        n_sink = max(0, min(SINK_TOKENS - t0, ntok))
        if n_sink > 0:
            v[:, :, :n_sink, :] *= SINK_FACTOR
        return k.to(torch.float16).contiguous(), v.to(torch.float16).contiguous()

    def q(self, n_q_heads: int, step: int = 0, dtype=torch.float16):
        """Decode query for step `step`: [B, Hq, d] in fp16 or bf16."""
        g = torch.Generator(device=self.device)
        g.manual_seed(_mix(self.seed, self.layer, step, 2))
        q = torch.randn((self.batch, n_q_heads, self.head_dim), generator=g,
                        device=self.device, dtype=torch.float32)
        return q.to(dtype).contiguous()


def query_history(workload: "KVWorkload", n_q_heads: int, n: int, rank: int = 8, noise: float = 0.1,
                  dtype=torch.float16):
    """Past queries [B, Hq, n, d] for the SQuat-style key coder, drawn with a
    low-rank structure (the SQuat page describes the future queries as
    concentrated in a subspace of past ones): the query heads that share KV
    head h draw q = A_h z + noise, with A_h [d, rank] fixed per KV head
    (columns scaled 3 .. 1), z ~ N(0, 1) per query, noise ~ N(0, noise^2) per
    element. Generator seeded with hash(S, L, 5)."""
    B, Hkv, d = workload.batch, workload.n_kv_heads, workload.head_dim
    g = torch.Generator(device=workload.device)
    g.manual_seed(_mix(workload.seed, workload.layer, 5))
    a = torch.randn(Hkv, d, rank, generator=g, device=workload.device)
    a = a * torch.linspace(3.0, 1.0, rank, device=workload.device)
    z = torch.randn(B, n_q_heads, rank, n, generator=g, device=workload.device)
    head_of = torch.arange(n_q_heads, device=workload.device) // (n_q_heads // Hkv)
    q = torch.einsum("hdr,bhrn->bhnd", a[head_of], z)
    q = q + noise * torch.randn(B, n_q_heads, n, d, generator=g, device=workload.device)
    return q.to(dtype).contiguous()


def row_lengths(batch: int, t_min: int, t_max: int, seed: int) -> list:
    """Seeded per-row sequence lengths, uniform over [t_min, t_max]."""
    g = torch.Generator()
    g.manual_seed(_mix(seed, 3))
    return [int(x) for x in torch.randint(t_min, t_max + 1, (batch,), generator=g)]


def page_order(n_pages: int, seed: int) -> torch.Tensor:
    """Seeded random permutation of page indices [0, n_pages), int32."""
    g = torch.Generator()
    g.manual_seed(_mix(seed, 4))
    return torch.randperm(n_pages, generator=g).to(torch.int32)


# The workloads the method is measured on. `T` is the number of tokens
# appended before the decode attention; "prefill" means append(T) then flush.
CONFIGS = {
    "tiny": dict(batch=1, n_kv_heads=1, n_q_heads=1, head_dim=128, T=1024, bits=2, seed=1),
    "llama2_7b_layer": dict(batch=8, n_kv_heads=32, n_q_heads=32, head_dim=128, T=4096, bits=2, seed=2),
    "long_context": dict(batch=1, n_kv_heads=32, n_q_heads=32, head_dim=128, T=131072, bits=2, seed=3),
    "gqa_streaming": dict(batch=64, n_kv_heads=8, n_q_heads=32, head_dim=128, T=8192, bits=2, seed=4,
                          decode_steps=256),
    "full_stack": dict(batch=128, n_kv_heads=8, n_q_heads=32, head_dim=128, T=4096, seed=5,
                       layers=32, layer_bits=[2] * 16 + [4] * 16, q_dtype="bf16"),
    # The Llama-2-7B-shaped layer with the SQuat-style key coder: a rank-8 query
    # subspace from 512 past queries per head, lambda 0.1.
    "llama2_7b_layer_squat": dict(batch=8, n_kv_heads=32, n_q_heads=32, head_dim=128, T=4096, bits=2, seed=2,
                                  squat_rank=8, squat_lambda=0.1, squat_queries=512),
    # A serving batch: the GQA shape above with each sequence at its own length,
    # uniform over [512, 8192] tokens (T is the longest possible).
    "gqa_ragged": dict(batch=64, n_kv_heads=8, n_q_heads=32, head_dim=128, T=8192, bits=2, seed=6,
                       ragged=(512, 8192)),
    # The same serving batch with paged blocks: every row's blocks on pages of a
    # shared pool, taken in a random order.
    "gqa_paged": dict(batch=64, n_kv_heads=8, n_q_heads=32, head_dim=128, T=8192, bits=2, seed=6,
                      ragged=(512, 8192), paged=True),
    # A serving batch of 256 sequences with the same length mix, paged: more
    # rows than one launch's row table holds (128), so each call runs two
    # launches.
    "gqa_paged_256": dict(batch=256, n_kv_heads=8, n_q_heads=32, head_dim=128, T=8192, bits=2, seed=7,
                          ragged=(512, 8192), paged=True),
}
