"""Seeded synthetic inputs and the workload shapes, shared by the tests, the bench and the
oracle's callers.

This module holds no arithmetic of the attention method: it only draws normal numbers, rounds
them to bf16 (round to nearest even) and names the workloads. It imports nothing else from
this package, so the oracle side and the GPU side can both use it without sharing code.

Host draws: numpy ``Generator(PCG64(SeedSequence([seed, tensor_id])))``, ``standard_normal``
in float32, then (for bf16 workloads) rounded to bf16 and returned as float32 arrays holding
exactly bf16-representable values. Device draws (for sizes the host cannot generate quickly)
use a seeded ``torch.Generator`` on the GPU; tests copy what they need back to the host so the
oracle sees the same bits.

Tensor ids: q = 0, k = 1, v = 2, g = 3, state = 4, k_cache = 5, v_cache = 6 (plus 10 * layer
for stacked layers).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

TID_Q, TID_K, TID_V, TID_G, TID_STATE, TID_KCACHE, TID_VCACHE = 0, 1, 2, 3, 4, 5, 6


def bf16_round(x):
    """Round float32 values to the nearest bf16 (ties to even); returns float32 holding the
    rounded values. NaN/Inf are not expected in these inputs."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).reshape(a.shape)


def host_normal(seed, tensor_id, shape, dtype="bf16", std=1.0):
    """Seeded N(0, std^2) draw on the host; bf16 workloads get bf16-rounded values."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(tensor_id)])))
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x = (x * np.float32(std)).astype(np.float32)
    return bf16_round(x) if dtype == "bf16" else x


def device_normal(seed, tensor_id, shape, dtype="bf16", std=1.0, device="cuda"):
    """Seeded N(0, std^2) draw on the GPU with torch (for the large workloads). The result is a
    torch tensor in bf16 or float32. Same (seed, tensor_id) -> same bits on a given torch build."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 1000003 + int(tensor_id))
    x = torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16) if dtype == "bf16" else x


@dataclass(frozen=True)
class Workload:
    """One workload: shapes and hyper-parameters, named by what it is."""

    name: str
    kind: str  # "linear", "sparse", "stack", "decode", "tiny"
    batch: int
    seq_len: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str
    seed: int
    block: int = 64
    topk: int = 64
    n_local: int = 2
    rope_base: float = 10000.0
    norm_eps: float = 1e-6
    chunk: int = 64
    layers: tuple = field(default=())


WORKLOADS = {
    # Tiny CPU-checkable case (both layer types): fp32, chunk 64, top-4 with n_local = 1.
    "tiny": Workload("tiny", "tiny", 1, 512, 2, 2, 64, "f32", 101, block=64, topk=4, n_local=1),
    # Linear-attention layer prefill, 32K tokens.
    "linear_32k": Workload("linear_32k", "linear", 1, 32768, 32, 32, 128, "bf16", 102),
    # Sparse layer prefill, 128K tokens, GQA 32 query heads over 2 KV heads.
    "sparse_128k": Workload("sparse_128k", "sparse", 1, 131072, 32, 2, 128, "bf16", 103),
    # Hybrid stack L, L, L, S at 256K tokens (linear: 32 heads MHA; sparse: 32/2 GQA).
    "stack_256k": Workload("stack_256k", "stack", 1, 262144, 32, 2, 128, "bf16", 104,
                           layers=("L", "L", "L", "S")),
    # Decode step at a 1M-token context, batch 8.
    "decode_1m": Workload("decode_1m", "decode", 8, 1048576, 32, 2, 128, "bf16", 105),
    # Packed batch of 16 prompts of mixed lengths (varlen_lengths) totalling 262,144 tokens,
    # through the L, L, L, S stack.
    "varlen_256k": Workload("varlen_256k", "varlen", 16, 262144, 32, 2, 128, "bf16", 108,
                            layers=("L", "L", "L", "S")),
}


def varlen_lengths(seed, nseq, total, lo=1024, hi=49152):
    """Seeded prompt lengths of a packed batch: log-uniform draws in [lo, hi], scaled to sum to
    `total` (floors, the remainder added to the last). No arithmetic of the method."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), 99])))
    raw = np.exp(rng.uniform(np.log(lo), np.log(hi), size=nseq))
    n = np.floor(raw / raw.sum() * total).astype(np.int64)
    n[-1] += total - int(n.sum())
    return [int(x) for x in n]
