"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and builds shapes; it holds none of the
method's arithmetic.  Both the GPU library and the CPU oracle receive the very
same tensors from here (the oracle gets a host copy), so neither side depends
on the other.

Draw recipe: float32 N(0, std) from a seeded ``torch.Generator`` on the target
device, then a round-to-nearest-even cast to the requested dtype.  Embedding
tables use std 0.02, attention operands std 1.  Token ids are uniform integers.
Seeds: Q=0, K=1, V=2, tables=3 (+s for stream s), ids=4, K cache=5, V cache=6,
new K=7, new V=8.
"""
from dataclasses import dataclass

import torch

SEED_Q, SEED_K, SEED_V, SEED_TABLES, SEED_IDS = 0, 1, 2, 3, 4
SEED_KCACHE, SEED_VCACHE, SEED_KNEW, SEED_VNEW = 5, 6, 7, 8


def normal(shape, seed, dtype=torch.bfloat16, device="cpu", std=1.0):
    """float32 N(0, std) from a seeded generator, cast (RNE) to ``dtype``."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=gen, dtype=torch.float32, device=device)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def token_ids(B, L, V, seed=SEED_IDS, device="cpu", force_edges=False):
    """int32 ids uniform in [0, V); optionally force 0 and V-1 to appear."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    ids = torch.randint(0, V, (B, L), generator=gen, dtype=torch.int64, device=device).to(torch.int32)
    if force_edges and ids.numel() >= 2:
        flat = ids.view(-1)
        flat[0] = 0
        flat[-1] = V - 1
    return ids


def tables(n, V, D, dtype=torch.bfloat16, device="cpu", std=0.02, seed=SEED_TABLES):
    """n independent [V, D] embedding tables."""
    return [normal((V, D), seed + 100 * s, dtype, device, std) for s in range(n)]


def qkv(B, L, n, Hq, Hkv, d, dtype=torch.bfloat16, device="cpu"):
    """Q [B, nL, Hq, d], K/V [B, nL, Hkv, d], each N(0, 1)."""
    nL = n * L
    return (normal((B, nL, Hq, d), SEED_Q, dtype, device),
            normal((B, nL, Hkv, d), SEED_K, dtype, device),
            normal((B, nL, Hkv, d), SEED_V, dtype, device))


def decode_inputs(B, n, Hq, Hkv, d, T_cap, dtype=torch.bfloat16, device="cpu"):
    """q [B,n,Hq,d], k_new/v_new [B,n,Hkv,d], caches [B,T_cap,n,Hkv,d]."""
    return (normal((B, n, Hq, d), SEED_Q, dtype, device),
            normal((B, n, Hkv, d), SEED_KNEW, dtype, device),
            normal((B, n, Hkv, d), SEED_VNEW, dtype, device),
            normal((B, T_cap, n, Hkv, d), SEED_KCACHE, dtype, device),
            normal((B, T_cap, n, Hkv, d), SEED_VCACHE, dtype, device))


@dataclass(frozen=True)
class PrefillShape:
    name: str
    B: int
    L: int
    n: int
    Hq: int
    Hkv: int
    d: int
    mode: int        # 0 intra, 1 cross
    window: int      # tokens, 0 = none
    dtype: torch.dtype


@dataclass(frozen=True)
class DecodeShape:
    name: str
    B: int
    ctx: int         # tokens already cached per sequence
    n: int
    Hq: int
    Hkv: int
    d: int
    dtype: torch.dtype


# The workloads of the method's measurement plan (synthetic stand-ins for the
# pages' training and serving runs; see the design notes for the recipe).
TINY_INTRA = PrefillShape("tiny-intra n2 L64 h4 d32 f32", 1, 64, 2, 4, 4, 32, 0, 0, torch.float32)
TINY_CROSS = PrefillShape("tiny-cross n2 L64 h4 d32 f32", 1, 64, 2, 4, 4, 32, 1, 0, torch.float32)
TINY_N1 = PrefillShape("tiny-n1 L64 h4 d32 f32", 1, 64, 1, 4, 4, 32, 0, 0, torch.float32)
INTRA_4K = PrefillShape("intra n4 L4096 32q/8kv d128 bf16", 1, 4096, 4, 32, 8, 128, 0, 0, torch.bfloat16)
INTRA_4K_N1 = PrefillShape("intra n1 L4096 32q/8kv d128 bf16", 1, 4096, 1, 32, 8, 128, 0, 0, torch.bfloat16)
CROSS_4K = PrefillShape("cross n4 L4096 32q/8kv d128 bf16", 1, 4096, 4, 32, 8, 128, 1, 0, torch.bfloat16)
LONG_INTRA_W = PrefillShape("intra-W4096 n4 L32768 16q/4kv d128 bf16", 1, 32768, 4, 16, 4, 128, 0, 4096, torch.bfloat16)
LONG_CROSS = PrefillShape("cross n4 L32768 16q/4kv d128 bf16", 1, 32768, 4, 16, 4, 128, 1, 0, torch.bfloat16)
LONG_CROSS_W = PrefillShape("cross-W4096 n4 L32768 16q/4kv d128 bf16", 1, 32768, 4, 16, 4, 128, 1, 4096, torch.bfloat16)
DECODE_8K = DecodeShape("decode B64 ctx8192 n4 32q/8kv d128 bf16", 64, 8192, 4, 32, 8, 128, torch.bfloat16)
EMBED_DECODE = dict(B=64, L=1, n=4, V=160000, D=7168, dtype=torch.bfloat16)
EMBED_PREFILL = dict(B=1, L=4096, n=4, V=160000, D=7168, dtype=torch.bfloat16)

