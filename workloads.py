"""Seeded synthetic inputs and workload shapes for decode attention over a KV cache.

This module is shared by the tests, the benchmark and the smoke check. It holds random draws and
shape bookkeeping only: no attention arithmetic, no cache layout logic and no codec. Both the CPU
oracle and the HIP path receive the arrays produced here and nothing else in common.

Value distribution: K, V and Q entries are standard normal, drawn in float32 from a seeded
generator and, for fp16 workloads, rounded to fp16 (round to nearest even) by NumPy or torch.

Workload shapes follow the pages' model dimensions:
  * tiny character GPT: 6 heads x 64-dim heads, context 256 (From Neuron to GPT, "KV cache"
    chapter, trainer section: 6 blocks, 6 heads, embedding 384, context 256);
  * LLaMA-7B: 32 layers x 32 heads x 128 (KV Cache Mechanism Explained, section 3.1);
  * LLaMA-13B: 40 layers x 40 heads x 128 (KV Cache and PagedAttention, section 1.1);
  * parallel sampling: 8 candidates, 1024-token prompt, 128 generated tokens (KV Cache and
    PagedAttention, section 5.1).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BLOCK_SIZE = 16


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def normal_f32(gen: np.random.Generator, shape) -> np.ndarray:
    """Standard normal float32 draws."""
    return gen.standard_normal(size=shape, dtype=np.float32)


def normal(gen: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """Standard normal draws stored in `dtype` ("f32" or "f16")."""
    x = normal_f32(gen, shape)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    raise ValueError(dtype)


def uniform_lengths(gen: np.random.Generator, n: int, lo: int, hi: int) -> np.ndarray:
    """n integers drawn uniformly from the closed range [lo, hi]."""
    return gen.integers(lo, hi + 1, size=n).astype(np.int64)


def permutation(gen: np.random.Generator, n: int) -> np.ndarray:
    return gen.permutation(n).astype(np.int32)


def torch_normal(shape, dtype, device, seed: int):
    """Standard normal tensor drawn on `device` by torch's seeded generator (large workloads
    whose inputs are generated in device memory). Returns a tensor of `dtype`."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return x.to(dtype)


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "contig" or "paged"
    layers: int
    batch: int
    heads: int
    head_dim: int
    kv_dtype: str             # "f32", "f16", "e4m3"
    q_dtype: str
    seed: int
    # contiguous: capacity per sequence; paged: unused
    s_max: int = 0
    # attended length after the append (contig / fp8): every sequence has this length
    ctx: int = 0
    # paged with drawn lengths: closed range of the attended length
    ctx_lo: int = 0
    ctx_hi: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))


TINY_GPT = Workload(
    name="tiny-gpt-6x64-f32-contig-ctx256", kind="contig", layers=1, batch=1, heads=6,
    head_dim=64, kv_dtype="f32", q_dtype="f32", seed=1, s_max=256, ctx=256,
    extra={"prefill": 16, "decode_steps": 240})

LLAMA7B_CONTIG = Workload(
    name="llama7b-32x32x128-f16-contig-b16-ctx2048", kind="contig", layers=32, batch=16,
    heads=32, head_dim=128, kv_dtype="f16", q_dtype="f16", seed=2, s_max=2048, ctx=2048)

LLAMA13B_PAGED = Workload(
    name="llama13b-40x40x128-f16-paged16-b32-ctxU64-2048", kind="paged", layers=40, batch=32,
    heads=40, head_dim=128, kv_dtype="f16", q_dtype="f16", seed=3, ctx_lo=64, ctx_hi=2048)

# Parallel sampling runs LLaMA-13B's 40 layers (one block table per candidate serves all of
# them), so a step reads each layer's shared prompt from memory as a model would.
PARALLEL_SAMPLING = Workload(
    name="parallel-sampling-8x(1024+128)-40x128-f16-paged16", kind="paged", layers=40, batch=8,
    heads=40, head_dim=128, kv_dtype="f16", q_dtype="f16", seed=4,
    extra={"prompt": 1024, "generate": 128, "cow_variant_prompt": 1020})

# The copy-on-write variant: a 1020-token prompt ends inside a block, so the first generated
# token of candidates 0-6 copies the shared partial block; candidate 7 writes in place.
PARALLEL_SAMPLING_COW = Workload(
    name="parallel-sampling-8x(1020+128)-40x128-f16-paged16-cow", kind="paged", layers=40,
    batch=8, heads=40, head_dim=128, kv_dtype="f16", q_dtype="f16", seed=4,
    extra={"prompt": 1020, "generate": 128})

LONGCTX_FP8 = Workload(
    name="llama7b-32x32x128-e4m3-paged16-b64-ctx4096", kind="paged", layers=32, batch=64,
    heads=32, head_dim=128, kv_dtype="e4m3", q_dtype="f16", seed=5, ctx=4096)

ALL = [TINY_GPT, LLAMA7B_CONTIG, LLAMA13B_PAGED, PARALLEL_SAMPLING, LONGCTX_FP8]

# The int8 cache (KV Cache Mechanism Explained, section 8, item 3 names FP8/INT8 for the cached
# history): the fp8 long-context shapes with int8 codes and per-block scales.
LONGCTX_I8 = Workload(
    name="llama7b-32x32x128-i8-paged16-b64-ctx4096", kind="paged", layers=32, batch=64,
    heads=32, head_dim=128, kv_dtype="i8", q_dtype="f16", seed=9, ctx=4096)

# Shared K/V heads (grouped-query attention): 64 query heads over 8 K/V heads (G = 8), the
# attention shape of a LLaMA-2-70B-class model, with the LLaMA-13B batch's length mix.
# `heads` counts the K/V heads; the query heads are heads * extra["group"].
GQA8_PAGED = Workload(
    name="gqa-64q8kv-x128-f16-paged16-b32-ctxU64-2048", kind="paged", layers=80, batch=32,
    heads=8, head_dim=128, kv_dtype="f16", q_dtype="f16", seed=6, ctx_lo=64, ctx_hi=2048,
    extra={"group": 8})


# Rolling window (KV Cache Mechanism Explained, section 8, item 2): LLaMA-13B shapes at a 2048
# context with the cache window held to the last 1024 tokens (the page pairs a window cache with
# LLaMA-13B at context 2048 and gives no window size).
LLAMA13B_WINDOW = Workload(
    name="llama13b-40x40x128-f16-paged16-b32-ctx2048-window1024", kind="paged", layers=40,
    batch=32, heads=40, head_dim=128, kv_dtype="f16", q_dtype="f16", seed=7, ctx=2048,
    extra={"window": 1024})


# Prefill (the chunked multi-query attention on either side of decode): LLaMA-7B head shapes,
# four 2048-token prompts each prefilled whole (causal attention over the prompt), 32 layers.
LLAMA7B_PREFILL = Workload(
    name="llama7b-32x32x128-f16-paged16-prefill-b4x2048", kind="paged", layers=32, batch=4,
    heads=32, head_dim=128, kv_dtype="f16", q_dtype="f16", seed=8, ctx=2048,
    extra={"prompt": 2048})


# Whole-cache compression to 8 bits ("KV Cache Mechanism Explained", section 6.1, item 1;
# "KV Cache and PagedAttention", section 7.2, item 1): the long-context shapes' fp16 cache (64
# sequences of 4096 tokens, LLaMA-7B heads) re-encoded block by block into an int8 cache, 8
# layers per step (the fp16 and int8 pools of 8 layers take 52 GB).
COMPRESS_I8 = Workload(
    name="llama7b-32x32x128-f16-to-i8-compress-paged16-b64-ctx4096-8layers", kind="paged",
    layers=8, batch=64, heads=32, head_dim=128, kv_dtype="i8", q_dtype="f16", seed=10, ctx=4096,
    extra={"compress_from": "f16"})


def llama13b_lengths(w: Workload = LLAMA13B_PAGED, seed: int | None = None) -> np.ndarray:
    """Attended lengths of the LLaMA-13B paged batch: uniform in [ctx_lo, ctx_hi]."""
    g = rng(w.seed if seed is None else seed)
    return uniform_lengths(g, w.batch, w.ctx_lo, w.ctx_hi)


def llama13b_pool_order(num_blocks: int, seed: int) -> np.ndarray:
    """Shuffled physical-block order for the LLaMA-13B paged pool (a seeded permutation)."""
    return permutation(rng(seed + 1000), num_blocks)


def blocks_for(n_tokens: int, block_size: int = BLOCK_SIZE) -> int:
    return -(-int(n_tokens) // block_size)
