"""KV-cache size and block-count formulas.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).
"""
from __future__ import annotations


def kv_bytes_per_token(layers: int, heads: int, head_dim: int, elt_bytes: int) -> int:
    """Bytes of K and V cached per token over all layers: layers x 2 x heads x head_dim x bytes
    ("KV Cache Mechanism Explained", section 3.1, the LLaMA-7B cache-size formula)."""
    return layers * 2 * heads * head_dim * elt_bytes


def kv_bytes(layers: int, heads: int, head_dim: int, seq_len: int, elt_bytes: int) -> int:
    """Bytes of one sequence's cache ("KV Cache and PagedAttention", section 1.1: 2 x L x H x T x
    d x b for one sequence)."""
    return kv_bytes_per_token(layers, heads, head_dim, elt_bytes) * seq_len


def blocks_needed(tokens: int, block_size: int = 16) -> int:
    """Physical blocks holding `tokens` tokens ("KV Cache and PagedAttention", section 2.2)."""
    return -(-tokens // block_size)


def wasted_slots(tokens: int, block_size: int = 16) -> int:
    """Unused slots in the last, partly filled block (section 2.2: at most block_size - 1)."""
    return blocks_needed(tokens, block_size) * block_size - tokens


def sampling_token_capacity(n: int, prompt: int, generated: int, shared: bool) -> int:
    """Token capacity held by n candidates of one prompt ("KV Cache and PagedAttention",
    section 5.1): every candidate stores its own copy, or the prompt is stored once."""
    return prompt + n * generated if shared else n * (prompt + generated)
