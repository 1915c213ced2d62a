"""Byte accounting for KV caches and for one decode step.

The cache-size formula is the one "Transformer推理核心：KV Cache、GQA与RoPE原理与
工程实践" §5.3 and "Transformer架构优化实战2026" §四 give: two tensors (K and V)
per layer, each kv_heads x head_dim values per token per sequence.
"""
from __future__ import annotations

import numpy as np


def kv_cache_bytes(batch: int, layers: int, kv_heads: int, seq_len: int,
                   head_dim: int, dtype_bytes: int) -> int:
    """2 * batch * layers * kv_heads * seq_len * head_dim * dtype_bytes."""
    return 2 * batch * layers * kv_heads * seq_len * head_dim * dtype_bytes


def decode_kv_read_bytes(seq_lens, kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    """K and V bytes one decode step must read for one layer: the cache formula
    summed over sequences of different lengths (layers = 1, batch folded into
    the sum of lengths)."""
    total_tokens = int(np.asarray(seq_lens, dtype=np.int64).sum())
    return kv_cache_bytes(1, 1, kv_heads, total_tokens, head_dim, dtype_bytes)


def decode_aux_bytes(batch: int, n_heads: int, kv_heads: int, head_dim: int,
                     dtype_bytes: int, n_table_entries: int = 0) -> int:
    """Other compulsory bytes of one step: q, k_new, v_new reads, the appended
    K/V rows, q_rot written and read back (fp32), out (fp32), lse (fp32),
    positions/lengths and block-table entries (int32)."""
    qkv_in = batch * (n_heads + 2 * kv_heads) * head_dim * dtype_bytes
    append = 2 * batch * kv_heads * head_dim * dtype_bytes
    q_rot = 2 * batch * n_heads * head_dim * 4
    out = batch * n_heads * (head_dim + 1) * 4
    ints = 2 * batch * 4 + 4 * n_table_entries
    return qkv_in + append + q_rot + out + ints


def window_key_count(seq_lens, n_query: int) -> int:
    """Keys attended by all queries of a step with T = n_query new tokens per
    sequence (query t of sequence b sees the tokens j < L_b - T + 1 + t),
    summed over queries and sequences.  A prompt from empty (L = T) gives
    T (T + 1) / 2 per sequence."""
    T = int(n_query)
    total = 0
    for L in np.asarray(seq_lens, dtype=np.int64):
        a = int(L) - T + 1                       # keys of query 0
        if a >= 1:
            total += T * a + T * (T - 1) // 2
        else:
            top = a + T - 1                      # keys of the last query
            total += top * (top + 1) // 2 if top > 0 else 0
    return total


def window_attention_flops(seq_lens, n_query: int, n_heads: int, head_dim: int) -> int:
    """Multiply-adds of q K^T and P V, two flops each: 4 * head_dim per
    (query head, attended key)."""
    return 4 * head_dim * n_heads * window_key_count(seq_lens, n_query)
