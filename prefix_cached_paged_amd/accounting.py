"""Algorithmic work of the paged-attention calls: the numerators of the roofline figures.

Only work the method needs is counted: attended (query, key) pairs for EXTEND
(masked pairs, padding, softmax and recombination are not counted), and the
K/V rows a DECODE step must read. The per-token KV byte count follows the
formula of "Inside SGLang", Step 6 (kv heads x (K + V width) x layers x bytes
per value); one call of this library handles one layer.
"""

from __future__ import annotations

import numpy as np


def kv_bytes_per_token(n_kv_heads: int, head_dim: int, layers: int, elem_bytes: int) -> int:
    """Bytes of K plus V one token holds in the pool across ``layers`` layers."""
    return n_kv_heads * (2 * head_dim) * layers * elem_bytes


def extend_pairs(prefix_lens, extend_lens) -> int:
    """Attended (query, key) pairs per head: suffix row i of a request sees p + i + 1 keys."""
    p = np.asarray(prefix_lens, dtype=np.int64)
    e = np.asarray(extend_lens, dtype=np.int64)
    return int(np.sum(e * p + e * (e + 1) // 2))


def extend_flops(prefix_lens, extend_lens, n_q_heads: int, head_dim: int) -> int:
    """2*D for Q K^T plus 2*D for P V per attended pair and query head."""
    return 4 * head_dim * n_q_heads * extend_pairs(prefix_lens, extend_lens)


def decode_kv_bytes(seq_lens, n_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """K and V bytes a DECODE step reads: every context token, every kv head, one layer."""
    L = int(np.sum(np.asarray(seq_lens, dtype=np.int64)))
    return L * kv_bytes_per_token(n_kv_heads, head_dim, 1, elem_bytes)


def decode_total_bytes(seq_lens, batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                       elem_bytes: int) -> int:
    """KV bytes plus the 4-byte slot index per key and the q read / o write."""
    L = int(np.sum(np.asarray(seq_lens, dtype=np.int64)))
    return (decode_kv_bytes(seq_lens, n_kv_heads, head_dim, elem_bytes) + 4 * L
            + 2 * batch * n_q_heads * head_dim * elem_bytes)


def kv_store_bytes(n_new: int, n_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Read the new K and V rows, write them to the pool, read the slot indices."""
    return 2 * n_new * kv_bytes_per_token(n_kv_heads, head_dim, 1, elem_bytes) + 4 * n_new
