"""Page-granular request tables (page size P > 1), oracle side.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

"A walkthrough of SGLang", Exercises, exercise 2 describes the page-size option: the pool is
allocated by pages of P slots instead of one slot per token, and a request's table then names
one page per P positions ("Origins: the paper and the first commit" notes that the first
version used P = 1, one slot per token, and that larger pages came later). The pages do not
print the address arithmetic; the plainest reading, used here, is that page k of a request
holds its positions kP .. kP + P - 1 in order, so position j lives at slot

    page_table[row, j // P] * P + j % P.

Attention over a paged table is then exactly the token-granular definition over the slots
that formula names.
"""

from __future__ import annotations

import numpy as np

from .attention import decode_attention, extend_attention


def token_table(page_table: np.ndarray, page_size: int, width: int) -> np.ndarray:
    """``[rows, width]`` slot table of a page table: entry (r, j) is the slot of position j of
    row r, or -1 where that position's page entry is negative (unused)."""
    P = int(page_size)
    if P < 1:
        raise ValueError("page_size must be positive")
    pt = np.asarray(page_table, dtype=np.int64)
    if width > pt.shape[1] * P:
        raise ValueError("page table row too short for the requested width")
    j = np.arange(width)
    pages = pt[:, j // P]
    slots = pages * P + (j % P)[None, :]
    return np.where(pages < 0, -1, slots).astype(np.int64)


def extend_attention_paged(q, k_pool, v_pool, page_table, page_size, req_pool_indices, prefix_lens,
                           extend_lens, extend_start_loc, n_kv_heads, sm_scale, **kw):
    """EXTEND attention with keys addressed through a page table (see the module docstring)."""
    width = int(np.max(np.asarray(prefix_lens) + np.asarray(extend_lens), initial=0))
    table = token_table(page_table, page_size, max(width, 1))
    return extend_attention(q, k_pool, v_pool, table, req_pool_indices, prefix_lens, extend_lens,
                            extend_start_loc, n_kv_heads, sm_scale, **kw)


def decode_attention_paged(q, k_pool, v_pool, page_table, page_size, req_pool_indices, seq_lens,
                           n_kv_heads, sm_scale, **kw):
    """DECODE attention with keys addressed through a page table (see the module docstring)."""
    width = int(np.max(np.asarray(seq_lens), initial=0))
    table = token_table(page_table, page_size, max(width, 1))
    return decode_attention(q, k_pool, v_pool, table, req_pool_indices, seq_lens, n_kv_heads, sm_scale,
                            **kw)
