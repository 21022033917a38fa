"""CPU oracle for paged-KV attention over a token-granular slot pool.

TEST INFRASTRUCTURE ONLY. Nothing in the product library may import, call or
link this package: only the tests, the smoke check and the benchmark's
``cpu_baseline`` leg use it. It shares no code, tables or helpers with the HIP
path; the only thing both sides see is the seeded input arrays.

What it computes is the plain definition of the method, in float64:

* ``kv_store`` -- write new K/V rows into pool slots by index
  ("Origins: the paper and the first commit", section "Execution: RadixAttention
  and two sets of kernels": the store writes this layer's K and V at the slots
  the batch allocated, or raises when no location is given).
* ``extend_attention`` -- the new suffix rows of each request attend causally to
  the request's cached prefix plus themselves, every key gathered through
  ``req_to_token`` ("Origins...", self-test answer 2 and section "Batching: Req,
  Batch and the three forward modes"; "Inside SGLang", Step 3, the four steps
  of attention for one head).
* ``decode_attention`` -- one query per request over its whole context
  ("Inside SGLang", Step 3, "Prefill and decode have different shapes").
* ``paged`` -- page-granular request tables (page size P > 1, "A walkthrough of SGLang",
  Exercises, exercise 2): position j at slot page_table[row, j // P] * P + j % P.
* ``fp8`` -- the FP8 E4M3 KV pool ("Inside SGLang", Step 6): exact decode of each byte,
  the store's encoding (``kv_store_fp8``); the attention functions take per-pool scales.

Parity status of every function is pinned by tests under ``tests/`` (brute
force on tiny inputs, closed forms, invariants, a textbook library routine on
the square prefill case, and the constants the pages print).
"""

from .formats import to_f64, bf16_bits_to_f64
from .attention import (
    kv_store,
    extend_attention,
    decode_attention,
    gather_request_kv,
)
from .fp8 import e4m3_bits_to_f64, e4m3_round, kv_store_fp8, quantize_bf16
from .paged import token_table, extend_attention_paged, decode_attention_paged
from .bruteforce import (
    extend_attention_loops,
    decode_attention_loops,
)

__all__ = [
    "to_f64",
    "bf16_bits_to_f64",
    "kv_store",
    "extend_attention",
    "decode_attention",
    "gather_request_kv",
    "extend_attention_loops",
    "decode_attention_loops",
    "e4m3_bits_to_f64",
    "e4m3_round",
    "kv_store_fp8",
    "quantize_bf16",
    "token_table",
    "extend_attention_paged",
    "decode_attention_paged",
]
