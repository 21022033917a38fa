"""Seeded synthetic inputs for paged-KV attention (shared by the HIP path's tests and the oracle's).

This module holds no attention arithmetic. It only draws lengths, request-table
rows, slot assignments and K/V/Q values, and rounds values to the element
format the pool stores. Both the HIP path and the CPU oracle consume the same
arrays, so both see identical bits.

Structure follows the pages' description of the state the kernels read:

* a token-granular pool, one slot per token ("Origins: the paper and the first
  commit", "Memory: a two-level pool paged by token"), laid out
  ``[slot, kv_head, head_dim]`` with K and V in separate arrays;
* a request table ``req_to_token[request, position] -> slot`` ("A walkthrough of
  SGLang", Main line 4), whose rows for requests that share a prefix hold the
  same leading slot numbers ("Inside SGLang", Step 3, "Paged KV and the kernels
  that read it");
* EXTEND batches whose input is the suffix only, with prefix/extend/seq lengths
  ("Origins...", "Batching: Req, Batch and the three forward modes"), and DECODE
  batches with one new token per request.

Recipe (all draws from ``seed``):

1. lengths (integers, inclusive ranges) from ``numpy.random.default_rng(seed)``;
2. a permutation of request-table rows, so the first indirection level is
   exercised; unused rows and columns hold -1;
3. a permutation of all pool slots; request positions take its entries in
   request-major order, EXTEND requests first, then DECODE requests. Requests
   with ``shared_prefix`` reuse the first request's prefix slots;
4. context K then context V (rows already in the pool: EXTEND prefixes, DECODE
   positions 0 .. L-2);
5. new K then new V (rows ``kv_store`` writes: EXTEND suffixes, then each DECODE
   request's current token at position L-1);
6. EXTEND Q then DECODE Q.

Values are normal with standard deviation ``sigma`` in float32. Each value
stream is drawn in fixed chunks of ``CHUNK`` values, chunk ``c`` of stream
``t`` from ``default_rng([seed, t, c])``, so the bits do not depend on how many
threads fill them. bfloat16 pools hold the round-to-nearest-even bit patterns
(``uint16``) of those float32 values. Pool slots that no request references are
filled with NaN, so a read of a wrong slot poisons the output.

Pages (``page_size`` P > 1, "A walkthrough of SGLang", Exercises, exercise 2: allocation by
pages of P slots): step 3 draws a permutation of the S / P pages instead, each request takes
pages in request-major order, and position j of a request lives at slot
``page[j // P] * P + j % P``; requests with ``shared_prefix`` share the first request's prefix
pages (the prefix length must then be a multiple of P). ``page_table[row, k]`` holds the k-th
page of the row (-1 where unused), and ``req_to_token`` holds the same slots token by token.

Variants: ``"normal"``; ``"peaked"`` (Q scaled by 8 / sigma**2 so that scaled
scores have standard deviation about 8); ``"needle"`` (per request and kv head,
one seeded key visible to every query of the request is set to ``NEEDLE_GAIN``
times a vector u, and the group's query heads are set to u, so the softmax puts
almost all weight on that key).
"""

from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field

import numpy as np

CHUNK = 1 << 22
NEEDLE_GAIN = 12.0
BF16_NAN = np.uint16(0x7FC0)

_STREAM_K_CTX, _STREAM_V_CTX, _STREAM_K_NEW, _STREAM_V_NEW, _STREAM_Q_EXT, _STREAM_Q_DEC = 1, 2, 3, 4, 5, 6
_STREAM_NEEDLE = 7


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even (finite inputs)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_stream(seed: int, stream: int, n: int, sigma: float) -> np.ndarray:
    """``n`` float32 normal values of standard deviation ``sigma`` from stream ``stream``."""
    out = np.empty(n, dtype=np.float32)
    chunks = [(c, c * CHUNK, min(n, (c + 1) * CHUNK)) for c in range((n + CHUNK - 1) // CHUNK)]

    def fill(job):
        c, a, b = job
        g = np.random.default_rng([seed, stream, c])
        g.standard_normal(b - a, dtype=np.float32, out=out[a:b])
        if sigma != 1.0:
            out[a:b] *= np.float32(sigma)

    if len(chunks) <= 1:
        for j in chunks:
            fill(j)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, chunks))
    return out


def _encode(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_to_bf16_bits(x)
    if dtype == "fp32":
        return x.astype(np.float32, copy=False)
    raise ValueError(dtype)


@dataclass(frozen=True)
class Spec:
    """Shape of one synthetic workload. Lengths are fixed tuples or drawn ranges."""

    name: str
    dtype: str                      # "bf16" (values stored as uint16 bits) or "fp32"
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    num_slots: int
    sigma: float = 1.0
    sm_scale: float | None = None   # default 1/sqrt(head_dim)
    extend_prefix: tuple = ()       # prefix length per EXTEND request
    extend_lens: tuple = ()         # extend (new-token) length per EXTEND request
    shared_prefix: bool = False     # every EXTEND request reuses request 0's prefix slots
    decode_lens: tuple = ()         # fixed DECODE context lengths (current token included)
    decode_batch: int = 0           # or: this many DECODE requests ...
    decode_range: tuple | None = None  # ... with lengths uniform in [lo, hi]
    spare_rows: int = 4             # request-table rows no request uses (held at -1)
    page_size: int = 1              # slots per page; 1 = token-granular (no page table)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def scale(self) -> float:
        return self.sm_scale if self.sm_scale is not None else 1.0 / float(np.sqrt(self.head_dim))


@dataclass
class ExtendBatch:
    req_pool_indices: np.ndarray    # [B] int32
    prefix_lens: np.ndarray         # [B] int32
    extend_lens: np.ndarray         # [B] int32
    extend_start_loc: np.ndarray    # [B] int32
    q: np.ndarray                   # [total_extend_tokens, Hq, D]

    @property
    def batch(self) -> int:
        return int(self.prefix_lens.shape[0])

    @property
    def total_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def max_extend_len(self) -> int:
        return int(self.extend_lens.max()) if self.batch else 0

    @property
    def max_seq_len(self) -> int:
        return int((self.prefix_lens + self.extend_lens).max()) if self.batch else 0


@dataclass
class DecodeBatch:
    req_pool_indices: np.ndarray    # [B] int32
    seq_lens: np.ndarray            # [B] int32
    q: np.ndarray                   # [B, Hq, D]

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.batch else 0


@dataclass
class Workload:
    spec: Spec
    seed: int
    variant: str
    k_pool: np.ndarray              # [S, Hkv, D]: context rows written, everything else NaN
    v_pool: np.ndarray
    req_to_token: np.ndarray        # [R, W] int32
    store_loc: np.ndarray           # [n_new] int32: slots of the rows kv_store writes
    k_new: np.ndarray               # [n_new, Hkv, D]
    v_new: np.ndarray
    extend: ExtendBatch | None = None
    decode: DecodeBatch | None = None
    needles: dict = field(default_factory=dict)  # (kind, request, kv_head) -> position
    page_table: np.ndarray | None = None  # [R, W / P] int32 when page_size > 1

    @property
    def sm_scale(self) -> float:
        return self.spec.scale


def _draw_lengths(spec: Spec, rng: np.random.Generator):
    ext_p = np.asarray(spec.extend_prefix, dtype=np.int64)
    ext_e = np.asarray(spec.extend_lens, dtype=np.int64)
    if ext_p.shape != ext_e.shape:
        raise ValueError("extend_prefix and extend_lens differ in length")
    if spec.decode_range is not None:
        lo, hi = spec.decode_range
        dec = rng.integers(lo, hi + 1, size=spec.decode_batch).astype(np.int64)
    else:
        dec = np.asarray(spec.decode_lens, dtype=np.int64)
    if dec.size and dec.min() < 1:
        raise ValueError("a DECODE request needs at least its current token")
    if spec.shared_prefix and ext_p.size and np.any(ext_p != ext_p[0]):
        raise ValueError("shared_prefix needs equal prefix lengths")
    return ext_p, ext_e, dec


def make_workload(spec: Spec, seed: int, variant: str = "normal") -> Workload:
    """Draw one workload (see the module docstring for the recipe)."""
    if variant not in ("normal", "peaked", "needle"):
        raise ValueError(f"unknown variant {variant!r}")
    if spec.n_q_heads % spec.n_kv_heads:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    rng = np.random.default_rng(seed)
    S, Hkv, Hq, D = spec.num_slots, spec.n_kv_heads, spec.n_q_heads, spec.head_dim
    G = Hq // Hkv

    # 1. lengths
    ext_p, ext_e, dec_L = _draw_lengths(spec, rng)
    Be, Bd = ext_p.size, dec_L.size

    # 2. request-table rows
    R = Be + Bd + spec.spare_rows
    row_perm = rng.permutation(R)
    ext_rows = row_perm[:Be]
    dec_rows = row_perm[Be:Be + Bd]
    seq_ext = ext_p + ext_e
    W = int(max([1] + list(seq_ext) + list(dec_L)))
    W = (W + 15) // 16 * 16 + 16
    r2t = np.full((R, W), -1, dtype=np.int32)

    # 3. slot assignment
    P = spec.page_size
    page_table = None
    if P == 1:
        slot_perm = rng.permutation(S)
        cursor = 0

        def take(n):
            nonlocal cursor
            if cursor + n > S:
                raise ValueError(f"workload {spec.name} needs more than {S} slots")
            s = slot_perm[cursor:cursor + n]
            cursor += n
            return s

        def place(row, lo, n, shared_slots=None):
            """Slots of positions lo .. lo+n-1 of a request-table row."""
            s = take(n) if shared_slots is None else shared_slots
            r2t[row, lo:lo + n] = s
            return s
    else:
        if P < 1 or P & (P - 1) or S % P:
            raise ValueError("page_size must be a power of two dividing the pool")
        page_perm = rng.permutation(S // P)
        pcur = 0
        page_table = np.full((R, (W + P - 1) // P), -1, dtype=np.int32)

        def place(row, lo, n, shared_slots=None):
            """Slots of positions lo .. lo+n-1 of a row, taking new pages as positions reach them."""
            nonlocal pcur
            if shared_slots is not None:
                page_table[row, lo // P:(lo + n) // P] = shared_slots[::P] // P
                r2t[row, lo:lo + n] = shared_slots
                return shared_slots
            for k in range(lo // P, (lo + n + P - 1) // P):
                if page_table[row, k] < 0:
                    if pcur >= S // P:
                        raise ValueError(f"workload {spec.name} needs more than {S // P} pages")
                    page_table[row, k] = page_perm[pcur]
                    pcur += 1
            j = np.arange(lo, lo + n)
            s = page_table[row, j // P].astype(np.int64) * P + j % P
            r2t[row, lo:lo + n] = s
            return s

    ctx_slots, new_slots = [], []
    shared = None
    for b in range(Be):
        p, e = int(ext_p[b]), int(ext_e[b])
        if spec.shared_prefix and shared is not None:
            pre = place(ext_rows[b], 0, p, shared)
        else:
            if spec.shared_prefix and p % P:
                raise ValueError("a shared prefix must fill whole pages")
            pre = place(ext_rows[b], 0, p)
            ctx_slots.append(pre)
            if spec.shared_prefix:
                shared = pre
        new_slots.append(place(ext_rows[b], p, e))
    for b in range(Bd):
        L = int(dec_L[b])
        ctx_slots.append(place(dec_rows[b], 0, L - 1))
        new_slots.append(place(dec_rows[b], L - 1, 1))
    ctx_slots = np.concatenate(ctx_slots) if ctx_slots else np.zeros(0, np.int64)
    new_slots = np.concatenate(new_slots) if new_slots else np.zeros(0, np.int64)
    n_ctx, n_new = ctx_slots.size, new_slots.size
    row = Hkv * D

    # 4-6. values (float32, before rounding)
    k_ctx = normal_stream(seed, _STREAM_K_CTX, n_ctx * row, spec.sigma).reshape(n_ctx, Hkv, D)
    v_ctx = normal_stream(seed, _STREAM_V_CTX, n_ctx * row, spec.sigma).reshape(n_ctx, Hkv, D)
    k_new = normal_stream(seed, _STREAM_K_NEW, n_new * row, spec.sigma).reshape(n_new, Hkv, D)
    v_new = normal_stream(seed, _STREAM_V_NEW, n_new * row, spec.sigma).reshape(n_new, Hkv, D)
    n_qe = int(ext_e.sum())
    q_ext = normal_stream(seed, _STREAM_Q_EXT, n_qe * Hq * D, spec.sigma).reshape(n_qe, Hq, D)
    q_dec = normal_stream(seed, _STREAM_Q_DEC, Bd * Hq * D, spec.sigma).reshape(Bd, Hq, D)

    starts = np.zeros(Be, dtype=np.int64)
    if Be:
        starts[1:] = np.cumsum(ext_e)[:-1]

    needles = {}
    if variant == "peaked":
        gain = np.float32(8.0 / (spec.sigma * spec.sigma))
        q_ext *= gain
        q_dec *= gain
    elif variant == "needle":
        # 7. needle positions and directions, from their own stream
        nrng = np.random.default_rng([seed, _STREAM_NEEDLE])
        ctx_row_of_slot = {int(s): i for i, s in enumerate(ctx_slots)}
        new_row_of_slot = {int(s): i for i, s in enumerate(new_slots)}

        def plant(kind, b, g, row_idx, pos, q_rows):
            slot = int(r2t[row_idx, pos])
            u = nrng.standard_normal(D).astype(np.float32)
            if slot in ctx_row_of_slot:
                k_ctx[ctx_row_of_slot[slot], g, :] = np.float32(NEEDLE_GAIN) * u
            else:
                k_new[new_row_of_slot[slot], g, :] = np.float32(NEEDLE_GAIN) * u
            q_rows[:, g * G:(g + 1) * G, :] = u[None, None, :]
            needles[(kind, b, g)] = pos

        used = set()
        for b in range(Be):
            p, e = int(ext_p[b]), int(ext_e[b])
            if e == 0:
                continue
            for g in range(Hkv):
                if p == 0:
                    pos = 0
                else:
                    pos = int(nrng.integers(0, p))
                    if spec.shared_prefix:
                        while (pos, g) in used and len(used) < p * Hkv:
                            pos = int(nrng.integers(0, p))
                        used.add((pos, g))
                plant("extend", b, g, ext_rows[b], pos, q_ext[starts[b]:starts[b] + e])
        for b in range(Bd):
            L = int(dec_L[b])
            for g in range(Hkv):
                pos = int(nrng.integers(0, L))
                plant("decode", b, g, dec_rows[b], pos, q_dec[b:b + 1])

    # encode into the stored element format
    k_ctx, v_ctx = _encode(k_ctx, spec.dtype), _encode(v_ctx, spec.dtype)
    k_new, v_new = _encode(k_new, spec.dtype), _encode(v_new, spec.dtype)
    q_ext, q_dec = _encode(q_ext, spec.dtype), _encode(q_dec, spec.dtype)

    if spec.dtype == "bf16":
        k_pool = np.full((S, Hkv, D), BF16_NAN, dtype=np.uint16)
        v_pool = np.full((S, Hkv, D), BF16_NAN, dtype=np.uint16)
    else:
        k_pool = np.full((S, Hkv, D), np.nan, dtype=np.float32)
        v_pool = np.full((S, Hkv, D), np.nan, dtype=np.float32)
    if n_ctx:
        k_pool[ctx_slots] = k_ctx
        v_pool[ctx_slots] = v_ctx

    i32 = lambda a: np.ascontiguousarray(a, dtype=np.int32)
    extend = None
    if Be:
        extend = ExtendBatch(i32(ext_rows), i32(ext_p), i32(ext_e), i32(starts), q_ext)
    decode = None
    if Bd:
        decode = DecodeBatch(i32(dec_rows), i32(dec_L), q_dec)
    return Workload(spec, seed, variant, k_pool, v_pool, r2t, i32(new_slots), k_new, v_new,
                    extend, decode, needles, page_table)


# The five workloads the method is measured on. Seeds for timing runs are
# TIMING_SEEDS[id]; parity runs also use seed + 100 and seed + 200.
CONFIGS = {
    1: Spec("tiny-extend-fp32", "fp32", 4, 4, 64, 1024, 1.0,
            extend_prefix=(0, 16, 64, 128), extend_lens=(32, 16, 8, 1)),
    2: Spec("decode-64req-ctx512-4096-bf16", "bf16", 32, 8, 128, 524288, 1.0,
            decode_batch=64, decode_range=(512, 4096)),
    3: Spec("shared-prefix-extend-32x(4096+256)-bf16", "bf16", 32, 8, 128, 262144, 1.0,
            extend_prefix=(4096,) * 32, extend_lens=(256,) * 32, shared_prefix=True),
    4: Spec("mixed-chunk-2048on14336+decode-128req-bf16", "bf16", 32, 8, 128, 1048576, 1.0,
            extend_prefix=(14336,), extend_lens=(2048,),
            decode_batch=128, decode_range=(1024, 8192)),
    5: Spec("long-context-8192on65536+decode-8req-32K-128K-bf16", "bf16", 64, 8, 128, 2097152, 0.5,
            extend_prefix=(65536,), extend_lens=(8192,),
            decode_batch=8, decode_range=(32768, 131072)),
}
TIMING_SEEDS = {1: 1001, 2: 1002, 3: 1003, 4: 1004, 5: 1005, 6: 1006}

# Further workloads, not among the five: 6 is a short suffix on a long cached prefix (the
# multi-turn case), whose few row tiles take the EXTEND key splits.
EXTRA = {
    6: Spec("short-suffix-100on10000-bf16", "bf16", 32, 8, 128, 1048576, 1.0,
            extend_prefix=(10000,), extend_lens=(100,)),
}


def workload_spec(wid: int) -> Spec:
    """The Spec of workload `wid` (1..5, or one of EXTRA)."""
    return CONFIGS[wid] if wid in CONFIGS else EXTRA[wid]
