"""Plain float64 definition of paged-KV EXTEND and DECODE attention.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Every key and value is gathered through the two-level indirection
``req_to_token[req_pool_indices[b], position] -> slot -> pool[slot, kv_head, :]``
("A walkthrough of SGLang", Main line 4: row r, column i of the request table is
the KV slot of request r's token i; the pool is read by slot), then dense
attention is taken over the gathered rows exactly as written for one head in
"Inside SGLang", Step 3: scores Q K^T, scaled by the softmax scale, minus
infinity above the causal diagonal, softmax along each row, times V.

Readings of points the pages leave open (each is listed with its reason in the
design notes of the repository):

* causal alignment in EXTEND is bottom-right: suffix row i of a request with
  prefix length p sits at absolute position p + i and sees keys 0 .. p + i,
  itself included (the pages set seq_len = prefix + extend and feed only the
  suffix to the model; "Origins...", "Batching: Req, Batch and the three
  forward modes");
* query head h reads kv head h // G with G = n_q_heads / n_kv_heads
  (contiguous groups; "Inside SGLang", Step 3, two query heads share each key
  and value head);
* the softmax scale is an argument and is applied to the raw score before the
  mask;
* a request with extend length 0 contributes no rows; a DECODE request with
  seq_len 0 is an error.

No blocking, online softmax or reordering is used: each query row's full score
row over its keys is formed, normalised and multiplied by V. Query rows are only
processed in groups of at most ``row_block`` to bound memory; every group still
forms complete score rows.
"""

from __future__ import annotations

import numpy as np

from .formats import to_f64


def _check_pool(k_pool: np.ndarray, v_pool: np.ndarray) -> tuple[int, int, int]:
    if k_pool.shape != v_pool.shape or k_pool.ndim != 3:
        raise ValueError(f"pools must both be [slots, kv_heads, head_dim], got {k_pool.shape} and {v_pool.shape}")
    if k_pool.dtype != v_pool.dtype:
        raise ValueError("K and V pools must share one element format")
    return k_pool.shape


def kv_store(k_pool, v_pool, k_new, v_new, loc):
    """Return copies of the pools with row ``loc[i]`` replaced by the i-th new row.

    Follows "Origins: the paper and the first commit", section "Execution:
    RadixAttention and two sets of kernels": the layer's new K and V are written
    into the key and value buffers at the slots given by the batch's output
    locations, and the store refuses to run when no location is given.

    Reading of a point the pages leave open: all entries of ``loc`` must be
    distinct and inside the pool; the oracle raises otherwise. Rows not named in
    ``loc`` are left bit-for-bit as they were.
    """
    if loc is None:
        raise ValueError("kv_store needs the slot locations of the new rows")
    S, Hkv, D = _check_pool(k_pool, v_pool)
    loc = np.asarray(loc)
    if loc.ndim != 1:
        raise ValueError("loc must be one-dimensional")
    n = loc.shape[0]
    if k_new.shape != (n, Hkv, D) or v_new.shape != (n, Hkv, D):
        raise ValueError(f"new rows must be [{n}, {Hkv}, {D}], got {k_new.shape} and {v_new.shape}")
    if k_new.dtype != k_pool.dtype or v_new.dtype != v_pool.dtype:
        raise ValueError("new rows must have the pool's element format")
    if n and (loc.min() < 0 or loc.max() >= S):
        raise ValueError("a slot location lies outside the pool")
    if np.unique(loc).shape[0] != n:
        raise ValueError("slot locations must be distinct")
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    for i in range(n):
        k_out[loc[i]] = k_new[i]
        v_out[loc[i]] = v_new[i]
    return k_out, v_out


def _heads(kv_heads, Hkv):
    """The kv heads to compute: all of them, or the listed subset (in that order)."""
    if kv_heads is None:
        return list(range(Hkv))
    sel = [int(g) for g in kv_heads]
    if any(g < 0 or g >= Hkv for g in sel):
        raise ValueError("kv_heads lists a head outside the pool")
    return sel


def gather_request_kv(k_pool, v_pool, req_to_token, row, length, k_scale=1.0, v_scale=1.0,
                      kv_heads=None):
    """Gather one request's keys and values by slot, as float64 ``[length, kv_heads, head_dim]``.

    The slot of the request's token ``j`` is ``req_to_token[row, j]``
    ("SGLang" notes, section "KV memory": request/position -> KV pool index ->
    KV tensors). Only the gathered rows are converted, never the whole pool.
    FP8 pools (uint8) hold ``scale * e4m3(byte)``: the scales multiply the decoded rows
    ("Inside SGLang", Step 6, per-tensor KV scales; 1.0 for bf16/fp32 pools).
    With ``kv_heads`` only those heads are gathered, in that order (axis 1).
    """
    S = k_pool.shape[0]
    if length < 0 or length > req_to_token.shape[1]:
        raise ValueError("context length exceeds the request table row")
    slots = np.asarray(req_to_token[row, :length], dtype=np.int64)
    if length and (slots.min() < 0 or slots.max() >= S):
        raise ValueError(f"request table row {row} names a slot outside the pool")
    if kv_heads is None:
        kb, vb = to_f64(k_pool[slots]), to_f64(v_pool[slots])
    else:
        sel = np.asarray(kv_heads, dtype=np.int64)[None, :]
        kb, vb = to_f64(k_pool[slots[:, None], sel]), to_f64(v_pool[slots[:, None], sel])
    if k_scale != 1.0:
        kb = kb * float(np.float32(k_scale))
    if v_scale != 1.0:
        vb = vb * float(np.float32(v_scale))
    return kb, vb


def causal_hidden(length: int, prefix: int, rows: np.ndarray) -> np.ndarray:
    """``[len(rows), length]`` mask of keys a suffix row may NOT see.

    Suffix row ``i`` sits at absolute position ``prefix + i`` and sees keys
    ``0 .. prefix + i`` (bottom-right causal alignment); later keys are hidden.
    """
    return np.arange(length)[None, :] > (prefix + rows)[:, None]


def _softmax_rows_times_v(scores: np.ndarray, v: np.ndarray) -> np.ndarray:
    """softmax over the last axis of ``scores`` (masked entries are -inf), then times ``v``."""
    m = scores.max(axis=-1, keepdims=True)
    p = np.exp(scores - m)
    p /= p.sum(axis=-1, keepdims=True)
    return p @ v


def extend_attention(q, k_pool, v_pool, req_to_token, req_pool_indices, prefix_lens,
                     extend_lens, extend_start_loc, n_kv_heads, sm_scale,
                     tokens=None, row_block=512, k_scale=1.0, v_scale=1.0, suffix=None,
                     kv_heads=None):
    """EXTEND attention: each request's new suffix rows over its prefix plus themselves.

    Follows "Origins: the paper and the first commit": self-test answer 2 (with
    a prefix cache only the missed suffix is computed, and attention reads the
    prefix's cached KV together with the KV just computed) and section
    "Batching: Req, Batch and the three forward modes" (the model input is the
    suffix only; seq_len = prefix + extend). The per-head arithmetic is the four
    steps of "Inside SGLang", Step 3.

    ``q`` is ``[total_extend_tokens, n_q_heads, head_dim]`` with requests back to
    back from ``extend_start_loc[b]``. All keys, suffix included, are read from
    the pool through ``req_to_token`` (so the suffix must already be stored).

    With ``suffix = (k_new, v_new)`` (each ``[total_extend_tokens, n_kv_heads,
    head_dim]``, rows in the order of ``q``) the keys and values of the suffix
    positions ``p .. p + e - 1`` are those rows instead of pool rows: the ragged
    reading of the same passages, where attention takes the prefix from the pool
    and the suffix straight from the just-computed K/V ("Origins...", self-test
    answer 2; "Inside SGLang", Step 3, a ragged kernel for the new tokens beside
    a paged one for the cached prefix). Only the first ``p`` entries of the
    request's table row are read then.

    Returns float64 ``[total_extend_tokens, n_q_heads, head_dim]``; with
    ``tokens`` (global row indices) only those rows are computed and returned in
    that order. With ``kv_heads`` only the query heads of those kv heads are
    computed; the other heads stay NaN.
    """
    S, Hkv, D = _check_pool(k_pool, v_pool)
    if Hkv != n_kv_heads:
        raise ValueError("pool kv-head count does not match n_kv_heads")
    N, Hq, Dq = q.shape
    if suffix is not None:
        if k_scale != 1.0 or v_scale != 1.0:
            raise ValueError("ragged suffix rows are taken with pools of the same element format")
        for a in suffix:
            if a.shape != (N, Hkv, D) or a.dtype != k_pool.dtype:
                raise ValueError(f"suffix rows must be [{N}, {Hkv}, {D}] in the pool's format")
    if Dq != D:
        raise ValueError("q head_dim does not match the pool")
    if Hq % Hkv:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    G = Hq // Hkv
    sel = _heads(kv_heads, Hkv)
    qf = to_f64(q)
    B = len(req_pool_indices)
    want = None
    if tokens is not None:
        want = {int(t): i for i, t in enumerate(tokens)}
        out = np.full((len(tokens), Hq, D), np.nan)
    else:
        out = np.full((N, Hq, D), np.nan)
    for b in range(B):
        r = int(req_pool_indices[b])
        p = int(prefix_lens[b])
        e = int(extend_lens[b])
        s0 = int(extend_start_loc[b])
        if p < 0 or e < 0 or s0 < 0 or s0 + e > N:
            raise ValueError(f"request {b}: inconsistent prefix/extend/start")
        if e == 0:
            continue
        L = p + e
        rows = np.arange(e)
        if want is not None:
            rows = np.array([i for i in range(e) if (s0 + i) in want], dtype=np.int64)
            if rows.size == 0:
                continue
        if suffix is None:
            kb, vb = gather_request_kv(k_pool, v_pool, req_to_token, r, L, k_scale, v_scale, sel)
        else:
            kp_, vp_ = gather_request_kv(k_pool, v_pool, req_to_token, r, p, k_scale, v_scale, sel)
            kb = np.concatenate([kp_, to_f64(suffix[0][s0:s0 + e][:, sel])])
            vb = np.concatenate([vp_, to_f64(suffix[1][s0:s0 + e][:, sel])])
        for c0 in range(0, rows.size, row_block):
            rb = rows[c0:c0 + row_block]
            masked = causal_hidden(L, p, rb)                       # [rows, L]
            for gi, g in enumerate(sel):
                heads = slice(g * G, (g + 1) * G)
                qg = qf[s0 + rb, heads, :].transpose(1, 0, 2)      # [G, rows, D]
                sc = (qg @ kb[:, gi, :].T) * sm_scale              # [G, rows, L]
                sc[:, masked] = -np.inf
                og = _softmax_rows_times_v(sc, vb[:, gi, :])       # [G, rows, D]
                og = og.transpose(1, 0, 2)                         # [rows, G, D]
                if want is None:
                    out[s0 + rb, heads, :] = og
                else:
                    for k, i in enumerate(rb):
                        out[want[s0 + int(i)], heads, :] = og[k]
    return out


def decode_attention(q, k_pool, v_pool, req_to_token, req_pool_indices, seq_lens,
                     n_kv_heads, sm_scale, requests=None, k_scale=1.0, v_scale=1.0, kv_heads=None):
    """DECODE attention: one query per request over positions 0 .. seq_len-1.

    Follows "Inside SGLang", Step 3, "Prefill and decode have different
    shapes": during decode each request has one new query, its score row is
    1 by n over every earlier token, and those keys and values are read
    ("Paged KV and the kernels that read it") from the slots the request's
    table row names. The current token's K/V is expected to be stored already
    ("Origins...", "Batching": one slot is allocated per request per decode
    step), so no mask applies.

    ``q`` is ``[batch, n_q_heads, head_dim]``. Returns float64 of the same shape
    (or only the listed ``requests``, in that order). With ``kv_heads`` only the
    query heads of those kv heads are computed; the other heads stay NaN.
    """
    S, Hkv, D = _check_pool(k_pool, v_pool)
    if Hkv != n_kv_heads:
        raise ValueError("pool kv-head count does not match n_kv_heads")
    B, Hq, Dq = q.shape
    if Dq != D or Hq % Hkv:
        raise ValueError("bad q shape")
    G = Hq // Hkv
    sel = _heads(kv_heads, Hkv)
    qf = to_f64(q)
    reqs = range(B) if requests is None else [int(b) for b in requests]
    out = np.full((len(reqs), Hq, D), np.nan)
    for k, b in enumerate(reqs):
        L = int(seq_lens[b])
        if L <= 0:
            raise ValueError(f"request {b}: a decode query needs at least one key")
        kb, vb = gather_request_kv(k_pool, v_pool, req_to_token, int(req_pool_indices[b]), L,
                                   k_scale, v_scale, sel)
        for gi, g in enumerate(sel):
            heads = slice(g * G, (g + 1) * G)
            sc = (qf[b, heads, :] @ kb[:, gi, :].T) * sm_scale     # [G, L]
            out[k, heads, :] = _softmax_rows_times_v(sc, vb[:, gi, :])
    return out
