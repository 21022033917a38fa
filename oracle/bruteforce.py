"""Loop-only attention for tiny inputs: a second, independent statement of the definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Pure Python scalar loops with ``math.exp``: no numpy matmul, no vectorised
softmax. Each query row, head by head, walks its visible keys one by one
("Inside SGLang", Step 3: scores, scale, causal mask, softmax, times V). The
vectorised oracle must agree with this to rounding on every tiny case.
"""

from __future__ import annotations

import math

from .formats import to_f64


def _row(qv, keys, vals, scale):
    scores = [scale * sum(a * b for a, b in zip(qv, k)) for k in keys]
    top = max(scores)
    w = [math.exp(s - top) for s in scores]
    z = sum(w)
    D = len(vals[0])
    return [sum(w[j] * vals[j][d] for j in range(len(vals))) / z for d in range(D)]


def extend_attention_loops(q, k_pool, v_pool, req_to_token, req_pool_indices, prefix_lens,
                           extend_lens, extend_start_loc, n_kv_heads, sm_scale):
    """Nested-loop EXTEND attention; returns a list ``out[token][head][d]``."""
    qf = to_f64(q).tolist()
    kf = k_pool
    vf = v_pool
    N, Hq, D = len(qf), len(qf[0]), len(qf[0][0])
    G = Hq // n_kv_heads
    out = [[[float("nan")] * D for _ in range(Hq)] for _ in range(N)]
    for b in range(len(req_pool_indices)):
        r = int(req_pool_indices[b])
        p, e, s0 = int(prefix_lens[b]), int(extend_lens[b]), int(extend_start_loc[b])
        for i in range(e):
            pos = p + i
            slots = [int(req_to_token[r][j]) for j in range(pos + 1)]
            for h in range(Hq):
                g = h // G
                keys = [to_f64(kf[s, g]).tolist() for s in slots]
                vals = [to_f64(vf[s, g]).tolist() for s in slots]
                out[s0 + i][h] = _row(qf[s0 + i][h], keys, vals, sm_scale)
    return out


def decode_attention_loops(q, k_pool, v_pool, req_to_token, req_pool_indices, seq_lens,
                           n_kv_heads, sm_scale):
    """Nested-loop DECODE attention; returns a list ``out[request][head][d]``."""
    qf = to_f64(q).tolist()
    B, Hq = len(qf), len(qf[0])
    G = Hq // n_kv_heads
    out = []
    for b in range(B):
        r = int(req_pool_indices[b])
        slots = [int(req_to_token[r][j]) for j in range(int(seq_lens[b]))]
        rows = []
        for h in range(Hq):
            g = h // G
            keys = [to_f64(k_pool[s, g]).tolist() for s in slots]
            vals = [to_f64(v_pool[s, g]).tolist() for s in slots]
            rows.append(_row(qf[b][h], keys, vals, sm_scale))
        out.append(rows)
    return out
