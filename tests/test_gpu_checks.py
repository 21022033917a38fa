"""Debug checks of the device-side contracts (rax_check_*), on the GPU.

Seeded workloads satisfy every contract, so their counts must all be zero. Contract breaks are
then planted in copies of the index arrays on the host (out-of-pool slots and pages, repeated
and out-of-range store slots, bad lengths, bad request rows, prefix slots the ragged call also
stores to) and the counts are compared with a plain Python reading of the contracts as the
header states them. Only the check calls see the planted arrays; no attention or store call
is given them.
"""

import numpy as np
import pytest
import torch

from prefix_cached_paged_amd import rax as R
from prefix_cached_paged_amd import workloads as W
from prefix_cached_paged_amd.device import to_dev

from parity import say

pytestmark = pytest.mark.gpu

ZERO = dict.fromkeys(R.CHECK_ITEMS, 0)


def expect_store(loc, S):
    c = dict(ZERO)
    seen = set()
    for x in np.asarray(loc).tolist():
        if x < 0 or x >= S:
            c["slot"] += 1
        elif x in seen:
            c["duplicate"] += 1
        else:
            seen.add(x)
    return c, seen


def expect_requests(table, P, rpi, lens, S, max_seq, ext=None, ragged=False, stored=frozenset()):
    """ext = (extend_lens, extend_start_loc, total_tokens, max_extend_len) for EXTEND."""
    c = dict(ZERO)
    rows = table.shape[0]
    for b in range(len(rpi)):
        if ext is not None:
            e_lens, starts, total, max_ext = ext
            p, e, s = int(lens[b]), int(e_lens[b]), int(starts[b])
            if p < 0 or e < 0 or e > max_ext or p + e > max_seq or s < 0 or s + e > total:
                c["length"] += 1
                continue
            L = p if ragged else p + e
            if e <= 0 or L <= 0:
                continue
        else:
            L = int(lens[b])
            if L > max_seq:
                c["length"] += 1
                continue
            if L <= 0:
                continue
        r = int(rpi[b])
        if r < 0 or r >= rows:
            c["row"] += 1
            continue
        j = np.arange(L)
        entry = table[r, j // P].astype(np.int64)
        bad = (entry < 0) | ((entry + 1) * P > S)
        c["slot"] += int(bad.sum())
        if stored:
            slots = (entry * P + j % P)[~bad]
            c["overlap"] += sum(1 for x in slots.tolist() if x in stored)
    return c


def run_extend(table, P, e_arrays, total, max_ext, max_seq, S, ragged=False, store_loc=None):
    rpi, p, e, s = (to_dev(np.ascontiguousarray(a, np.int32)) for a in e_arrays)
    return R.check_extend(to_dev(np.ascontiguousarray(table, np.int32)), rpi, p, e, s, total, max_ext, max_seq, S,
                          page_size=P, ragged=ragged,
                          store_loc=None if store_loc is None else to_dev(np.ascontiguousarray(store_loc, np.int32)))


def run_decode(table, P, rpi, seq, max_seq, S):
    return R.check_decode(to_dev(np.ascontiguousarray(table, np.int32)), to_dev(np.asarray(rpi, np.int32)),
                          to_dev(np.asarray(seq, np.int32)), max_seq, S, page_size=P)


SPEC = W.Spec("chk", "bf16", 32, 8, 128, 20000, extend_prefix=(100, 40, 7, 300, 0), extend_lens=(50, 20, 9, 64, 30),
              decode_lens=(30, 500, 1000, 1))


@pytest.mark.parametrize("page_size", [1, 16])
def test_seeded_workloads_break_nothing(page_size):
    import dataclasses
    spec = dataclasses.replace(SPEC, page_size=page_size)
    wl = W.make_workload(spec, 1201)
    e, d = wl.extend, wl.decode
    n = e.total_tokens
    S = spec.num_slots
    table = wl.page_table if page_size > 1 else wl.req_to_token
    say(f"checks on a seeded workload, page size {page_size}")
    assert R.check_kv_store(to_dev(wl.store_loc), S) == ZERO
    arrays = (e.req_pool_indices, e.prefix_lens, e.extend_lens, e.extend_start_loc)
    assert run_extend(table, page_size, arrays, n, e.max_extend_len, e.max_seq_len, S) == ZERO
    assert run_extend(table, page_size, arrays, n, e.max_extend_len, e.max_seq_len, S, ragged=True,
                      store_loc=wl.store_loc[:n]) == ZERO
    assert run_decode(table, page_size, d.req_pool_indices, d.seq_lens, d.max_seq_len, S) == ZERO


def test_planted_breaks_are_counted():
    wl = W.make_workload(SPEC, 1202)
    e, d = wl.extend, wl.decode
    n = e.total_tokens
    S = SPEC.num_slots
    rows = wl.req_to_token.shape[0]

    # kv_store: two slots outside the pool, two repeats
    loc = wl.store_loc.copy()
    loc[3], loc[5] = -1, S
    loc[8] = loc[9] = loc[7]
    want, _ = expect_store(loc, S)
    assert want["slot"] == 2 and want["duplicate"] == 2
    say("planted store breaks")
    assert R.check_kv_store(to_dev(loc), S) == want

    # EXTEND: two bad slots in request 0's row, a length break (request 1), a bad row (request 2)
    table = wl.req_to_token.copy()
    rpi, p, el, st = (a.copy() for a in (e.req_pool_indices, e.prefix_lens, e.extend_lens, e.extend_start_loc))
    max_seq, max_ext = e.max_seq_len, e.max_extend_len
    table[rpi[0], 2] = S + 5
    table[rpi[0], 4] = -3
    p[1] = max_seq
    rpi[2] = rows
    ext = (el, st, n, max_ext)
    want = expect_requests(table, 1, rpi, p, S, max_seq, ext)
    assert want["slot"] == 2 and want["length"] == 1 and want["row"] == 1, want
    say("planted EXTEND breaks")
    got = run_extend(table, 1, (rpi, p, el, st), n, max_ext, max_seq, S)
    assert got == want, (got, want)

    # ragged with a store: one stored slot is one of request 3's prefix slots, one repeat
    store = wl.store_loc[:n].copy()
    store[0] = table[rpi[3], 0]
    store[2] = store[1]
    sw, stored = expect_store(store, S)
    want = expect_requests(table, 1, rpi, p, S, max_seq, ext, ragged=True, stored=stored)
    for k in ("slot", "duplicate"):
        want[k] += sw[k]
    assert want["overlap"] >= 1 and want["duplicate"] == 1, want
    say("planted ragged-store breaks")
    got = run_extend(table, 1, (rpi, p, el, st), n, max_ext, max_seq, S, ragged=True, store_loc=store)
    assert got == want, (got, want)

    # DECODE: a length past max_seq_len, a bad row, out-of-pool slots in request 2's row
    table = wl.req_to_token.copy()
    drpi, seq = d.req_pool_indices.copy(), d.seq_lens.copy()
    max_seq = d.max_seq_len
    seq[0] = max_seq + 1
    drpi[1] = -1
    table[drpi[2], 10:20] = S
    want = expect_requests(table, 1, drpi, seq, S, max_seq)
    assert want["length"] == 1 and want["row"] == 1 and want["slot"] == 10, want
    say("planted DECODE breaks")
    assert run_decode(table, 1, drpi, seq, max_seq, S) == want


def test_planted_page_breaks_are_counted():
    import dataclasses
    P = 16
    spec = dataclasses.replace(SPEC, page_size=P)
    wl = W.make_workload(spec, 1203)
    e, d = wl.extend, wl.decode
    S = spec.num_slots
    pt = wl.page_table.copy()
    pt[e.req_pool_indices[0], 0] = -1           # request 0: positions 0..15 bad
    pt[e.req_pool_indices[3], 2] = S // P       # request 3: a page just past the pool
    arrays = (e.req_pool_indices, e.prefix_lens, e.extend_lens, e.extend_start_loc)
    want = expect_requests(pt, P, e.req_pool_indices, e.prefix_lens, S, e.max_seq_len,
                           (e.extend_lens, e.extend_start_loc, e.total_tokens, e.max_extend_len))
    assert want["slot"] == 2 * P, want
    say("planted page breaks")
    got = run_extend(pt, P, arrays, e.total_tokens, e.max_extend_len, e.max_seq_len, S)
    assert got == want, (got, want)
    want = expect_requests(pt, P, d.req_pool_indices, d.seq_lens, S, d.max_seq_len)
    assert run_decode(pt, P, d.req_pool_indices, d.seq_lens, d.max_seq_len, S) == want


def test_empty_calls_zero_the_counts():
    S = 1000
    table = to_dev(np.zeros((2, 64), np.int32))
    none = to_dev(np.zeros(0, np.int32))
    say("empty checks")
    assert R.check_kv_store(none, S) == ZERO
    assert R.check_extend(table, none, none, none, none, 0, 0, 0, S) == ZERO
    assert R.check_decode(table, none, none, 0, S) == ZERO
    # counts the caller left non-zero are overwritten
    counts = torch.full((len(R.CHECK_ITEMS),), 7, dtype=torch.int32, device="cuda")
    rc = R.load().rax_check_decode(table.data_ptr(), 2, 64, 1, None, None, 0, 0, S, counts.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream)
    assert rc == 0 and counts.tolist() == [0] * len(R.CHECK_ITEMS)
