"""Pins of the oracle's page-granular tables (page size P > 1).

* hand-worked slot tables (tests/golden/paged_slots.json);
* the workload generator, which places positions in pages with code of its own, names the
  same slots token by token;
* attention over a page table equals the loop-only brute force over the same slots.
"""

import json
import os

import numpy as np
import pytest

import oracle
from prefix_cached_paged_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "paged_slots.json")


def test_golden_slot_tables():
    for c in json.load(open(GOLDEN))["cases"]:
        got = oracle.token_table(np.array(c["page_table"]), c["page_size"], c["width"])
        assert got.tolist() == c["slots"], c


def test_page_size_one_is_the_token_table():
    pt = np.random.default_rng(3).integers(0, 1000, (5, 40))
    assert np.array_equal(oracle.token_table(pt, 1, 40), pt)


SPECS = [
    W.Spec("pg-ext", "bf16", 8, 2, 16, 4096, extend_prefix=(0, 37, 64, 5), extend_lens=(20, 30, 1, 60),
           decode_lens=(1, 17, 100, 64), page_size=16),
    W.Spec("pg-shared", "fp32", 4, 4, 8, 2048, extend_prefix=(32,) * 3, extend_lens=(5, 1, 40), shared_prefix=True,
           decode_lens=(33,), page_size=8),
    W.Spec("pg-big", "bf16", 4, 1, 8, 8192, extend_prefix=(200,), extend_lens=(70,), decode_lens=(300, 2), page_size=64),
]


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: s.name)
def test_generator_pages_match_token_table(spec):
    wl = W.make_workload(spec, 21)
    P = spec.page_size
    table = oracle.token_table(wl.page_table, P, wl.req_to_token.shape[1])
    rows = list(wl.extend.req_pool_indices) + list(wl.decode.req_pool_indices)
    lens = list(wl.extend.prefix_lens + wl.extend.extend_lens) + list(wl.decode.seq_lens)
    for r, L in zip(rows, lens):
        assert np.array_equal(table[r, :L], wl.req_to_token[r, :L])
        assert np.all(table[r, :L] // P == np.repeat(wl.page_table[r, :(L + P - 1) // P], P)[:L])


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: s.name)
def test_paged_attention_matches_loops(spec):
    wl = W.make_workload(spec, 22)
    kp, vp = oracle.kv_store(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.store_loc)
    e, d = wl.extend, wl.decode
    got = oracle.extend_attention_paged(e.q, kp, vp, wl.page_table, spec.page_size, e.req_pool_indices,
                                        e.prefix_lens, e.extend_lens, e.extend_start_loc, spec.n_kv_heads,
                                        wl.sm_scale)
    ref = oracle.extend_attention_loops(e.q, kp, vp, wl.req_to_token, e.req_pool_indices, e.prefix_lens,
                                        e.extend_lens, e.extend_start_loc, spec.n_kv_heads, wl.sm_scale)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    got = oracle.decode_attention_paged(d.q, kp, vp, wl.page_table, spec.page_size, d.req_pool_indices,
                                        d.seq_lens, spec.n_kv_heads, wl.sm_scale)
    ref = oracle.decode_attention_loops(d.q, kp, vp, wl.req_to_token, d.req_pool_indices, d.seq_lens,
                                        spec.n_kv_heads, wl.sm_scale)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
