"""Seeded generator: determinism, structure of the request table and pool, bf16 rounding."""

import numpy as np
import pytest

from prefix_cached_paged_amd import accounting as A
from prefix_cached_paged_amd import workloads as W


def test_same_seed_same_bytes_and_thread_independence(monkeypatch):
    spec = W.Spec("det", "bf16", 8, 2, 64, 50000, extend_prefix=(3000, 0), extend_lens=(700, 90),
                  decode_batch=6, decode_range=(10, 4000))
    a = W.make_workload(spec, 77)
    monkeypatch.setattr(W, "CHUNK", W.CHUNK)          # same chunking ...
    monkeypatch.setattr(W, "_threads", lambda: 1)     # ... but one thread
    b = W.make_workload(spec, 77)
    for x, y in [(a.k_pool, b.k_pool), (a.v_pool, b.v_pool), (a.req_to_token, b.req_to_token),
                 (a.k_new, b.k_new), (a.extend.q, b.extend.q), (a.decode.q, b.decode.q),
                 (a.decode.seq_lens, b.decode.seq_lens)]:
        assert np.array_equal(x, y)
    c = W.make_workload(spec, 78)
    assert not np.array_equal(a.decode.seq_lens, c.decode.seq_lens)


def test_round_to_bf16_ties_to_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 1.0 + 2 ** -8 + 2 ** -20],
                 dtype=np.float32)
    got = W.round_to_bf16_bits(x)
    # 1+2^-8 is halfway between 1.0 (0x3F80) and 1.0078125 (0x3F81): ties to even -> 0x3F80
    # 1+3*2^-8 is halfway between 0x3F81 and 0x3F82: ties to even -> 0x3F82
    assert list(got) == [0x3F80, 0x3F80, 0x3F82, 0x3F80, 0xC020, 0x3F81]


def test_request_table_structure():
    spec = W.Spec("struct", "bf16", 4, 2, 8, 4096, extend_prefix=(100, 100, 100), extend_lens=(5, 0, 9),
                  shared_prefix=True, decode_lens=(1, 50))
    wl = W.make_workload(spec, 3)
    e, d = wl.extend, wl.decode
    rows = list(e.req_pool_indices) + list(d.req_pool_indices)
    assert len(set(rows)) == len(rows)
    spare = sorted(set(range(wl.req_to_token.shape[0])) - set(rows))
    assert len(spare) == spec.spare_rows
    assert np.all(wl.req_to_token[spare] == -1)
    # shared prefix: identical leading slots
    pre = wl.req_to_token[e.req_pool_indices[0], :100]
    for r in e.req_pool_indices[1:]:
        assert np.array_equal(wl.req_to_token[r, :100], pre)
    # every other referenced slot is used once
    refs = [pre]
    for b, r in enumerate(e.req_pool_indices):
        refs.append(wl.req_to_token[r, 100:100 + e.extend_lens[b]])
        assert np.all(wl.req_to_token[r, 100 + e.extend_lens[b]:] == -1)
    for b, r in enumerate(d.req_pool_indices):
        refs.append(wl.req_to_token[r, :d.seq_lens[b]])
    allref = np.concatenate(refs)
    assert len(np.unique(allref)) == allref.size
    # store rows are the suffixes then the decode current tokens
    want_loc = np.concatenate([wl.req_to_token[r, 100:100 + e.extend_lens[b]] for b, r in enumerate(e.req_pool_indices)]
                              + [[wl.req_to_token[r, d.seq_lens[b] - 1]] for b, r in enumerate(d.req_pool_indices)])
    assert np.array_equal(wl.store_loc, want_loc)
    # unreferenced and not-yet-stored slots are NaN in the pre-store pool
    ctx = np.setdiff1d(allref, wl.store_loc)
    nan = np.ones(4096, bool)
    nan[ctx] = False
    assert np.all(wl.k_pool[nan] == W.BF16_NAN) and np.all(wl.v_pool[nan] == W.BF16_NAN)
    assert not np.any(wl.k_pool[ctx] == W.BF16_NAN)
    assert np.array_equal(e.extend_start_loc, [0, 5, 5])


def test_values_have_the_configured_spread():
    spec = W.Spec("sigma", "fp32", 4, 2, 128, 20000, sigma=0.5, decode_lens=(10000,))
    wl = W.make_workload(spec, 4)
    used = wl.req_to_token[wl.decode.req_pool_indices[0], :9999]
    k = wl.k_pool[used]
    assert abs(k.std() - 0.5) < 0.01 and abs(k.mean()) < 0.01


def test_peaked_variant_scales_q():
    spec = W.Spec("pk", "fp32", 2, 2, 8, 64, decode_lens=(5,))
    a = W.make_workload(spec, 9)
    b = W.make_workload(spec, 9, variant="peaked")
    np.testing.assert_allclose(b.decode.q, a.decode.q * 8, rtol=1e-6)


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_config_shapes(cfg):
    """Small configs are drawn in full; their shapes and work match the stated configs."""
    spec = W.CONFIGS[cfg]
    wl = W.make_workload(spec, W.TIMING_SEEDS[cfg])
    assert wl.k_pool.shape == (spec.num_slots, spec.n_kv_heads, spec.head_dim)
    if cfg == 1:
        assert wl.k_pool.dtype == np.float32
        assert wl.extend.q.shape == (57, 4, 64)
        assert A.extend_pairs(wl.extend.prefix_lens, wl.extend.extend_lens) == 1597
        assert np.count_nonzero(~np.isnan(wl.k_pool[:, 0, 0])) == 265 - 57
    if cfg == 2:
        assert wl.decode.q.shape == (64, 32, 128)
        assert wl.decode.seq_lens.min() >= 512 and wl.decode.seq_lens.max() <= 4096
    if cfg == 3:
        assert wl.extend.q.shape == (8192, 32, 128)
        assert A.extend_pairs(wl.extend.prefix_lens, wl.extend.extend_lens) == 34_607_104
        assert wl.store_loc.size == 8192


def test_pair_count_matches_brute_force_count():
    p = [0, 3, 17, 5]
    e = [4, 1, 0, 9]
    brute = sum(sum(1 for i in range(ee) for j in range(pp + ee) if j <= pp + i) for pp, ee in zip(p, e))
    assert A.extend_pairs(p, e) == brute
    assert A.extend_flops(p, e, 3, 16) == brute * 4 * 16 * 3
