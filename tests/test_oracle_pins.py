"""Pins of the CPU oracle against things other than itself.

* brute force: pure-Python loops with math.exp on tiny inputs;
* a library routine: torch's scaled_dot_product_attention in float64 with the
  lower-right causal bias and enable_gqa, on the dense rows gathered by hand;
* closed forms: a single key returns its V exactly, identical keys give the mean
  of the visible V rows, a needle key returns its V;
* invariants: slot relabelling, prefix-extend = tail of full prefill, GQA =
  repeat-interleaved MHA, EXTEND with one new token = DECODE;
* the constants the pages print (tests/golden/pages_constants.json).

A plausible mistake in the oracle (a dropped term, a wrong mask offset, a wrong
kv-head index, a transposed operand) fails at least one of these; the planted
mistake tests at the end check exactly that, on the CPU.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from torch.nn.attention.bias import causal_lower_right

import oracle
from oracle import attention as oatt
from prefix_cached_paged_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")

TINY_SPECS = [
    W.Spec("t-mha", "fp32", 2, 2, 8, 96, extend_prefix=(0, 5, 9), extend_lens=(7, 3, 1)),
    W.Spec("t-gqa2", "bf16", 4, 2, 8, 128, extend_prefix=(3, 0), extend_lens=(6, 4),
           decode_lens=(1, 4, 11)),
    W.Spec("t-gqa3", "fp32", 6, 2, 4, 128, extend_prefix=(12,), extend_lens=(5,),
           decode_lens=(7, 2)),
    W.Spec("t-mqa", "bf16", 4, 1, 8, 128, extend_prefix=(4, 4, 4), extend_lens=(2, 5, 0),
           shared_prefix=True, decode_lens=(19,)),
    W.Spec("t-empty-ext", "fp32", 3, 3, 4, 64, extend_prefix=(2, 0), extend_lens=(0, 3)),
]


def stored(wl):
    """Pools after the new rows are written (oracle kv_store)."""
    return oracle.kv_store(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.store_loc)


def run_extend(wl, kp, vp, **kw):
    e = wl.extend
    return oracle.extend_attention(e.q, kp, vp, wl.req_to_token, e.req_pool_indices, e.prefix_lens,
                                   e.extend_lens, e.extend_start_loc, wl.spec.n_kv_heads,
                                   wl.sm_scale, **kw)


def run_decode(wl, kp, vp, **kw):
    d = wl.decode
    return oracle.decode_attention(d.q, kp, vp, wl.req_to_token, d.req_pool_indices, d.seq_lens,
                                   wl.spec.n_kv_heads, wl.sm_scale, **kw)


# --------------------------------------------------------------------------- brute force

@pytest.mark.parametrize("spec", TINY_SPECS, ids=lambda s: s.name)
@pytest.mark.parametrize("seed", [11, 12])
def test_extend_matches_loops(spec, seed):
    wl = W.make_workload(spec, seed)
    if wl.extend is None:
        pytest.skip("no extend part")
    kp, vp = stored(wl)
    got = run_extend(wl, kp, vp)
    e = wl.extend
    ref = np.array(oracle.extend_attention_loops(e.q, kp, vp, wl.req_to_token, e.req_pool_indices,
                                                 e.prefix_lens, e.extend_lens, e.extend_start_loc,
                                                 spec.n_kv_heads, wl.sm_scale))
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("spec", [s for s in TINY_SPECS if s.decode_lens], ids=lambda s: s.name)
@pytest.mark.parametrize("seed", [21, 22])
def test_decode_matches_loops(spec, seed):
    wl = W.make_workload(spec, seed)
    kp, vp = stored(wl)
    got = run_decode(wl, kp, vp)
    d = wl.decode
    ref = np.array(oracle.decode_attention_loops(d.q, kp, vp, wl.req_to_token, d.req_pool_indices,
                                                 d.seq_lens, spec.n_kv_heads, wl.sm_scale))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- library routine

def _sdpa_request(q_rows, kb, vb, p, scale):
    """torch float64 SDPA for one request: q_rows [e, Hq, D], kb/vb [L, Hkv, D]."""
    qt = torch.from_numpy(q_rows).permute(1, 0, 2)[None]          # [1, Hq, e, D]
    kt = torch.from_numpy(kb).permute(1, 0, 2)[None]              # [1, Hkv, L, D]
    vt = torch.from_numpy(vb).permute(1, 0, 2)[None]
    e, L = q_rows.shape[0], kb.shape[0]
    mask = causal_lower_right(e, L) if p is not None else None
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale, enable_gqa=True)
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("seed", [31, 32, 33])
def test_extend_matches_torch_sdpa_lower_right(seed):
    spec = W.Spec("sdpa", "bf16", 8, 2, 16, 2048, extend_prefix=(0, 1, 40, 300),
                  extend_lens=(50, 33, 1, 64))
    wl = W.make_workload(spec, seed)
    kp, vp = stored(wl)
    got = run_extend(wl, kp, vp)
    e = wl.extend
    qf = oracle.to_f64(e.q)
    for b in range(e.batch):
        p, n, s0 = int(e.prefix_lens[b]), int(e.extend_lens[b]), int(e.extend_start_loc[b])
        kb, vb = oracle.gather_request_kv(kp, vp, wl.req_to_token, int(e.req_pool_indices[b]), p + n)
        ref = _sdpa_request(qf[s0:s0 + n], kb, vb, p, wl.sm_scale)
        np.testing.assert_allclose(got[s0:s0 + n], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", [41, 42])
def test_decode_matches_torch_sdpa(seed):
    spec = W.Spec("sdpa-dec", "bf16", 8, 2, 16, 4096, decode_lens=(1, 2, 77, 1000))
    wl = W.make_workload(spec, seed)
    kp, vp = stored(wl)
    got = run_decode(wl, kp, vp)
    d = wl.decode
    qf = oracle.to_f64(d.q)
    for b in range(d.batch):
        kb, vb = oracle.gather_request_kv(kp, vp, wl.req_to_token, int(d.req_pool_indices[b]),
                                          int(d.seq_lens[b]))
        ref = _sdpa_request(qf[b:b + 1], kb, vb, None, wl.sm_scale)
        np.testing.assert_allclose(got[b:b + 1], ref, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- closed forms

def test_single_key_returns_its_value_exactly():
    spec = W.Spec("one", "bf16", 4, 2, 8, 64, extend_prefix=(0,), extend_lens=(1,), decode_lens=(1,))
    wl = W.make_workload(spec, 5)
    kp, vp = stored(wl)
    o_e = run_extend(wl, kp, vp)
    o_d = run_decode(wl, kp, vp)
    G = spec.n_q_heads // spec.n_kv_heads
    for h in range(spec.n_q_heads):
        slot_e = wl.req_to_token[wl.extend.req_pool_indices[0], 0]
        slot_d = wl.req_to_token[wl.decode.req_pool_indices[0], 0]
        assert np.array_equal(o_e[0, h], oracle.to_f64(vp[slot_e, h // G]))
        assert np.array_equal(o_d[0, h], oracle.to_f64(vp[slot_d, h // G]))


def test_identical_keys_give_running_mean_of_values():
    spec = W.Spec("same-k", "fp32", 2, 1, 8, 256, extend_prefix=(7,), extend_lens=(9,), decode_lens=(13,))
    wl = W.make_workload(spec, 6)
    kp, vp = stored(wl)
    kp = kp.copy()
    ref_row = kp[wl.req_to_token[wl.extend.req_pool_indices[0], 0]].copy()
    used = wl.req_to_token[wl.req_to_token >= 0]
    kp[used] = ref_row
    o = run_extend(wl, kp, vp)
    e = wl.extend
    r = e.req_pool_indices[0]
    vals = oracle.to_f64(vp[wl.req_to_token[r, :16], 0])
    for i in range(9):
        want = vals[:7 + i + 1].mean(axis=0)
        np.testing.assert_allclose(o[i, 0], want, rtol=0, atol=1e-14)
        np.testing.assert_allclose(o[i, 1], want, rtol=0, atol=1e-14)
    od = run_decode(wl, kp, vp)
    rd = wl.decode.req_pool_indices[0]
    np.testing.assert_allclose(od[0, 0], oracle.to_f64(vp[wl.req_to_token[rd, :13], 0]).mean(axis=0),
                               rtol=0, atol=1e-14)


def test_needle_returns_its_value():
    spec = W.Spec("needle", "bf16", 8, 2, 64, 8192, extend_prefix=(500, 0), extend_lens=(20, 30),
                  decode_lens=(3000, 5))
    wl = W.make_workload(spec, 7, variant="needle")
    kp, vp = stored(wl)
    G = 4
    o_e = run_extend(wl, kp, vp)
    e = wl.extend
    for b in range(e.batch):
        for g in range(2):
            pos = wl.needles[("extend", b, g)]
            v = oracle.to_f64(vp[wl.req_to_token[e.req_pool_indices[b], pos], g])
            rows = o_e[e.extend_start_loc[b]:e.extend_start_loc[b] + e.extend_lens[b], g * G:(g + 1) * G]
            np.testing.assert_allclose(rows, np.broadcast_to(v, rows.shape), rtol=0, atol=1e-6)
    o_d = run_decode(wl, kp, vp)
    d = wl.decode
    for b in range(d.batch):
        for g in range(2):
            pos = wl.needles[("decode", b, g)]
            v = oracle.to_f64(vp[wl.req_to_token[d.req_pool_indices[b], pos], g])
            np.testing.assert_allclose(o_d[b, g * G:(g + 1) * G], np.broadcast_to(v, (G, 64)), rtol=0, atol=1e-6)


# --------------------------------------------------------------------------- invariants

def _relabel_slots(wl, kp, vp, seed):
    """Move every pool row to a new slot and rewrite the request table to match."""
    S = kp.shape[0]
    perm = np.random.default_rng(seed).permutation(S)       # old slot s -> new slot perm[s]
    kq = np.empty_like(kp)
    vq = np.empty_like(vp)
    kq[perm] = kp
    vq[perm] = vp
    r2t = wl.req_to_token.copy()
    m = r2t >= 0
    r2t[m] = perm[r2t[m]]
    return kq, vq, r2t


@pytest.mark.parametrize("spec", TINY_SPECS[:4], ids=lambda s: s.name)
def test_slot_relabelling_is_exact(spec):
    wl = W.make_workload(spec, 8)
    kp, vp = stored(wl)
    kq, vq, r2t = _relabel_slots(wl, kp, vp, 99)
    if wl.extend is not None:
        a = run_extend(wl, kp, vp)
        e = wl.extend
        b = oracle.extend_attention(e.q, kq, vq, r2t, e.req_pool_indices, e.prefix_lens, e.extend_lens,
                                    e.extend_start_loc, spec.n_kv_heads, wl.sm_scale)
        assert np.array_equal(a, b, equal_nan=True)
    if wl.decode is not None:
        d = wl.decode
        a = run_decode(wl, kp, vp)
        b = oracle.decode_attention(d.q, kq, vq, r2t, d.req_pool_indices, d.seq_lens, spec.n_kv_heads,
                                    wl.sm_scale)
        assert np.array_equal(a, b)


def test_prefix_extend_equals_tail_of_full_prefill():
    spec = W.Spec("tail", "bf16", 4, 2, 16, 1024, extend_prefix=(90,), extend_lens=(40,))
    wl = W.make_workload(spec, 9)
    kp, vp = stored(wl)
    part = run_extend(wl, kp, vp)
    e = wl.extend
    # the same 130 tokens as one prefill: prefix 0, extend 130, q = [unknown 90 rows | the 40 rows]
    q_full = np.concatenate([np.zeros((90, 4, 16), dtype=e.q.dtype), e.q])
    full = oracle.extend_attention(q_full, kp, vp, wl.req_to_token, e.req_pool_indices,
                                   np.array([0]), np.array([130]), np.array([0]), 2, wl.sm_scale)
    np.testing.assert_allclose(part, full[90:], rtol=0, atol=1e-14)


@pytest.mark.parametrize("G", [2, 4])
def test_gqa_equals_repeat_interleaved_mha(G):
    spec = W.Spec("gqa", "bf16", 2 * G, 2, 8, 512, extend_prefix=(10, 3), extend_lens=(5, 8),
                  decode_lens=(17,))
    wl = W.make_workload(spec, 10)
    kp, vp = stored(wl)
    k_mha = np.repeat(kp, G, axis=1)
    v_mha = np.repeat(vp, G, axis=1)
    e, d = wl.extend, wl.decode
    a = run_extend(wl, kp, vp)
    b = oracle.extend_attention(e.q, k_mha, v_mha, wl.req_to_token, e.req_pool_indices, e.prefix_lens,
                                e.extend_lens, e.extend_start_loc, 2 * G, wl.sm_scale)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)
    a = run_decode(wl, kp, vp)
    b = oracle.decode_attention(d.q, k_mha, v_mha, wl.req_to_token, d.req_pool_indices, d.seq_lens,
                                2 * G, wl.sm_scale)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)


def test_extend_one_token_equals_decode():
    spec = W.Spec("e1", "fp32", 4, 2, 8, 512, extend_prefix=(37,), extend_lens=(1,))
    wl = W.make_workload(spec, 11)
    kp, vp = stored(wl)
    e = wl.extend
    a = run_extend(wl, kp, vp)
    b = oracle.decode_attention(e.q, kp, vp, wl.req_to_token, e.req_pool_indices, np.array([38]), 2,
                                wl.sm_scale)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)


def test_subset_rows_match_full():
    spec = W.Spec("sub", "bf16", 4, 2, 8, 2048, extend_prefix=(5, 60), extend_lens=(30, 70),
                  decode_lens=(9, 40, 3))
    wl = W.make_workload(spec, 12)
    kp, vp = stored(wl)
    full = run_extend(wl, kp, vp)
    tok = [99, 0, 31, 45]
    np.testing.assert_allclose(run_extend(wl, kp, vp, tokens=tok), full[tok], rtol=0, atol=1e-15)
    fd = run_decode(wl, kp, vp)
    np.testing.assert_allclose(run_decode(wl, kp, vp, requests=[2, 0]), fd[[2, 0]], rtol=0, atol=1e-15)


# --------------------------------------------------------------------------- kv_store

def test_kv_store_changes_exactly_the_named_rows():
    spec = W.Spec("store", "bf16", 4, 2, 8, 256, extend_prefix=(20,), extend_lens=(17,), decode_lens=(5, 9))
    wl = W.make_workload(spec, 13)
    kp, vp = stored(wl)
    touched = np.zeros(256, bool)
    touched[wl.store_loc] = True
    assert np.array_equal(kp[~touched], wl.k_pool[~touched])
    assert np.array_equal(vp[~touched], wl.v_pool[~touched])
    assert np.array_equal(kp[wl.store_loc], wl.k_new)
    assert np.array_equal(vp[wl.store_loc], wl.v_new)


def test_kv_store_rejects_bad_locations():
    spec = W.Spec("store2", "fp32", 2, 2, 4, 32, extend_prefix=(0,), extend_lens=(4,))
    wl = W.make_workload(spec, 14)
    with pytest.raises(ValueError):
        oracle.kv_store(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, None)
    bad = wl.store_loc.copy()
    bad[1] = bad[0]
    with pytest.raises(ValueError):
        oracle.kv_store(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, bad)
    bad = wl.store_loc.copy()
    bad[0] = 32
    with pytest.raises(ValueError):
        oracle.kv_store(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, bad)


def test_decode_rejects_empty_context():
    spec = W.Spec("dec0", "fp32", 2, 2, 4, 32, decode_lens=(3,))
    wl = W.make_workload(spec, 15)
    kp, vp = stored(wl)
    with pytest.raises(ValueError):
        oracle.decode_attention(wl.decode.q, kp, vp, wl.req_to_token, wl.decode.req_pool_indices,
                                np.array([0]), 2, wl.sm_scale)


def test_unstored_suffix_poisons_output():
    """Keys are read from the pool: skipping the store leaves NaN rows visible."""
    spec = W.Spec("nan", "bf16", 2, 2, 4, 64, extend_prefix=(3,), extend_lens=(2,))
    wl = W.make_workload(spec, 16)
    o = run_extend(wl, wl.k_pool, wl.v_pool)
    assert np.all(np.isnan(o))


def _suffix_rows(wl):
    """The step's new rows that belong to the EXTEND suffixes (they come first, in q's order)."""
    n = wl.extend.total_tokens
    return wl.k_new[:n], wl.v_new[:n]


@pytest.mark.parametrize("seed", [35, 36])
def test_ragged_suffix_matches_torch_sdpa(seed):
    """Suffix keys taken from the new rows (pool suffix slots left NaN): torch's attention over
    the prefix rows gathered by hand plus the new rows."""
    spec = W.Spec("ragged", "bf16", 8, 2, 16, 2048, extend_prefix=(0, 1, 40, 300),
                  extend_lens=(50, 33, 1, 64))
    wl = W.make_workload(spec, seed)
    kn, vn = _suffix_rows(wl)
    got = run_extend(wl, wl.k_pool, wl.v_pool, suffix=(kn, vn))
    e = wl.extend
    qf = oracle.to_f64(e.q)
    assert np.all(np.isfinite(got))
    for b in range(e.batch):
        p, n, s0 = int(e.prefix_lens[b]), int(e.extend_lens[b]), int(e.extend_start_loc[b])
        slots = wl.req_to_token[int(e.req_pool_indices[b]), :p]
        kb = np.concatenate([oracle.to_f64(wl.k_pool[slots]), oracle.to_f64(kn[s0:s0 + n])])
        vb = np.concatenate([oracle.to_f64(wl.v_pool[slots]), oracle.to_f64(vn[s0:s0 + n])])
        ref = _sdpa_request(qf[s0:s0 + n], kb, vb, p, wl.sm_scale)
        np.testing.assert_allclose(got[s0:s0 + n], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("spec", TINY_SPECS[:4], ids=lambda s: s.name)
def test_ragged_suffix_equals_stored_suffix(spec):
    """Both readings of where the suffix K/V come from give the same result: attention over the
    new rows equals attention over the pool after kv_store, bit for bit in float64."""
    wl = W.make_workload(spec, 37)
    if wl.extend is None:
        pytest.skip("no EXTEND part")
    kp, vp = stored(wl)
    a = run_extend(wl, kp, vp)
    b = run_extend(wl, wl.k_pool, wl.v_pool, suffix=_suffix_rows(wl))
    assert np.array_equal(a, b, equal_nan=True)


def test_ragged_suffix_rejects_bad_rows():
    spec = W.Spec("rag-bad", "bf16", 2, 2, 4, 64, extend_prefix=(3,), extend_lens=(2,))
    wl = W.make_workload(spec, 38)
    kn, vn = _suffix_rows(wl)
    with pytest.raises(ValueError):
        run_extend(wl, wl.k_pool, wl.v_pool, suffix=(kn[:1], vn[:1]))
    with pytest.raises(ValueError):
        run_extend(wl, wl.k_pool, wl.v_pool, suffix=(kn.astype(np.float32), vn))


# --------------------------------------------------------------------------- formats and constants

def test_bf16_bit_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0x0001, 0x3E00, 0x7FC0], dtype=np.uint16)
    v = oracle.bf16_bits_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 0.0 and math.copysign(1, v[3]) < 0
    assert math.isinf(v[4]) and v[5] == 2.0 ** -133 and v[6] == 0.125 and math.isnan(v[7])


def test_pages_constants():
    g = json.load(open(GOLDEN))
    s = g["sm_scale_head_dim_128"]
    spec = W.Spec("scale", "bf16", 1, 1, s["head_dim"], 8)
    assert round(spec.scale, s["decimals"]) == s["value"]
    from prefix_cached_paged_amd import accounting as A
    k = g["qwen3_0_6b_kv_bytes_per_token"]
    per_tok = A.kv_bytes_per_token(k["n_kv_heads"], k["head_dim"], k["layers"], k["elem_bytes"])
    assert per_tok == k["value"]
    d = g["qwen3_0_6b_decode_kv_gb_at_32768"]
    one_layer = A.decode_kv_bytes([d["context_tokens"]], k["n_kv_heads"], k["head_dim"], k["elem_bytes"])
    assert round(one_layer * k["layers"] / 1e9, d["decimals"]) == d["value"]
    h = g["qwen3_0_6b_heads"]
    assert h["n_q_heads"] // h["n_kv_heads"] == 2


# --------------------------------------------------------------------------- planted mistakes

def _mutant_softmax_drop_max(scores, v):
    m = scores.max(axis=-1, keepdims=True)
    p = np.exp(scores - m)
    return (p @ v) / p.shape[-1]          # wrong normaliser


@pytest.mark.parametrize("mutation", ["normaliser", "mask_offset", "kv_head", "transpose_v"])
def test_planted_oracle_mistakes_are_caught(monkeypatch, mutation):
    """Each plausible mistake planted in the oracle breaks agreement with the loop version."""
    spec = W.Spec("mut", "fp32", 4, 2, 8, 256, extend_prefix=(6, 0), extend_lens=(5, 8))
    wl = W.make_workload(spec, 17)
    kp, vp = stored(wl)
    e = wl.extend
    ref = np.array(oracle.extend_attention_loops(e.q, kp, vp, wl.req_to_token, e.req_pool_indices,
                                                 e.prefix_lens, e.extend_lens, e.extend_start_loc, 2,
                                                 wl.sm_scale))
    if mutation == "normaliser":
        monkeypatch.setattr(oatt, "_softmax_rows_times_v", _mutant_softmax_drop_max)
    elif mutation == "mask_offset":
        orig_mask = oatt.causal_hidden
        monkeypatch.setattr(oatt, "causal_hidden", lambda L, p, rows: orig_mask(L, p - 1, rows))
    elif mutation == "kv_head":
        orig_gather = oatt.gather_request_kv

        def swapped(*a, **k):
            kb, vb = orig_gather(*a, **k)
            return kb[:, ::-1], vb[:, ::-1]
        monkeypatch.setattr(oatt, "gather_request_kv", swapped)
    elif mutation == "transpose_v":
        orig_sm = oatt._softmax_rows_times_v

        def tv(scores, v):
            m = scores.max(axis=-1, keepdims=True)
            p = np.exp(scores - m)
            p /= p.sum(axis=-1, keepdims=True)
            n = min(v.shape)
            vt = v.copy()
            vt[:n, :n] = v[:n, :n].T
            return p @ vt
        monkeypatch.setattr(oatt, "_softmax_rows_times_v", tv)
    got = run_extend(wl, kp, vp)
    assert not np.allclose(got, ref, rtol=0, atol=1e-6, equal_nan=False)


# --------------------------------------------------------------------------- kv-head subsets

@pytest.mark.parametrize("spec", TINY_SPECS[1:4], ids=lambda s: s.name)
def test_kv_head_subset_is_a_slice_of_the_full_result(spec):
    """Computing only some kv heads (the unit the CPU baseline's worker processes take) gives the
    full computation's values for their query heads, bit for bit, and NaN for the others; the
    ragged reading takes the same subset of the new rows."""
    wl = W.make_workload(spec, 41)
    kp, vp = stored(wl)
    Hkv, G = spec.n_kv_heads, spec.n_q_heads // spec.n_kv_heads
    full_e, full_d = run_extend(wl, kp, vp), run_decode(wl, kp, vp)
    full_r = run_extend(wl, wl.k_pool, wl.v_pool, suffix=_suffix_rows(wl))
    for sel in ([Hkv - 1], list(range(Hkv))[::-1]):
        heads = np.concatenate([np.arange(g * G, (g + 1) * G) for g in sel])
        rest = np.setdiff1d(np.arange(spec.n_q_heads), heads)
        for full, part in ((full_e, run_extend(wl, kp, vp, kv_heads=sel)),
                           (full_d, run_decode(wl, kp, vp, kv_heads=sel)),
                           (full_r, run_extend(wl, wl.k_pool, wl.v_pool, suffix=_suffix_rows(wl), kv_heads=sel))):
            assert np.array_equal(part[:, heads], full[:, heads], equal_nan=True)
            assert np.all(np.isnan(part[:, rest]))
    with pytest.raises(ValueError):
        run_decode(wl, kp, vp, kv_heads=[Hkv])
