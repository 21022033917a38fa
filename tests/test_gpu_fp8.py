"""FP8 E4M3 KV pools on the GPU against the float64 oracle: the store, EXTEND and DECODE.

The store is compared byte for byte with ``oracle.kv_store_fp8``. For attention, the cached
prefix/context rows are encoded by the oracle (as if an earlier step had stored them), the
step's new rows go through the GPU store, and the GPU attention over the FP8 pools is compared
with the oracle's attention over the same bytes and scales. Slots no request names hold the
E4M3 NaN byte, so a read of a wrong slot poisons the output.
"""

import numpy as np
import pytest
import torch

import oracle
from prefix_cached_paged_amd import rax as R
from prefix_cached_paged_amd import workloads as W
from prefix_cached_paged_amd.device import to_dev, to_host_bits

from parity import assert_close, say

pytestmark = pytest.mark.gpu

NAN8 = 0x7F


def test_store_matches_oracle_bytes():
    rng = np.random.default_rng(701)
    S, H, D, n = 5000, 8, 128, 777
    for k_scale, v_scale in [(1.0, 1.0), (0.02, 0.05), (3.0, 0.7), (2.0 ** -6, 2.0 ** 5)]:
        x = np.concatenate([rng.normal(0, 1, n * H * D // 2), rng.normal(0, 300, n * H * D // 4),
                            rng.normal(0, 1e-3, n * H * D // 4)]).astype(np.float32)
        rng.shuffle(x)
        kn = (x.view(np.uint32) >> 16).astype(np.uint16).reshape(n, H, D)   # truncation: any bf16
        vn = kn[::-1].copy()
        kp = rng.integers(0, 256, (S, H, D), dtype=np.uint8)
        vp = rng.integers(0, 256, (S, H, D), dtype=np.uint8)
        loc = rng.permutation(S)[:n].astype(np.int32)
        ref_k, ref_v = oracle.kv_store_fp8(kp, vp, kn, vn, loc, k_scale, v_scale)
        dk, dv = to_dev(kp), to_dev(vp)
        R.kv_store_fp8(to_dev(kn), to_dev(vn), to_dev(loc), dk, dv, k_scale, v_scale)
        torch.cuda.synchronize()
        assert np.array_equal(dk.cpu().numpy(), ref_k), f"K bytes differ at scale {k_scale}"
        assert np.array_equal(dv.cpu().numpy(), ref_v), f"V bytes differ at scale {v_scale}"


def fp8_pools(wl, k_scale, v_scale):
    """Pools with every row a request reads (except the step's new rows) encoded by the oracle,
    and the NaN byte elsewhere."""
    S = wl.k_pool.shape[0]
    kp = np.full(wl.k_pool.shape, NAN8, np.uint8)
    vp = np.full(wl.v_pool.shape, NAN8, np.uint8)
    reads = []
    if wl.decode is not None:
        reads += list(zip(wl.decode.req_pool_indices, wl.decode.seq_lens))
    if wl.extend is not None:
        reads += list(zip(wl.extend.req_pool_indices, wl.extend.prefix_lens + wl.extend.extend_lens))
    used = np.unique(np.concatenate([wl.req_to_token[int(r), :int(L)] for r, L in reads]).astype(np.int64))
    rows = np.setdiff1d(used, np.asarray(wl.store_loc, np.int64))
    assert rows.size == 0 or rows.max() < S
    kp[rows] = oracle.quantize_bf16(wl.k_pool[rows], k_scale)
    vp[rows] = oracle.quantize_bf16(wl.v_pool[rows], v_scale)
    return kp, vp


def run_decode_fp8(wl, k_scale, v_scale):
    kp, vp = fp8_pools(wl, k_scale, v_scale)
    dk, dv = to_dev(kp), to_dev(vp)
    R.kv_store_fp8(to_dev(wl.k_new), to_dev(wl.v_new), to_dev(wl.store_loc), dk, dv, k_scale, v_scale)
    d = wl.decode
    q = to_dev(d.q)
    o = torch.empty_like(q)
    R.decode_attention_fp8(q, o, dk, dv, to_dev(wl.req_to_token), to_dev(d.req_pool_indices),
                           to_dev(d.seq_lens), d.max_seq_len, wl.sm_scale, k_scale, v_scale)
    torch.cuda.synchronize()
    ref_k, ref_v = oracle.kv_store_fp8(kp, vp, wl.k_new, wl.v_new, wl.store_loc, k_scale, v_scale)
    ref = oracle.decode_attention(d.q, ref_k, ref_v, wl.req_to_token, d.req_pool_indices, d.seq_lens,
                                  wl.spec.n_kv_heads, wl.sm_scale, k_scale=k_scale, v_scale=v_scale)
    return oracle.to_f64(to_host_bits(o)), ref


# Sized so that the rows each case encodes on the host stay within a few million elements.
SPECS = [
    W.Spec("fp8-dec-g4", "bf16", 32, 8, 128, 60000, decode_lens=(1, 2, 63, 64, 65, 257, 1000, 2500)),
    W.Spec("fp8-dec-g1", "bf16", 8, 8, 128, 60000, decode_lens=(1, 130, 3000)),
    W.Spec("fp8-dec-g8", "bf16", 64, 8, 128, 60000, decode_lens=(5, 513, 4000)),
    W.Spec("fp8-dec-g16", "bf16", 16, 1, 128, 60000, decode_lens=(77, 4096, 12345)),
    W.Spec("fp8-dec-d64", "bf16", 16, 4, 64, 60000, decode_lens=(1, 64, 999, 5000)),
    W.Spec("fp8-dec-g48", "bf16", 48, 1, 128, 60000, decode_lens=(5, 4000, 65)),
    W.Spec("fp8-dec-1kv-g8", "bf16", 8, 1, 128, 60000, decode_lens=(1, 64, 65, 200, 3000)),
    W.Spec("fp8-dec-2kv-d64", "bf16", 8, 2, 64, 60000, decode_lens=(2, 129, 2500)),
    W.Spec("fp8-dec-many", "bf16", 32, 8, 128, 60000, decode_batch=64, decode_range=(1, 120)),
    W.Spec("fp8-dec-long", "bf16", 8, 1, 128, 120000, decode_lens=(50000, 3)),
    # more than 1,024 requests: the plan runs as its own kernel before the split
    W.Spec("fp8-dec-plan", "bf16", 8, 2, 128, 30000, decode_batch=1500, decode_range=(1, 16)),
]
# scales that put about 4 standard deviations at the top of the E4M3 range, and the default 1.0
CASES = [("normal", "range"), ("normal", "one"), ("peaked", "range"), ("needle", "range")]


@pytest.mark.parametrize("variant,scales", CASES)
@pytest.mark.parametrize("spec", SPECS, ids=lambda s: s.name)
def test_decode_fp8(spec, variant, scales):
    wl = W.make_workload(spec, 702, variant)
    if scales == "one":
        k_scale = v_scale = 1.0
    else:
        k_scale = v_scale = 4 * spec.sigma / 448
        if variant == "needle":
            k_scale = 16.0 / 448  # the needle key is 12 sigma: keep it inside the range
    say(f"{spec.name}/{variant}: scales {k_scale:.4g} {v_scale:.4g}")
    got, ref = run_decode_fp8(wl, k_scale, v_scale)
    assert_close(got, ref, "bf16", f"{spec.name}/{variant} fp8 decode")


def test_decode_fp8_single_key_is_v_times_scale():
    """One key: the output is v_scale * e4m3(V), the bf16 rounding of that product."""
    spec = W.Spec("fp8-one", "bf16", 32, 8, 128, 1000, decode_lens=(1, 1, 1))
    wl = W.make_workload(spec, 703)
    got, ref = run_decode_fp8(wl, 0.5, 0.25)       # power-of-two scales: products exact in bf16
    assert np.array_equal(got, ref)


def run_extend_fp8(wl, k_scale, v_scale):
    kp, vp = fp8_pools(wl, k_scale, v_scale)
    dk, dv = to_dev(kp), to_dev(vp)
    R.kv_store_fp8(to_dev(wl.k_new), to_dev(wl.v_new), to_dev(wl.store_loc), dk, dv, k_scale, v_scale)
    e = wl.extend
    q = to_dev(e.q)
    o = torch.full_like(q, float("nan"))    # rows the kernel skips stay NaN
    R.extend_attention_fp8(q, o, dk, dv, to_dev(wl.req_to_token), to_dev(e.req_pool_indices),
                           to_dev(e.prefix_lens), to_dev(e.extend_lens), to_dev(e.extend_start_loc),
                           int(np.max(e.extend_lens)), int(np.max(e.prefix_lens + e.extend_lens)),
                           wl.sm_scale, k_scale, v_scale)
    torch.cuda.synchronize()
    ref_k, ref_v = oracle.kv_store_fp8(kp, vp, wl.k_new, wl.v_new, wl.store_loc, k_scale, v_scale)
    ref = oracle.extend_attention(e.q, ref_k, ref_v, wl.req_to_token, e.req_pool_indices, e.prefix_lens,
                                  e.extend_lens, e.extend_start_loc, wl.spec.n_kv_heads, wl.sm_scale,
                                  k_scale=k_scale, v_scale=v_scale)
    return oracle.to_f64(to_host_bits(o)), ref


# Every group size of the kernel; contexts of 1, 2, 3 and many 64-key tiles (the prologue and
# both loops), prefixes of 0 and off tile boundaries, suffixes that end mid-tile.
EXT_SPECS = [
    W.Spec("fp8-ext-g4", "bf16", 32, 8, 128, 60000, extend_prefix=(0, 1, 63, 64, 500, 1500),
           extend_lens=(65, 1, 64, 129, 300, 257)),
    W.Spec("fp8-ext-g1", "bf16", 4, 4, 128, 30000, extend_prefix=(0, 200, 37), extend_lens=(300, 129, 1)),
    W.Spec("fp8-ext-g2", "bf16", 8, 4, 128, 30000, extend_prefix=(10, 0), extend_lens=(190, 64)),
    W.Spec("fp8-ext-g8", "bf16", 64, 8, 128, 60000, extend_prefix=(1000, 5), extend_lens=(33, 200)),
    W.Spec("fp8-ext-g16", "bf16", 16, 1, 128, 30000, extend_prefix=(129, 0, 2000), extend_lens=(20, 17, 70)),
    W.Spec("fp8-ext-g32", "bf16", 32, 1, 128, 30000, extend_prefix=(0, 700), extend_lens=(40, 9)),
    W.Spec("fp8-ext-short", "bf16", 32, 8, 128, 30000, extend_prefix=(0, 0, 64, 100), extend_lens=(1, 64, 64, 28)),
    # head_dim 64: four E4M3 units per row, the copy lanes of units 4-7 repeat units 0-3
    W.Spec("fp8-ext-d64-g4", "bf16", 32, 8, 64, 60000, extend_prefix=(0, 63, 500), extend_lens=(129, 65, 300)),
    W.Spec("fp8-ext-d64-g1", "bf16", 4, 4, 64, 30000, extend_prefix=(37, 0), extend_lens=(200, 1)),
    # group sizes of the run-time group kernel
    W.Spec("fp8-ext-g7", "bf16", 28, 4, 128, 60000, extend_prefix=(0, 63, 1000), extend_lens=(100, 37, 73)),
    W.Spec("fp8-ext-d64-g3", "bf16", 6, 2, 64, 30000, extend_prefix=(0, 500), extend_lens=(200, 86)),
    # one (request, kv head) pair: its 32 row tiles shared out over all XCDs
    W.Spec("fp8-ext-1pair", "bf16", 8, 1, 128, 30000, extend_prefix=(300,), extend_lens=(1000,)),
    # few row tiles: each row tile's keys split over several workgroups and merged
    W.Spec("fp8-ext-split", "bf16", 32, 8, 128, 30000, extend_prefix=(9000, 0), extend_lens=(100, 30)),
    W.Spec("fp8-ext-split-mqa", "bf16", 8, 1, 128, 30000, extend_prefix=(6000,), extend_lens=(200,)),
]


@pytest.mark.parametrize("variant,scales", CASES)
@pytest.mark.parametrize("spec", EXT_SPECS, ids=lambda s: s.name)
def test_extend_fp8(spec, variant, scales):
    wl = W.make_workload(spec, 704, variant)
    if scales == "one":
        k_scale = v_scale = 1.0
    else:
        k_scale = v_scale = 4 * spec.sigma / 448
        if variant == "needle":
            k_scale = 16.0 / 448
    say(f"{spec.name}/{variant}: scales {k_scale:.4g} {v_scale:.4g}")
    got, ref = run_extend_fp8(wl, k_scale, v_scale)
    assert_close(got, ref, "bf16", f"{spec.name}/{variant} fp8 extend")


def test_extend_fp8_first_row_is_v_times_scale():
    """A suffix row at position 0 (no prefix) sees one key: v_scale * e4m3(V) exactly."""
    spec = W.Spec("fp8-ext-one", "bf16", 32, 8, 128, 1000, extend_prefix=(0, 0), extend_lens=(1, 5))
    wl = W.make_workload(spec, 705)
    got, ref = run_extend_fp8(wl, 0.5, 0.25)
    first = np.asarray(wl.extend.extend_start_loc)
    assert np.array_equal(got[first], ref[first])
    assert_close(got, ref, "bf16", "fp8 extend, one key")


# FP8 pools through page tables: page sizes 8 to 64, both head_dims, EXTEND and DECODE in one
# workload. Against the oracle over the same bytes, and bit for bit against the token-table
# FP8 calls on the same slots.
PAGED_SPECS = [
    W.Spec("fp8-pg16-g4", "bf16", 32, 8, 128, 65536, extend_prefix=(0, 63, 500), extend_lens=(129, 65, 300),
           decode_lens=(1, 17, 2500), page_size=16),
    W.Spec("fp8-pg64-g8", "bf16", 64, 8, 128, 65536, extend_prefix=(1000, 0), extend_lens=(33, 64),
           decode_lens=(5, 513, 4000), page_size=64),
    W.Spec("fp8-pg8-d64-g4", "bf16", 16, 4, 64, 65536, extend_prefix=(37, 0), extend_lens=(200, 1),
           decode_lens=(64, 999), page_size=8),
]


@pytest.mark.parametrize("variant", ["normal", "peaked", "needle"])
@pytest.mark.parametrize("spec", PAGED_SPECS, ids=lambda s: s.name)
def test_paged_fp8(spec, variant):
    wl = W.make_workload(spec, 706, variant)
    k_scale = v_scale = 4 * spec.sigma / 448
    if variant == "needle":
        k_scale = 16.0 / 448
    P = spec.page_size
    say(f"paged fp8 {spec.name}/{variant}: P={P}")
    kp, vp = fp8_pools(wl, k_scale, v_scale)
    dk, dv = to_dev(kp), to_dev(vp)
    R.kv_store_fp8(to_dev(wl.k_new), to_dev(wl.v_new), to_dev(wl.store_loc), dk, dv, k_scale, v_scale)
    ref_k, ref_v = oracle.kv_store_fp8(kp, vp, wl.k_new, wl.v_new, wl.store_loc, k_scale, v_scale)
    pt, r2t = to_dev(wl.page_table), to_dev(wl.req_to_token)
    e, d = wl.extend, wl.decode
    qe, qd = to_dev(e.q), to_dev(d.q)
    oe, oe_tok = torch.full_like(qe, float("nan")), torch.full_like(qe, float("nan"))
    od, od_tok = torch.empty_like(qd), torch.empty_like(qd)
    per = (to_dev(e.req_pool_indices), to_dev(e.prefix_lens), to_dev(e.extend_lens), to_dev(e.extend_start_loc),
           int(np.max(e.extend_lens)), int(np.max(e.prefix_lens + e.extend_lens)), wl.sm_scale, k_scale, v_scale)
    R.extend_attention_paged_fp8(qe, oe, dk, dv, pt, P, *per)
    R.extend_attention_fp8(qe, oe_tok, dk, dv, r2t, *per)
    dper = (to_dev(d.req_pool_indices), to_dev(d.seq_lens), d.max_seq_len, wl.sm_scale, k_scale, v_scale)
    R.decode_attention_paged_fp8(qd, od, dk, dv, pt, P, *dper)
    R.decode_attention_fp8(qd, od_tok, dk, dv, r2t, *dper)
    torch.cuda.synchronize()
    ref_e = oracle.extend_attention_paged(e.q, ref_k, ref_v, wl.page_table, P, e.req_pool_indices, e.prefix_lens,
                                          e.extend_lens, e.extend_start_loc, spec.n_kv_heads, wl.sm_scale,
                                          k_scale=k_scale, v_scale=v_scale)
    ref_d = oracle.decode_attention_paged(d.q, ref_k, ref_v, wl.page_table, P, d.req_pool_indices, d.seq_lens,
                                          spec.n_kv_heads, wl.sm_scale, k_scale=k_scale, v_scale=v_scale)
    assert_close(oracle.to_f64(to_host_bits(oe)), ref_e, "bf16", f"{spec.name}/{variant} paged fp8 extend")
    assert_close(oracle.to_f64(to_host_bits(od)), ref_d, "bf16", f"{spec.name}/{variant} paged fp8 decode")
    assert torch.equal(oe.view(torch.int16), oe_tok.view(torch.int16)), "paged and token-table FP8 EXTEND differ"
    assert torch.equal(od.view(torch.int16), od_tok.view(torch.int16)), "paged and token-table FP8 DECODE differ"
