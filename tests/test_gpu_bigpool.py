"""Pools above 4 GiB for the token-table, FP8, page-table (bf16 and FP8) and ragged calls (the
64-bit addressing kernels).

A small seeded workload is spread over a large device pool by an affine slot map
s -> a * s + b (for page tables, pages p -> a * p + b, positions inside a page unchanged), so
that some of the rows a request reads lie beyond byte 2^32 of the pool. Relabelling slots leaves
attention unchanged (an oracle invariant pinned on the CPU), so the oracle runs on the small
workload. The large pools are filled on the device (NaN / the E4M3 NaN byte) and only the
referenced rows are copied in.
"""

import numpy as np
import pytest
import torch

import oracle
from prefix_cached_paged_amd import rax as R
from prefix_cached_paged_amd import workloads as W
from prefix_cached_paged_amd.device import to_dev, to_host_bits

from parity import assert_close, say

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]


def remap(table, a, b):
    t = np.asarray(table, np.int64)
    return np.where(t >= 0, t * a + b, -1).astype(np.int32)


def big_pool(small, n_big, a, b, fill):
    """Device pool of n_big rows with row a * s + b = small[s] for every s < len(small)."""
    shape = (n_big,) + tuple(small.shape[1:])
    if small.dtype == np.uint16:
        big = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    else:
        big = torch.full(shape, fill, dtype=torch.uint8, device="cuda")
    idx = torch.arange(small.shape[0], dtype=torch.int64, device="cuda") * a + b
    big[idx] = to_dev(small)
    return big


def test_fp8_extend_and_decode_pool_beyond_4gib():
    spec = W.Spec("big-fp8", "bf16", 32, 8, 128, 40000, extend_prefix=(3000, 0), extend_lens=(200, 130),
                  decode_lens=(2500, 7, 600))
    wl = W.make_workload(spec, 811)
    n_big, a, b = 4_600_000, 114, 7            # 4.6 GB per E4M3 pool; max slot 4,559,893
    assert (40000 - 1) * a + b < n_big and (40000 - 1) * a + b > (1 << 32) // (8 * 128)
    ks = vs = 4.0 * spec.sigma / 448
    used = np.unique(wl.req_to_token[wl.req_to_token >= 0]).astype(np.int64)
    rows = np.setdiff1d(used, wl.store_loc.astype(np.int64))
    kp8 = np.full(wl.k_pool.shape, 0x7F, np.uint8)
    vp8 = np.full(wl.v_pool.shape, 0x7F, np.uint8)
    kp8[rows] = oracle.quantize_bf16(wl.k_pool[rows], ks)
    vp8[rows] = oracle.quantize_bf16(wl.v_pool[rows], vs)
    say("big FP8 pools: filling on the device")
    dk, dv = big_pool(kp8, n_big, a, b, 0x7F), big_pool(vp8, n_big, a, b, 0x7F)
    r2t = to_dev(remap(wl.req_to_token, a, b))
    R.kv_store_fp8(to_dev(wl.k_new), to_dev(wl.v_new), to_dev(remap(wl.store_loc, a, b)), dk, dv, ks, vs)
    e, d = wl.extend, wl.decode
    qe, qd = to_dev(e.q), to_dev(d.q)
    oe, od = torch.empty_like(qe), torch.empty_like(qd)
    say("big FP8 pools: extend and decode")
    R.extend_attention_fp8(qe, oe, dk, dv, r2t, to_dev(e.req_pool_indices), to_dev(e.prefix_lens),
                           to_dev(e.extend_lens), to_dev(e.extend_start_loc), e.max_extend_len, e.max_seq_len,
                           wl.sm_scale, ks, vs)
    R.decode_attention_fp8(qd, od, dk, dv, r2t, to_dev(d.req_pool_indices), to_dev(d.seq_lens), d.max_seq_len,
                           wl.sm_scale, ks, vs)
    torch.cuda.synchronize()
    rk, rv = oracle.kv_store_fp8(kp8, vp8, wl.k_new, wl.v_new, wl.store_loc, ks, vs)
    ref_e = oracle.extend_attention(e.q, rk, rv, wl.req_to_token, e.req_pool_indices, e.prefix_lens, e.extend_lens,
                                    e.extend_start_loc, spec.n_kv_heads, wl.sm_scale, k_scale=ks, v_scale=vs)
    ref_d = oracle.decode_attention(d.q, rk, rv, wl.req_to_token, d.req_pool_indices, d.seq_lens, spec.n_kv_heads,
                                    wl.sm_scale, k_scale=ks, v_scale=vs)
    assert_close(oracle.to_f64(to_host_bits(oe)), ref_e, "bf16", "big FP8 extend")
    assert_close(oracle.to_f64(to_host_bits(od)), ref_d, "bf16", "big FP8 decode")


def test_fp8_paged_pool_beyond_4gib():
    """FP8 pools through a page table, pages mapped beyond byte 2^32 of the E4M3 pools."""
    P = 16
    spec = W.Spec("big-fp8-pg", "bf16", 32, 8, 128, 32768, extend_prefix=(2000, 0), extend_lens=(300, 100),
                  decode_lens=(3000, 1, 40), page_size=P)
    wl = W.make_workload(spec, 813)
    n_big, a, b = 4_600_000, 139, 5              # slots; 4.6 GB per E4M3 pool
    max_page = (32768 // P - 1) * a + b
    assert max_page < n_big // P and max_page * P > (1 << 32) // (8 * 128)
    slot_map = lambda s: np.where(np.asarray(s) >= 0, (np.asarray(s, np.int64) // P * a + b) * P + np.asarray(s) % P,
                                  -1).astype(np.int64)
    ks = vs = 4.0 * spec.sigma / 448
    used = np.unique(wl.req_to_token[wl.req_to_token >= 0]).astype(np.int64)
    rows = np.setdiff1d(used, wl.store_loc.astype(np.int64))
    kp8 = np.full(wl.k_pool.shape, 0x7F, np.uint8)
    vp8 = np.full(wl.v_pool.shape, 0x7F, np.uint8)
    kp8[rows] = oracle.quantize_bf16(wl.k_pool[rows], ks)
    vp8[rows] = oracle.quantize_bf16(wl.v_pool[rows], vs)
    say("big FP8 pools, page table: filling on the device")
    dk = torch.full((n_big, 8, 128), 0x7F, dtype=torch.uint8, device="cuda")
    dv = torch.full_like(dk, 0x7F)
    idx = torch.from_numpy(slot_map(np.arange(32768))).cuda()
    dk[idx] = to_dev(kp8)
    dv[idx] = to_dev(vp8)
    R.kv_store_fp8(to_dev(wl.k_new), to_dev(wl.v_new), to_dev(slot_map(wl.store_loc).astype(np.int32)), dk, dv,
                   ks, vs)
    pt = to_dev(remap(wl.page_table, a, b))
    e, d = wl.extend, wl.decode
    qe, qd = to_dev(e.q), to_dev(d.q)
    oe, od = torch.empty_like(qe), torch.empty_like(qd)
    say("big FP8 pools, page table: extend and decode")
    R.extend_attention_paged_fp8(qe, oe, dk, dv, pt, P, to_dev(e.req_pool_indices), to_dev(e.prefix_lens),
                                 to_dev(e.extend_lens), to_dev(e.extend_start_loc), e.max_extend_len, e.max_seq_len,
                                 wl.sm_scale, ks, vs)
    R.decode_attention_paged_fp8(qd, od, dk, dv, pt, P, to_dev(d.req_pool_indices), to_dev(d.seq_lens),
                                 d.max_seq_len, wl.sm_scale, ks, vs)
    torch.cuda.synchronize()
    rk, rv = oracle.kv_store_fp8(kp8, vp8, wl.k_new, wl.v_new, wl.store_loc, ks, vs)
    ref_e = oracle.extend_attention(e.q, rk, rv, wl.req_to_token, e.req_pool_indices, e.prefix_lens, e.extend_lens,
                                    e.extend_start_loc, spec.n_kv_heads, wl.sm_scale, k_scale=ks, v_scale=vs)
    ref_d = oracle.decode_attention(d.q, rk, rv, wl.req_to_token, d.req_pool_indices, d.seq_lens, spec.n_kv_heads,
                                    wl.sm_scale, k_scale=ks, v_scale=vs)
    assert_close(oracle.to_f64(to_host_bits(oe)), ref_e, "bf16", "big paged FP8 extend")
    assert_close(oracle.to_f64(to_host_bits(od)), ref_d, "bf16", "big paged FP8 decode")


def test_paged_and_ragged_pool_beyond_4gib():
    P = 16
    spec = W.Spec("big-pg", "bf16", 32, 8, 128, 32768, extend_prefix=(2000, 0), extend_lens=(300, 100),
                  decode_lens=(3000, 1, 40), page_size=P)
    wl = W.make_workload(spec, 812)
    n_big, a, b = 2_400_000, 73, 3              # pages; 4.9 GB per bf16 pool
    n_pages = n_big // P
    assert (32768 // P - 1) * a + b < n_pages and ((32768 // P - 1) * a + b) * P > (1 << 32) // (8 * 128 * 2)
    slot_map = lambda s: np.where(np.asarray(s) >= 0, (np.asarray(s, np.int64) // P * a + b) * P + np.asarray(s) % P,
                                  -1).astype(np.int32)
    pt = to_dev(remap(wl.page_table, a, b))
    r2t_np = slot_map(wl.req_to_token)
    say("big bf16 pools: filling on the device")
    # place small-pool row s at slot_map(s)
    dk = torch.full((n_big, 8, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    dv = torch.full_like(dk, float("nan"))
    idx = torch.from_numpy(slot_map(np.arange(32768)).astype(np.int64)).cuda()
    dk[idx] = to_dev(wl.k_pool)
    dv[idx] = to_dev(wl.v_pool)
    e, d = wl.extend, wl.decode
    n = e.total_tokens
    kn, vn = to_dev(wl.k_new), to_dev(wl.v_new)
    loc = to_dev(slot_map(wl.store_loc))
    qe, qd = to_dev(e.q), to_dev(d.q)
    oe, od, orag = torch.empty_like(qe), torch.empty_like(qd), torch.empty_like(qe)
    erest = (to_dev(e.req_pool_indices), to_dev(e.prefix_lens), to_dev(e.extend_lens), to_dev(e.extend_start_loc),
             e.max_extend_len, e.max_seq_len, wl.sm_scale)
    say("big bf16 pools: ragged extend with the fused store of the suffix rows")
    R.extend_attention_ragged(qe, orag, kn[:n], vn[:n], dk, dv, to_dev(r2t_np), *erest, store_loc=loc[:n])
    R.kv_store(kn[n:], vn[n:], loc[n:], dk, dv)       # the decode requests' current tokens
    say("big bf16 pools: paged extend and decode")
    R.extend_attention_paged(qe, oe, dk, dv, pt, P, *erest)
    R.decode_attention_paged(qd, od, dk, dv, pt, P, to_dev(d.req_pool_indices), to_dev(d.seq_lens), d.max_seq_len,
                             wl.sm_scale)
    torch.cuda.synchronize()
    kp, vp = oracle.kv_store(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.store_loc)
    ref_e = oracle.extend_attention(e.q, kp, vp, wl.req_to_token, e.req_pool_indices, e.prefix_lens, e.extend_lens,
                                    e.extend_start_loc, spec.n_kv_heads, wl.sm_scale)
    ref_d = oracle.decode_attention(d.q, kp, vp, wl.req_to_token, d.req_pool_indices, d.seq_lens, spec.n_kv_heads,
                                    wl.sm_scale)
    assert_close(oracle.to_f64(to_host_bits(orag)), ref_e, "bf16", "big ragged extend")
    assert_close(oracle.to_f64(to_host_bits(oe)), ref_e, "bf16", "big paged extend")
    assert_close(oracle.to_f64(to_host_bits(od)), ref_d, "bf16", "big paged decode")
    # the fused store wrote the suffix rows at their mapped slots
    got = to_host_bits(dk[loc[:n].long()])
    assert np.array_equal(got, wl.k_new[:n])


def test_token_table_pool_beyond_4gib():
    """bf16 pools read through the token table (the pool-reading EXTEND and DECODE) with rows
    beyond byte 2^32: the 64-bit addressing form of the bf16 kernels."""
    spec = W.Spec("big-tok", "bf16", 32, 8, 128, 40000, extend_prefix=(3000, 0), extend_lens=(200, 130),
                  decode_lens=(2500, 7, 600))
    wl = W.make_workload(spec, 813)
    n_big, a, b = 2_400_000, 59, 11              # 4.9 GB per bf16 pool; max slot 2,359,952
    assert (40000 - 1) * a + b < n_big and (40000 - 1) * a + b > (1 << 32) // (8 * 128 * 2)
    say("big bf16 token-table pools: filling on the device")
    dk = big_pool(wl.k_pool, n_big, a, b, None)
    dv = big_pool(wl.v_pool, n_big, a, b, None)
    r2t = to_dev(remap(wl.req_to_token, a, b))
    R.kv_store(to_dev(wl.k_new), to_dev(wl.v_new), to_dev(remap(wl.store_loc, a, b)), dk, dv)
    e, d = wl.extend, wl.decode
    qe, qd = to_dev(e.q), to_dev(d.q)
    oe, od = torch.empty_like(qe), torch.empty_like(qd)
    say("big bf16 token-table pools: extend and decode")
    R.extend_attention(qe, oe, dk, dv, r2t, to_dev(e.req_pool_indices), to_dev(e.prefix_lens),
                       to_dev(e.extend_lens), to_dev(e.extend_start_loc), e.max_extend_len, e.max_seq_len,
                       wl.sm_scale)
    R.decode_attention(qd, od, dk, dv, r2t, to_dev(d.req_pool_indices), to_dev(d.seq_lens), d.max_seq_len,
                       wl.sm_scale)
    torch.cuda.synchronize()
    kp, vp = oracle.kv_store(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.store_loc)
    ref_e = oracle.extend_attention(e.q, kp, vp, wl.req_to_token, e.req_pool_indices, e.prefix_lens, e.extend_lens,
                                    e.extend_start_loc, spec.n_kv_heads, wl.sm_scale)
    ref_d = oracle.decode_attention(d.q, kp, vp, wl.req_to_token, d.req_pool_indices, d.seq_lens, spec.n_kv_heads,
                                    wl.sm_scale)
    assert_close(oracle.to_f64(to_host_bits(oe)), ref_e, "bf16", "big token-table extend")
    assert_close(oracle.to_f64(to_host_bits(od)), ref_d, "bf16", "big token-table decode")
    # rows beyond byte 2^32 are among those read
    used = remap(wl.req_to_token[wl.req_to_token >= 0], a, b).astype(np.int64)
    assert (used * 8 * 128 * 2 >= (1 << 32)).sum() > 100
