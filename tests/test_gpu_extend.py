"""EXTEND parity on the GPU against the float64 oracle, plus invariants of the HIP path."""

import numpy as np
import pytest
import torch

import oracle
from prefix_cached_paged_amd import rax as R
from prefix_cached_paged_amd import workloads as W
from prefix_cached_paged_amd.device import to_dev, to_host_bits, upload

from parity import (assert_close, extend, oracle_decode, oracle_extend, out_f64, run_all, say, stored_pools)

pytestmark = pytest.mark.gpu

# Several 128-row tiles and ragged tails; prefixes that end mid key-tile; e = 0 and e = 1 rows.
SMALL = [
    W.Spec("ext-g4", "bf16", 32, 8, 128, 100000, extend_prefix=(0, 1, 63, 64, 500, 3000),
           extend_lens=(1, 40, 65, 128, 77, 300)),
    W.Spec("ext-g1", "bf16", 4, 4, 128, 50000, extend_prefix=(0, 200, 37), extend_lens=(300, 129, 0)),
    W.Spec("ext-g2", "bf16", 8, 4, 128, 50000, extend_prefix=(10, 0), extend_lens=(190, 64)),
    W.Spec("ext-g8", "bf16", 64, 8, 128, 100000, extend_prefix=(1000, 5), extend_lens=(33, 200)),
    W.Spec("ext-g16", "bf16", 16, 1, 128, 50000, extend_prefix=(129, 0), extend_lens=(20, 17)),
    W.Spec("ext-shared", "bf16", 32, 8, 128, 100000, extend_prefix=(700,) * 5, extend_lens=(100, 1, 64, 129, 3),
           shared_prefix=True),
    # head_dim 64: the same tiles with half-filled LDS rows
    W.Spec("ext-d64-g4", "bf16", 32, 8, 64, 100000, extend_prefix=(0, 1, 63, 64, 500, 3000),
           extend_lens=(1, 40, 65, 128, 77, 300)),
    W.Spec("ext-d64-g1", "bf16", 4, 4, 64, 50000, extend_prefix=(0, 200, 37), extend_lens=(300, 129, 0)),
    W.Spec("ext-d64-g8", "bf16", 64, 8, 64, 100000, extend_prefix=(1000, 5), extend_lens=(33, 200)),
    W.Spec("ext-d64-g32", "bf16", 32, 1, 64, 50000, extend_prefix=(0, 640), extend_lens=(500, 9)),
    # group sizes without their own kernel (the run-time group size): floor(256 / G) tokens per
    # workgroup, the rows past them idle
    W.Spec("ext-g3", "bf16", 6, 2, 128, 50000, extend_prefix=(0, 37, 500), extend_lens=(200, 86, 300)),
    W.Spec("ext-g7", "bf16", 28, 4, 128, 100000, extend_prefix=(0, 63, 1000), extend_lens=(100, 37, 73)),
    W.Spec("ext-d64-g5", "bf16", 40, 8, 64, 100000, extend_prefix=(64, 0), extend_lens=(103, 52)),
    W.Spec("ext-g12", "bf16", 12, 1, 128, 50000, extend_prefix=(129, 0), extend_lens=(43, 21)),
    W.Spec("ext-g64", "bf16", 64, 1, 128, 50000, extend_prefix=(0, 300), extend_lens=(9, 30)),
    # (request, kv head) pair counts that are not a multiple of 8: the tiles of the last pairs
    # are shared out over several XCDs (1 pair on 8, 3 pairs on 2 each, 13 = 8 + 5 pairs)
    W.Spec("ext-1pair", "bf16", 8, 1, 128, 50000, extend_prefix=(300,), extend_lens=(1000,)),
    W.Spec("ext-3pair", "bf16", 12, 3, 128, 50000, extend_prefix=(77,), extend_lens=(700,)),
    W.Spec("ext-13pair", "bf16", 16, 1, 128, 50000, extend_prefix=(0, 5, 64, 100, 129, 1, 2, 300, 0, 7, 40, 63, 8),
           extend_lens=(40, 17, 33, 1, 64, 90, 16, 5, 77, 2, 48, 31, 100)),
    # too few row tiles to fill the CUs: each row tile's keys are split over up to 16
    # workgroups and merged (a short suffix on a long prefix; the second request's tiles leave
    # most splits without keys; head_dim 64; a run-time group size)
    W.Spec("ext-split-mqa", "bf16", 8, 1, 128, 50000, extend_prefix=(10000,), extend_lens=(100,)),
    W.Spec("ext-split-g4", "bf16", 32, 8, 128, 50000, extend_prefix=(12000, 0), extend_lens=(100, 37)),
    W.Spec("ext-split-d64", "bf16", 16, 4, 64, 50000, extend_prefix=(5000, 700), extend_lens=(200, 64)),
    W.Spec("ext-split-g7", "bf16", 28, 4, 128, 50000, extend_prefix=(3000,), extend_lens=(300,)),
]


@pytest.mark.parametrize("variant", ["normal", "peaked", "needle"])
@pytest.mark.parametrize("spec", SMALL, ids=lambda s: s.name)
def test_extend_small(spec, variant):
    wl = W.make_workload(spec, 701, variant)
    say(f"extend {spec.name}/{variant}: B={wl.extend.batch} N={wl.extend.total_tokens}")
    dw, outs = run_all(wl)
    kp, vp = stored_pools(wl)
    ref = oracle_extend(wl, kp, vp)
    got = out_f64(outs["extend"])
    assert_close(got, ref, spec.dtype, f"{spec.name}/{variant}")


@pytest.mark.parametrize("seed_off", [0, 100, 200])
def test_extend_tiny_fp32(seed_off):
    """Tiny EXTEND in fp32: prefixes {0,16,64,128}, extends {32,16,8,1}, 4 heads, d=64: all rows."""
    spec = W.CONFIGS[1]
    wl = W.make_workload(spec, W.TIMING_SEEDS[1] + seed_off)
    dw, outs = run_all(wl)
    kp, vp = stored_pools(wl)
    assert_close(out_f64(outs["extend"]), oracle_extend(wl, kp, vp), "fp32", f"{spec.name} seed+{seed_off}")


@pytest.mark.parametrize("spec", [
    W.Spec("ext-fp32-d128-g3", "fp32", 6, 2, 128, 20000, extend_prefix=(0, 300), extend_lens=(70, 65)),
    W.Spec("ext-fp32-peaked", "fp32", 4, 4, 64, 4000, extend_prefix=(5, 1000), extend_lens=(100, 3)),
], ids=lambda s: s.name)
def test_extend_fp32(spec):
    wl = W.make_workload(spec, 702, "peaked" if "peaked" in spec.name else "normal")
    dw, outs = run_all(wl)
    kp, vp = stored_pools(wl)
    assert_close(out_f64(outs["extend"]), oracle_extend(wl, kp, vp), "fp32", spec.name)


def test_extend_one_token_matches_decode():
    """EXTEND with e = 1 on prefix p and DECODE over p + 1 keys agree (two different kernels)."""
    spec = W.Spec("e1", "bf16", 32, 8, 128, 50000, extend_prefix=(0, 63, 64, 2000), extend_lens=(1, 1, 1, 1))
    wl = W.make_workload(spec, 703)
    dw, outs = run_all(wl)
    e = dw.ext
    o2 = torch.empty_like(e["o"])
    seq = (e["prefix_lens"] + e["extend_lens"]).contiguous()
    R.decode_attention(e["q"], o2, dw.k_pool, dw.v_pool, dw.req_to_token, e["req_pool_indices"], seq,
                       e["max_seq_len"], wl.sm_scale)
    torch.cuda.synchronize()
    assert_close(out_f64(outs["extend"]), out_f64(o2), "bf16", "extend(e=1) vs decode")


def test_prefix_extend_matches_full_prefill_tail():
    spec = W.Spec("tail", "bf16", 32, 8, 128, 50000, extend_prefix=(300,), extend_lens=(200,))
    wl = W.make_workload(spec, 704)
    dw, outs = run_all(wl)
    part = out_f64(outs["extend"])
    e = dw.ext
    q_full = torch.cat([torch.zeros((300, 32, 128), dtype=e["q"].dtype, device="cuda"), e["q"]]).contiguous()
    o_full = torch.empty_like(q_full)
    z = torch.zeros(1, dtype=torch.int32, device="cuda")
    n = torch.full((1,), 500, dtype=torch.int32, device="cuda")
    R.extend_attention(q_full, o_full, dw.k_pool, dw.v_pool, dw.req_to_token, e["req_pool_indices"], z, n, z,
                       500, 500, wl.sm_scale)
    torch.cuda.synchronize()
    assert_close(part, out_f64(o_full)[300:], "bf16", "prefix-extend vs prefill tail")


def test_single_key_returns_value_bitwise():
    spec = W.Spec("one", "bf16", 32, 8, 128, 1000, extend_prefix=(0, 0), extend_lens=(1, 5))
    wl = W.make_workload(spec, 705)
    dw, outs = run_all(wl)
    got = to_host_bits(outs["extend"])
    for b, row in ((0, 0), (1, 1)):  # first suffix token of a request with no prefix sees only itself
        for h in range(32):
            assert np.array_equal(got[row, h], wl.v_new[row, h // 4])


def test_slot_permutation_bitwise_and_deterministic():
    spec = W.Spec("perm", "bf16", 32, 8, 128, 30000, extend_prefix=(100, 1000), extend_lens=(150, 70))
    wl = W.make_workload(spec, 706)
    dw, outs = run_all(wl)
    a = to_host_bits(outs["extend"]).copy()
    extend(dw, wl)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(dw.ext["o"]), a)
    perm = np.random.default_rng(6).permutation(spec.num_slots)
    kp, vp = stored_pools(wl)
    kq = np.empty_like(kp)
    vq = np.empty_like(vp)
    kq[perm] = kp
    vq[perm] = vp
    r2t = wl.req_to_token.copy()
    m = r2t >= 0
    r2t[m] = perm[r2t[m]]
    dw.k_pool.copy_(to_dev(kq))
    dw.v_pool.copy_(to_dev(vq))
    dw.req_to_token.copy_(to_dev(r2t))
    extend(dw, wl)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(dw.ext["o"]), a)


def test_gqa_equals_repeated_kv_bitwise():
    """The row arithmetic does not depend on G: G=4 vs. G=1 over repeat-interleaved KV is bitwise equal."""
    spec = W.Spec("gqa", "bf16", 16, 4, 128, 30000, extend_prefix=(0, 90), extend_lens=(130, 64))
    wl = W.make_workload(spec, 707)
    dw, outs = run_all(wl)
    a = to_host_bits(outs["extend"])
    kp, vp = stored_pools(wl)
    e = dw.ext
    o2 = torch.empty_like(e["o"])
    R.extend_attention(e["q"], o2, to_dev(np.repeat(kp, 4, axis=1)), to_dev(np.repeat(vp, 4, axis=1)),
                       dw.req_to_token, e["req_pool_indices"], e["prefix_lens"], e["extend_lens"],
                       e["extend_start_loc"], e["max_extend_len"], e["max_seq_len"], wl.sm_scale)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(o2), a)


@pytest.mark.timeout(600)
def test_extend_and_decode_pool_beyond_4gib():
    """A pool of 1,048,577 slots x 16 kv heads x 128 (4 GiB + 4 KiB per array) takes the 64-bit
    addressing path; slots are spread over the whole pool, so rows beyond 2^32 bytes are read."""
    spec = W.Spec("big-pool", "bf16", 64, 16, 128, 1_048_577, extend_prefix=(3000, 0), extend_lens=(100, 130),
                  decode_lens=(2000, 5))
    wl = W.make_workload(spec, 708)
    say("big pool generated")
    dw, outs = run_all(wl)
    kp, vp = stored_pools(wl)
    assert_close(out_f64(outs["extend"]), oracle_extend(wl, kp, vp), "bf16", "big-pool extend")
    assert_close(out_f64(outs["decode"]), oracle_decode(wl, kp, vp), "bf16", "big-pool decode")
