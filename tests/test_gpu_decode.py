"""DECODE parity on the GPU against the float64 oracle, plus invariants of the HIP path."""

import numpy as np
import pytest
import torch

import oracle
from prefix_cached_paged_amd import rax as R
from prefix_cached_paged_amd import workloads as W
from prefix_cached_paged_amd.device import to_dev, to_host_bits, upload

from parity import assert_close, decode, oracle_decode, out_f64, run_all, say, store, stored_pools

pytestmark = pytest.mark.gpu

# Lengths around the 64-key iteration and the split boundaries, single keys, long ragged tails.
SMALL = [
    W.Spec("dec-g4", "bf16", 32, 8, 128, 200000, decode_lens=(1, 2, 63, 64, 65, 255, 256, 257, 1000, 4097, 9000)),
    W.Spec("dec-g1", "bf16", 8, 8, 128, 100000, decode_lens=(1, 130, 3000)),
    W.Spec("dec-g2", "bf16", 8, 4, 128, 100000, decode_lens=(17, 700, 2500)),
    W.Spec("dec-g8", "bf16", 64, 8, 128, 300000, decode_lens=(5, 513, 20000)),
    W.Spec("dec-g16", "bf16", 16, 1, 128, 100000, decode_lens=(77, 4096, 12345)),
    W.Spec("dec-d64", "bf16", 16, 4, 64, 100000, decode_lens=(1, 64, 999, 5000)),
    # groups above 16: ceil(G / 16) waves of up to 16 query heads per kv head
    W.Spec("dec-g17", "bf16", 34, 2, 128, 100000, decode_lens=(1, 300, 4097)),
    W.Spec("dec-g24", "bf16", 48, 2, 128, 100000, decode_lens=(64, 2500, 700)),
    W.Spec("dec-g48", "bf16", 48, 1, 128, 100000, decode_lens=(5, 9000, 65)),
    W.Spec("dec-d64-g32", "bf16", 64, 2, 64, 100000, decode_lens=(129, 3000)),
    # one or two waves of work per range (kv heads x ceil(G / 16)): the other waves of each
    # workgroup exit at once
    W.Spec("dec-1kv-g8", "bf16", 8, 1, 128, 100000, decode_lens=(1, 2, 31, 32, 33, 97, 128, 129, 5000)),
    W.Spec("dec-2kv-g4", "bf16", 8, 2, 128, 100000, decode_lens=(1, 50, 300, 7000)),
    W.Spec("dec-1kv-g32-d64", "bf16", 32, 1, 64, 100000, decode_lens=(3, 65, 2000)),
    W.Spec("dec-1kv-many", "bf16", 16, 1, 128, 200000, decode_batch=200, decode_range=(1, 300)),
    W.Spec("dec-1kv-plan", "bf16", 8, 1, 64, 100000, decode_batch=1100, decode_range=(1, 40)),
    W.Spec("dec-many", "bf16", 32, 8, 128, 400000, decode_batch=96, decode_range=(1, 3000)),
    # head_dim 64 with more than 1,024 requests: the separate plan kernel
    W.Spec("dec-d64-plan", "bf16", 16, 4, 64, 100000, decode_batch=1200, decode_range=(1, 40)),
]


@pytest.mark.parametrize("variant", ["normal", "peaked", "needle"])
@pytest.mark.parametrize("spec", SMALL, ids=lambda s: s.name)
def test_decode_small(spec, variant):
    wl = W.make_workload(spec, 601, variant)
    say(f"decode {spec.name}/{variant}: B={wl.decode.batch} max_L={wl.decode.max_seq_len} "
        f"splits={R.decode_num_splits(R.BF16, wl.decode.batch, wl.decode.max_seq_len, spec.n_kv_heads)}")
    dw, outs = run_all(wl)
    kp, vp = stored_pools(wl)
    assert_close(out_f64(outs["decode"]), oracle_decode(wl, kp, vp), spec.dtype, f"{spec.name}/{variant}")


@pytest.mark.parametrize("variant", ["normal", "peaked", "needle"])
@pytest.mark.parametrize("spec", [
    W.Spec("dec-fp32-d64", "fp32", 4, 4, 64, 20000, decode_lens=(1, 64, 65, 1000, 3000)),
    W.Spec("dec-fp32-d128-g3", "fp32", 12, 4, 128, 20000, decode_lens=(2, 500, 4100)),
], ids=lambda s: s.name)
def test_decode_fp32(spec, variant):
    wl = W.make_workload(spec, 602, variant)
    dw, outs = run_all(wl)
    kp, vp = stored_pools(wl)
    assert_close(out_f64(outs["decode"]), oracle_decode(wl, kp, vp), "fp32", f"{spec.name}/{variant}")


@pytest.mark.parametrize("seed_off", [0, 100, 200])
def test_decode_64req_full(seed_off):
    """64 requests, contexts 512..4096, 32 q / 8 kv heads: every output against the oracle."""
    spec = W.CONFIGS[2]
    wl = W.make_workload(spec, W.TIMING_SEEDS[2] + seed_off)
    say(f"{spec.name} seed {W.TIMING_SEEDS[2] + seed_off}: generated")
    dw, outs = run_all(wl)
    kp, vp = stored_pools(wl)
    assert_close(out_f64(outs["decode"]), oracle_decode(wl, kp, vp), "bf16", f"{spec.name} seed+{seed_off}")


@pytest.mark.parametrize("variant", ["normal", "peaked", "needle"])
def test_decode_64req_variants(variant):
    spec = W.CONFIGS[2]
    wl = W.make_workload(spec, W.TIMING_SEEDS[2], variant)
    dw, outs = run_all(wl)
    kp, vp = stored_pools(wl)
    assert_close(out_f64(outs["decode"]), oracle_decode(wl, kp, vp), "bf16", f"{spec.name}/{variant}")


def test_single_key_returns_value_bitwise():
    """seq_len 1: p = exp2(0) = 1 and l = 1, so the output is the V row exactly (bf16 in, bf16 out)."""
    spec = W.Spec("one-key", "bf16", 32, 8, 128, 1000, decode_lens=(1, 1, 1))
    wl = W.make_workload(spec, 603)
    dw, outs = run_all(wl)
    got = to_host_bits(outs["decode"])
    G = 4
    for b in range(3):  # each request's only key is its current token, new row b
        for h in range(32):
            assert np.array_equal(got[b, h], wl.v_new[b, h // G])


def test_slot_permutation_is_bitwise_invariant_and_deterministic():
    spec = W.Spec("perm", "bf16", 32, 8, 128, 60000, decode_lens=(3, 700, 5000, 9999))
    wl = W.make_workload(spec, 604)
    dw, outs = run_all(wl)
    a = to_host_bits(outs["decode"]).copy()
    # run again: bitwise identical
    decode(dw, wl)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(dw.dec["o"]), a)
    # relabel every slot
    perm = np.random.default_rng(5).permutation(spec.num_slots)
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
    decode(dw, wl)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(dw.dec["o"]), a)


def test_gqa_equals_repeated_kv():
    """G=4 over kv heads vs. G=1 over repeat-interleaved kv heads: same per-head arithmetic."""
    spec = W.Spec("gqa", "bf16", 16, 4, 128, 30000, decode_lens=(5, 300, 2000))
    wl = W.make_workload(spec, 605)
    dw, outs = run_all(wl)
    a = to_host_bits(outs["decode"])
    kp, vp = stored_pools(wl)
    k_mha = to_dev(np.repeat(kp, 4, axis=1))
    v_mha = to_dev(np.repeat(vp, 4, axis=1))
    o2 = torch.empty_like(dw.dec["o"])
    d = dw.dec
    R.decode_attention(d["q"], o2, k_mha, v_mha, dw.req_to_token, d["req_pool_indices"], d["seq_lens"],
                       d["max_seq_len"], wl.sm_scale)
    torch.cuda.synchronize()
    b = to_host_bits(o2)
    ref = oracle_decode(wl, kp, vp)
    assert_close(oracle.to_f64(b), ref, "bf16", "repeated-kv MHA")
    # Splits differ (n_kv_heads enters the split rule) so only rounding-level agreement is expected.
    assert_close(oracle.to_f64(a), oracle.to_f64(b), "bf16", "GQA vs MHA")


def test_empty_batch_is_noop():
    spec = W.Spec("e", "bf16", 8, 2, 128, 100, decode_lens=(3,))
    wl = W.make_workload(spec, 606)
    dw = upload(wl)
    d = dw.dec
    R.decode_attention(d["q"][:0], d["o"][:0], dw.k_pool, dw.v_pool, dw.req_to_token, d["req_pool_indices"][:0],
                       d["seq_lens"][:0], d["max_seq_len"], wl.sm_scale)
    torch.cuda.synchronize()


# ---- the balanced key stream: ranges that hold many requests, requests spread over many ranges,
# empty requests, and streams long enough that the 4096-key range cap needs more than one
# resident round of workgroups.

def test_many_tiny_requests_share_ranges():
    """3,000 requests of 1..80 keys: one 256-key range overlaps up to 64 requests."""
    spec = W.Spec("dec-tiny-many", "bf16", 32, 8, 128, 400000, decode_batch=3000, decode_range=(1, 80))
    wl = W.make_workload(spec, 607)
    say(f"{spec.name}: B={wl.decode.batch} total keys={int(wl.decode.seq_lens.sum())}")
    dw, outs = run_all(wl)
    kp, vp = stored_pools(wl)
    assert_close(out_f64(outs["decode"]), oracle_decode(wl, kp, vp), "bf16", spec.name)


def test_one_long_request_among_short_ones():
    """A 131,072-key request spans many ranges; 40 short ones share ranges with its ends."""
    lens = (3, 64, 65, 700) * 5 + (131072,) + (1, 129, 4000, 63) * 5
    spec = W.Spec("dec-one-long", "bf16", 32, 8, 128, 200000, decode_lens=lens)
    wl = W.make_workload(spec, 608, "peaked")
    dw, outs = run_all(wl)
    kp, vp = stored_pools(wl)
    assert_close(out_f64(outs["decode"]), oracle_decode(wl, kp, vp), "bf16", spec.name)


def test_empty_requests_write_zeros():
    """Requests with seq_len 0 (or below) get all-zero rows; the others are unaffected."""
    spec = W.Spec("dec-empty", "bf16", 16, 4, 128, 60000, decode_lens=(500, 7, 3000, 64, 1, 2000, 300, 5))
    wl = W.make_workload(spec, 609)
    dw, outs = run_all(wl)
    kp, vp = stored_pools(wl)
    full = to_host_bits(outs["decode"]).copy()
    empty = [1, 3, 4, 7]
    sl = dw.dec["seq_lens"].clone()
    sl[empty[:3]] = 0
    sl[empty[3]] = -5
    d = dw.dec
    o2 = torch.full_like(d["o"], 7)
    R.decode_attention(d["q"], o2, dw.k_pool, dw.v_pool, dw.req_to_token, d["req_pool_indices"], sl,
                       d["max_seq_len"], wl.sm_scale)
    torch.cuda.synchronize()
    got = to_host_bits(o2)
    assert not got[empty].any(), "empty requests must give zero rows"
    keep = [b for b in range(wl.decode.batch) if b not in empty]
    # the other requests see the same keys as before; their partials now sit at other places
    assert_close(oracle.to_f64(got[keep]), oracle_decode(wl, kp, vp, requests=keep), "bf16", "non-empty")
    assert_close(oracle.to_f64(got[keep]), oracle.to_f64(full[keep]), "bf16", "vs all-present run")


def test_stream_longer_than_one_resident_round():
    """520 x 4096 keys over 2 kv heads: ranges clamp at 4096 keys and the grid exceeds one
    resident round (512 ranges); sampled requests against the oracle."""
    spec = W.Spec("dec-rounds", "bf16", 8, 2, 64, 2200000, decode_batch=520, decode_range=(4000, 4096))
    wl = W.make_workload(spec, 610, "peaked")
    B, L = wl.decode.batch, wl.decode.max_seq_len
    grid = R.decode_num_splits(R.BF16, B, L, spec.n_kv_heads)
    say(f"{spec.name}: total keys={int(wl.decode.seq_lens.sum())} grid={grid}")
    assert grid > 512
    dw, outs = run_all(wl)
    kp, vp = stored_pools(wl)
    reqs = sorted(set([0, 1, 2, B // 2, B - 2, B - 1]) | set(np.random.default_rng(1).choice(B, 20, replace=False).tolist()))
    assert_close(out_f64(outs["decode"])[reqs], oracle_decode(wl, kp, vp, requests=reqs), "bf16", spec.name)


def test_decode_on_a_side_stream_keeps_its_workspace():
    """The binding allocates the workspace on the caller's behalf and the kernels run on a side
    stream; right after the call returns, a new allocation of the same size on the current
    stream is filled. The workspace block must not be handed out again before the side stream
    has passed the DECODE kernels: the result still matches the oracle."""
    spec = W.Spec("side-stream", "bf16", 32, 8, 128, 200000, decode_lens=(3000, 9000, 20000, 513, 64))
    wl = W.make_workload(spec, 611)
    dw = upload(wl)
    store(dw)
    x = dw.dec
    nb = R.decode_workspace_bytes(R.BF16, wl.decode.batch, x["max_seq_len"], 32, 8, 128)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    x["o"].record_stream(side)
    R.decode_attention(x["q"], x["o"], dw.k_pool, dw.v_pool, dw.req_to_token, x["req_pool_indices"],
                       x["seq_lens"], x["max_seq_len"], wl.sm_scale, stream=side)
    junk = torch.empty(nb, dtype=torch.uint8, device=x["q"].device)
    junk.fill_(0xFF)
    torch.cuda.synchronize()
    kp, vp = stored_pools(wl)
    assert_close(out_f64(x["o"]), oracle_decode(wl, kp, vp), "bf16", "decode on a side stream")


def test_decode_workspace_serves_calls_of_several_shapes():
    """One workspace, sized for the largest call, serves DECODE calls of different batches and
    lengths in a row (nothing in it carries over between calls), and an empty request among
    others gets a zero row while the others still match the oracle."""
    specs = [W.Spec("ws-a", "bf16", 32, 8, 128, 300000, decode_batch=40, decode_range=(1, 5000)),
             W.Spec("ws-b", "bf16", 16, 4, 128, 100000, decode_lens=(3, 9000, 700)),
             W.Spec("ws-c", "bf16", 32, 8, 128, 300000, decode_batch=64, decode_range=(100, 3000))]
    need = max(R.decode_workspace_bytes(R.BF16, 64, 9000, 32, 8, 128), R.decode_workspace_bytes(R.BF16, 3, 9000, 16, 4, 128))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    for i, spec in enumerate(specs + specs[:1]):
        wl = W.make_workload(spec, 640 + i)
        dw = upload(wl)
        store(dw)
        x = dw.dec
        R.decode_attention(x["q"], x["o"], dw.k_pool, dw.v_pool, dw.req_to_token, x["req_pool_indices"],
                           x["seq_lens"], x["max_seq_len"], wl.sm_scale, workspace=ws)
        torch.cuda.synchronize()
        kp, vp = stored_pools(wl)
        assert_close(out_f64(x["o"]), oracle_decode(wl, kp, vp), "bf16", f"shared workspace call {i} ({spec.name})")
        ws.fill_(0xAB)   # stale contents must not matter to the next call
    # an empty request (seq_len 0) among others: zero output row, the others unchanged
    wl = W.make_workload(specs[0], 650)
    dw = upload(wl)
    store(dw)
    x = dw.dec
    lens = x["seq_lens"].clone()
    lens[7] = 0
    x["o"].fill_(float("nan"))
    R.decode_attention(x["q"], x["o"], dw.k_pool, dw.v_pool, dw.req_to_token, x["req_pool_indices"], lens,
                       x["max_seq_len"], wl.sm_scale, workspace=ws)
    torch.cuda.synchronize()
    assert np.all(to_host_bits(x["o"])[7] == 0)
    keep = [b for b in range(wl.decode.batch) if b != 7]
    kp, vp = stored_pools(wl)
    assert_close(out_f64(x["o"])[keep], oracle_decode(wl, kp, vp, requests=keep), "bf16", "batch with an empty request")
