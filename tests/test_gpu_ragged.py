"""Ragged EXTEND on the GPU: suffix K/V read from the just-computed rows, with and without the
fused store, against the float64 oracle's ragged reading.

The pools hold NaN at every suffix slot before the call, so a suffix key read from the pool
instead of from the new rows poisons the output. With the store, the pools afterwards must be
exactly the oracle's kv_store of the suffix rows; without it, untouched. The ragged output is
also compared bit for bit with kv_store followed by the pool-reading EXTEND: the kernels use
the same arithmetic in the same order and only the source of the suffix rows differs.
"""

import numpy as np
import pytest
import torch

import oracle
from prefix_cached_paged_amd import rax as R
from prefix_cached_paged_amd import workloads as W
from prefix_cached_paged_amd.device import to_dev, to_host_bits, upload

from parity import assert_close, extend, out_f64, say, store

pytestmark = pytest.mark.gpu

SPECS = [
    W.Spec("rag-g4", "bf16", 32, 8, 128, 100000, extend_prefix=(0, 1, 63, 64, 500, 3000),
           extend_lens=(1, 40, 65, 128, 77, 300)),
    W.Spec("rag-g1", "bf16", 4, 4, 128, 50000, extend_prefix=(0, 200, 37), extend_lens=(300, 129, 0)),
    W.Spec("rag-g2", "bf16", 8, 4, 128, 50000, extend_prefix=(10, 0), extend_lens=(190, 64)),
    W.Spec("rag-g8", "bf16", 64, 8, 128, 100000, extend_prefix=(1000, 5), extend_lens=(33, 200)),
    W.Spec("rag-g16", "bf16", 16, 1, 128, 50000, extend_prefix=(129, 0), extend_lens=(20, 17)),
    W.Spec("rag-g32", "bf16", 32, 1, 128, 50000, extend_prefix=(0, 640), extend_lens=(500, 9)),
    W.Spec("rag-shared", "bf16", 32, 8, 128, 100000, extend_prefix=(700,) * 5, extend_lens=(100, 1, 64, 129, 3),
           shared_prefix=True),
    W.Spec("rag-prefill", "bf16", 32, 8, 128, 50000, extend_prefix=(0, 0, 0), extend_lens=(1000, 64, 2)),
    W.Spec("rag-d64-g4", "bf16", 32, 8, 64, 100000, extend_prefix=(0, 63, 500), extend_lens=(129, 65, 300)),
    W.Spec("rag-fp32-d64", "fp32", 4, 4, 64, 4000, extend_prefix=(0, 16, 64, 128), extend_lens=(32, 16, 8, 1)),
    W.Spec("rag-fp32-d128-g3", "fp32", 6, 2, 128, 20000, extend_prefix=(0, 300), extend_lens=(70, 65)),
    W.Spec("rag-g7", "bf16", 28, 4, 128, 100000, extend_prefix=(0, 63, 500), extend_lens=(100, 37, 73)),
    # one (request, kv head) pair whose row tiles are shared out over all XCDs (fused store)
    W.Spec("rag-1pair", "bf16", 8, 1, 128, 50000, extend_prefix=(200,), extend_lens=(900,)),
    # key splits (few row tiles; the last split of each row tile does the fused store)
    W.Spec("rag-split", "bf16", 32, 8, 128, 50000, extend_prefix=(9000, 0), extend_lens=(90, 30)),
]


def run_ragged(dw, wl, store_loc):
    e = dw.ext
    n = wl.extend.total_tokens
    R.extend_attention_ragged(e["q"], e["o"], dw.k_new[:n], dw.v_new[:n], dw.k_pool, dw.v_pool, dw.req_to_token,
                              e["req_pool_indices"], e["prefix_lens"], e["extend_lens"], e["extend_start_loc"],
                              e["max_extend_len"], e["max_seq_len"], wl.sm_scale,
                              store_loc=dw.store_loc[:n] if store_loc else None)
    torch.cuda.synchronize()
    return e["o"]


@pytest.mark.parametrize("fused_store", [False, True])
@pytest.mark.parametrize("variant", ["normal", "peaked"])
@pytest.mark.parametrize("spec", SPECS, ids=lambda s: s.name)
def test_ragged_extend(spec, variant, fused_store):
    wl = W.make_workload(spec, 801, variant)
    e = wl.extend
    n = e.total_tokens
    say(f"ragged {spec.name}/{variant} store={fused_store}: B={e.batch} N={n}")
    dw = upload(wl)
    dw.ext["o"].fill_(float("nan"))
    got = out_f64(run_ragged(dw, wl, fused_store))
    ref = oracle.extend_attention(e.q, wl.k_pool, wl.v_pool, wl.req_to_token, e.req_pool_indices, e.prefix_lens,
                                  e.extend_lens, e.extend_start_loc, spec.n_kv_heads, wl.sm_scale,
                                  suffix=(wl.k_new[:n], wl.v_new[:n]))
    assert_close(got, ref, spec.dtype, f"ragged {spec.name}/{variant}")
    if fused_store:
        want_k, want_v = oracle.kv_store(wl.k_pool, wl.v_pool, wl.k_new[:n], wl.v_new[:n], wl.store_loc[:n])
    else:
        want_k, want_v = wl.k_pool, wl.v_pool
    assert np.array_equal(to_host_bits(dw.k_pool), want_k, equal_nan=spec.dtype == "fp32"), "K pool"
    assert np.array_equal(to_host_bits(dw.v_pool), want_v, equal_nan=spec.dtype == "fp32"), "V pool"


@pytest.mark.parametrize("variant", ["normal", "peaked"])
@pytest.mark.parametrize("spec", [SPECS[0], SPECS[3], SPECS[6], SPECS[8], SPECS[9], SPECS[10]], ids=lambda s: s.name)
def test_ragged_is_bitwise_store_then_extend(spec, variant):
    """The ragged call with its fused store equals the store followed by the pool-reading call,
    bit for bit (both split the keys of few row tiles the same way)."""
    wl = W.make_workload(spec, 802, variant)
    dw = upload(wl)
    got = run_ragged(dw, wl, True).clone()
    store(dw)
    want = extend(dw, wl)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16) if spec.dtype == "bf16" else got.view(torch.int32),
                       want.view(torch.int16) if spec.dtype == "bf16" else want.view(torch.int32))


# Ragged suffix with the prefix read through a page table: page sizes 2 to 64, a prefix that
# ends inside a page, head_dim 64, fp32. Against the oracle's ragged reading (the equivalent
# token table), the pools after the fused store, and bit for bit against the token-table ragged
# call on the same slots.
PAGED_SPECS = [
    W.Spec("ragpg16-g4", "bf16", 32, 8, 128, 131072, extend_prefix=(0, 1, 63, 500, 3000),
           extend_lens=(40, 65, 128, 77, 300), page_size=16),
    W.Spec("ragpg64-g8", "bf16", 64, 8, 128, 131072, extend_prefix=(1000, 5), extend_lens=(33, 200), page_size=64),
    W.Spec("ragpg2-g1", "bf16", 4, 4, 128, 65536, extend_prefix=(0, 37), extend_lens=(300, 129), page_size=2),
    W.Spec("ragpg8-d64", "bf16", 32, 8, 64, 65536, extend_prefix=(63, 208), extend_lens=(65, 190), page_size=8),
    W.Spec("ragpg4-fp32", "fp32", 4, 4, 64, 8192, extend_prefix=(0, 16, 64, 130), extend_lens=(32, 16, 8, 1),
           page_size=4),
    W.Spec("ragpg16-g5", "bf16", 40, 8, 128, 131072, extend_prefix=(70, 0), extend_lens=(103, 52), page_size=16),
    W.Spec("ragpg16-3pair", "bf16", 12, 3, 128, 65536, extend_prefix=(50,), extend_lens=(600,), page_size=16),
    W.Spec("ragpg16-split", "bf16", 32, 8, 128, 65536, extend_prefix=(7000,), extend_lens=(80,), page_size=16),
]


def run_ragged_paged(dw, wl, store_loc):
    e = dw.ext
    n = wl.extend.total_tokens
    R.extend_attention_ragged_paged(e["q"], e["o"], dw.k_new[:n], dw.v_new[:n], dw.k_pool, dw.v_pool,
                                    to_dev(wl.page_table), wl.spec.page_size, e["req_pool_indices"],
                                    e["prefix_lens"], e["extend_lens"], e["extend_start_loc"], e["max_extend_len"],
                                    e["max_seq_len"], wl.sm_scale,
                                    store_loc=dw.store_loc[:n] if store_loc else None)
    torch.cuda.synchronize()
    return e["o"]


@pytest.mark.parametrize("fused_store", [False, True])
@pytest.mark.parametrize("variant", ["normal", "peaked"])
@pytest.mark.parametrize("spec", PAGED_SPECS, ids=lambda s: s.name)
def test_ragged_paged_extend(spec, variant, fused_store):
    wl = W.make_workload(spec, 803, variant)
    e = wl.extend
    n = e.total_tokens
    say(f"ragged paged {spec.name}/{variant} P={spec.page_size} store={fused_store}: B={e.batch} N={n}")
    dw = upload(wl)
    dw.ext["o"].fill_(float("nan"))
    got_t = run_ragged_paged(dw, wl, fused_store).clone()
    got = out_f64(got_t)
    ref = oracle.extend_attention_paged(e.q, wl.k_pool, wl.v_pool, wl.page_table, spec.page_size,
                                        e.req_pool_indices, e.prefix_lens, e.extend_lens, e.extend_start_loc,
                                        spec.n_kv_heads, wl.sm_scale, suffix=(wl.k_new[:n], wl.v_new[:n]))
    assert_close(got, ref, spec.dtype, f"ragged paged {spec.name}/{variant}")
    if fused_store:
        want_k, want_v = oracle.kv_store(wl.k_pool, wl.v_pool, wl.k_new[:n], wl.v_new[:n], wl.store_loc[:n])
    else:
        want_k, want_v = wl.k_pool, wl.v_pool
    assert np.array_equal(to_host_bits(dw.k_pool), want_k, equal_nan=spec.dtype == "fp32"), "K pool"
    assert np.array_equal(to_host_bits(dw.v_pool), want_v, equal_nan=spec.dtype == "fp32"), "V pool"
    tok = run_ragged(dw, wl, False)
    as_int = (lambda t: t.view(torch.int16)) if spec.dtype == "bf16" else (lambda t: t.view(torch.int32))
    assert torch.equal(as_int(got_t), as_int(tok)), "paged and token-table ragged EXTEND differ"
