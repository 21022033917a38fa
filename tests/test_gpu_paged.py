"""Page tables (page size P > 1) on the GPU: EXTEND and DECODE through page_table against the
float64 oracle, and bit for bit against the token-granular path on the same workload.

The generator places every request's positions in pages of P slots and writes both a page
table and the equivalent token table, so the two paths read the same slots in the same order
and must agree exactly. Unreferenced slots hold NaN, so a wrong page or offset poisons the
output.
"""

import numpy as np
import pytest
import torch

import oracle
from prefix_cached_paged_amd import rax as R
from prefix_cached_paged_amd import workloads as W
from prefix_cached_paged_amd.device import to_dev, upload

from parity import assert_close, decode, extend, out_f64, say, store, stored_pools

pytestmark = pytest.mark.gpu

EXT_SPECS = [
    # key splits (few row tiles) through a page table
    W.Spec("pg16-split", "bf16", 32, 8, 128, 65536, extend_prefix=(9000,), extend_lens=(70,), page_size=16),
    W.Spec("pg16-g4", "bf16", 32, 8, 128, 131072, extend_prefix=(0, 1, 63, 64, 500, 3000),
           extend_lens=(1, 40, 65, 128, 77, 300), page_size=16),
    W.Spec("pg8-g1", "bf16", 4, 4, 128, 65536, extend_prefix=(0, 200, 37), extend_lens=(300, 129, 0), page_size=8),
    W.Spec("pg64-g8", "bf16", 64, 8, 128, 131072, extend_prefix=(1000, 5), extend_lens=(33, 200), page_size=64),
    W.Spec("pg32-g16", "bf16", 16, 1, 128, 65536, extend_prefix=(129, 0), extend_lens=(20, 17), page_size=32),
    W.Spec("pg2-g32", "bf16", 32, 1, 128, 65536, extend_prefix=(0, 640), extend_lens=(500, 9), page_size=2),
    W.Spec("pg16-d64-g2", "bf16", 8, 4, 64, 65536, extend_prefix=(0, 208, 1024), extend_lens=(190, 64, 77),
           page_size=16),
    W.Spec("pg16-shared", "bf16", 32, 8, 128, 131072, extend_prefix=(704,) * 5, extend_lens=(100, 1, 64, 129, 3),
           shared_prefix=True, page_size=16),
    W.Spec("pg4-fp32", "fp32", 4, 4, 64, 4096, extend_prefix=(0, 16, 64, 128), extend_lens=(32, 16, 8, 1),
           page_size=4),
    W.Spec("pg16-g7", "bf16", 28, 4, 128, 131072, extend_prefix=(0, 63, 1000), extend_lens=(100, 37, 73),
           page_size=16),
]
DEC_SPECS = [
    W.Spec("pg16-dec", "bf16", 32, 8, 128, 131072, decode_lens=(1, 2, 15, 16, 17, 257, 1000, 2500), page_size=16),
    W.Spec("pg64-dec-g8", "bf16", 64, 8, 128, 131072, decode_lens=(5, 513, 4000, 64), page_size=64),
    W.Spec("pg8-dec-many", "bf16", 32, 8, 128, 262144, decode_batch=1500, decode_range=(1, 120), page_size=8),
    W.Spec("pg32-dec-d64", "bf16", 16, 4, 64, 65536, decode_lens=(1, 64, 999, 5000), page_size=32),
    W.Spec("pg16-dec-g24", "bf16", 48, 2, 128, 65536, decode_lens=(17, 2500, 700), page_size=16),
    W.Spec("pg16-dec-1kv", "bf16", 8, 1, 128, 65536, decode_lens=(1, 40, 130, 3000), page_size=16),
    W.Spec("pg16-dec-fp32", "fp32", 8, 2, 128, 16384, decode_lens=(1, 40, 700), page_size=16),
]


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("variant", ["normal", "needle"])
@pytest.mark.parametrize("spec", EXT_SPECS, ids=lambda s: s.name)
def test_paged_extend(spec, variant):
    wl = W.make_workload(spec, 901, variant)
    e = wl.extend
    say(f"paged extend {spec.name}/{variant}: P={spec.page_size} B={e.batch} N={e.total_tokens}")
    dw = upload(wl)
    store(dw)
    x = dw.ext
    pt = to_dev(wl.page_table)
    R.extend_attention_paged(x["q"], x["o"], dw.k_pool, dw.v_pool, pt, spec.page_size, x["req_pool_indices"],
                             x["prefix_lens"], x["extend_lens"], x["extend_start_loc"], x["max_extend_len"],
                             x["max_seq_len"], wl.sm_scale)
    torch.cuda.synchronize()
    got = x["o"].clone()
    kp, vp = stored_pools(wl)
    ref = oracle.extend_attention_paged(e.q, kp, vp, wl.page_table, spec.page_size, e.req_pool_indices,
                                        e.prefix_lens, e.extend_lens, e.extend_start_loc, spec.n_kv_heads,
                                        wl.sm_scale)
    assert_close(out_f64(got), ref, spec.dtype, f"paged extend {spec.name}/{variant}")
    tok = extend(dw, wl)
    torch.cuda.synchronize()
    assert torch.equal(bits(got), bits(tok)), "paged and token-table EXTEND differ"


@pytest.mark.parametrize("variant", ["normal", "peaked"])
@pytest.mark.parametrize("spec", DEC_SPECS, ids=lambda s: s.name)
def test_paged_decode(spec, variant):
    wl = W.make_workload(spec, 902, variant)
    d = wl.decode
    say(f"paged decode {spec.name}/{variant}: P={spec.page_size} B={d.batch}")
    dw = upload(wl)
    store(dw)
    x = dw.dec
    pt = to_dev(wl.page_table)
    R.decode_attention_paged(x["q"], x["o"], dw.k_pool, dw.v_pool, pt, spec.page_size, x["req_pool_indices"],
                             x["seq_lens"], x["max_seq_len"], wl.sm_scale)
    torch.cuda.synchronize()
    got = x["o"].clone()
    kp, vp = stored_pools(wl)
    ref = oracle.decode_attention_paged(d.q, kp, vp, wl.page_table, spec.page_size, d.req_pool_indices, d.seq_lens,
                                        spec.n_kv_heads, wl.sm_scale)
    assert_close(out_f64(got), ref, spec.dtype, f"paged decode {spec.name}/{variant}")
    tok = decode(dw, wl)
    torch.cuda.synchronize()
    assert torch.equal(bits(got), bits(tok)), "paged and token-table DECODE differ"


def test_page_size_one_is_the_token_path():
    spec = W.Spec("pg1", "bf16", 32, 8, 128, 50000, extend_prefix=(300, 0), extend_lens=(200, 64),
                  decode_lens=(1, 700))
    wl = W.make_workload(spec, 903)
    dw = upload(wl)
    store(dw)
    x, y = dw.ext, dw.dec
    want_e, want_d = bits(extend(dw, wl)).clone(), bits(decode(dw, wl)).clone()
    R.extend_attention_paged(x["q"], x["o"], dw.k_pool, dw.v_pool, dw.req_to_token, 1, x["req_pool_indices"],
                             x["prefix_lens"], x["extend_lens"], x["extend_start_loc"], x["max_extend_len"],
                             x["max_seq_len"], wl.sm_scale)
    R.decode_attention_paged(y["q"], y["o"], dw.k_pool, dw.v_pool, dw.req_to_token, 1, y["req_pool_indices"],
                             y["seq_lens"], y["max_seq_len"], wl.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(bits(x["o"]), want_e) and torch.equal(bits(y["o"]), want_d)
