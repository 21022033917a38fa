"""kv_store on the GPU: written rows equal the new rows bit for bit; every other slot is unchanged."""

import numpy as np
import pytest
import torch

from prefix_cached_paged_amd import workloads as W
from prefix_cached_paged_amd.device import to_host_bits, upload

from parity import say, store, stored_pools

pytestmark = pytest.mark.gpu

SPECS = [
    W.Spec("store-bf16", "bf16", 32, 8, 128, 20000, extend_prefix=(100, 0, 7), extend_lens=(300, 1, 255),
           decode_lens=(1, 40, 999)),
    W.Spec("store-fp32-d64", "fp32", 4, 4, 64, 1024, extend_prefix=(0, 16, 64, 128), extend_lens=(32, 16, 8, 1)),
    W.Spec("store-bf16-d64", "bf16", 8, 1, 64, 5000, decode_lens=(3, 70)),
    W.Spec("store-bf16-h2", "bf16", 4, 2, 128, 4096, extend_prefix=(10,), extend_lens=(2000,)),
]


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: s.name)
def test_kv_store_bitwise(spec):
    wl = W.make_workload(spec, 501)
    say(f"kv_store {spec.name}: n_new={wl.store_loc.size}")
    dw = upload(wl)
    store(dw)
    torch.cuda.synchronize()
    kp, vp = stored_pools(wl)
    assert np.array_equal(to_host_bits(dw.k_pool).view(np.uint8), kp.view(np.uint8))
    assert np.array_equal(to_host_bits(dw.v_pool).view(np.uint8), vp.view(np.uint8))


def test_kv_store_empty_is_a_noop():
    spec = SPECS[0]
    wl = W.make_workload(spec, 502)
    dw = upload(wl)
    before = to_host_bits(dw.k_pool).copy()
    from prefix_cached_paged_amd import rax as R
    R.kv_store(dw.k_new[:0], dw.v_new[:0], dw.store_loc[:0], dw.k_pool, dw.v_pool)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(dw.k_pool), before)
