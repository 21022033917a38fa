"""The no-allocation DECODE entry point (rax_decode_attention_noalloc) through the C ABI.

It runs the kernels of rax_decode_attention with the plan and partials in the library's static
per-device scratch instead of a workspace, so its outputs must be those of the workspace call,
bit for bit, and match the oracle. Two calls in a row, the second with a smaller batch, check
that nothing of the first call's scratch contents leaks into the second.
"""

import numpy as np
import pytest
import torch

from prefix_cached_paged_amd import rax as R
from prefix_cached_paged_amd import workloads as W
from prefix_cached_paged_amd.device import to_host_bits, upload

from parity import assert_close, decode, oracle_decode, out_f64, say, store, stored_pools

pytestmark = pytest.mark.gpu

CASES = [
    (W.Spec("noalloc-large", "bf16", 32, 8, 128, 900000, decode_batch=96, decode_range=(1, 9000)), 631),
    (W.Spec("noalloc-small", "bf16", 32, 8, 128, 100000, decode_lens=(1, 65, 4097)), 632),
]


def run_noalloc(dw, wl):
    x = dw.dec
    R.decode_attention_noalloc(x["q"], x["o"], dw.k_pool, dw.v_pool, dw.req_to_token, x["req_pool_indices"],
                               x["seq_lens"], x["max_seq_len"], wl.sm_scale)
    return x["o"]


@pytest.mark.parametrize("variant", ["normal", "peaked"])
def test_noalloc_decode_equals_the_workspace_call(variant):
    for spec, seed in CASES:
        wl = W.make_workload(spec, seed, variant)
        d = wl.decode
        need = R.decode_workspace_bytes(R.BF16, d.batch, d.max_seq_len, spec.n_q_heads, spec.n_kv_heads,
                                        spec.head_dim)
        say(f"noalloc {spec.name}/{variant}: B={d.batch} max_L={d.max_seq_len} scratch use {need} of "
            f"{R.DECODE_SCRATCH_BYTES} bytes")
        assert 0 < need <= R.DECODE_SCRATCH_BYTES
        dw = upload(wl)
        store(dw)
        want = decode(dw, wl).clone()            # the workspace call
        torch.cuda.synchronize()
        dw.dec["o"].fill_(float("nan"))
        got = run_noalloc(dw, wl)
        torch.cuda.synchronize()
        assert np.array_equal(to_host_bits(got), to_host_bits(want)), f"{spec.name}: differs from the workspace call"
        kp, vp = stored_pools(wl)
        assert_close(out_f64(got), oracle_decode(wl, kp, vp), "bf16", f"noalloc {spec.name}/{variant}")
        del dw
        torch.cuda.empty_cache()


def test_noalloc_decode_refuses_shapes_beyond_its_scratch():
    spec = W.Spec("noalloc-one", "bf16", 32, 8, 128, 10000, decode_lens=(70,))
    wl = W.make_workload(spec, 633)
    dw = upload(wl)
    x = dw.dec
    with pytest.raises(R.RaxError, match="RAX_ERR_SCRATCH"):
        # a host bound of 1,000,000 keys per request sizes the ranges past the scratch
        R.decode_attention_noalloc(x["q"], x["o"], dw.k_pool, dw.v_pool,
                                   torch.zeros((1, 1 << 24), dtype=torch.int32, device=x["q"].device),
                                   x["req_pool_indices"].zero_(), x["seq_lens"], 1 << 24, wl.sm_scale)
