"""Full-size parity on the shared-prefix, mixed chunked-prefill and long-context workloads, in
the launch configuration the benchmark times (kv_store, then EXTEND and DECODE on one pool),
each in its normal, peaked and needle variant.

What the oracle computes per workload:
* shared prefix (32 requests x 256 new tokens on one 4,096-token prefix): every EXTEND row;
* mixed chunk (2,048 new tokens on a 14,336-token prefix + 128 DECODE requests): every EXTEND
  row and every DECODE request;
* long context (8,192 new tokens on a 65,536-token prefix + 8 DECODE requests of 32K-128K
  keys): one token in every 32 consecutive suffix tokens, at a position that cycles through
  the 32 (so every group of 32 tokens -- all 64 heads -- is compared at one token), the first
  and last suffix tokens, and every DECODE request. The oracle would need minutes for all 8,192
  rows over 65K-74K keys.

Long contexts make plain outputs tiny (~1e-3), so the needle and peaked variants matter there:
a wrong or missing key range moves their outputs by O(1).
"""

import numpy as np
import pytest
import torch

from prefix_cached_paged_amd import workloads as W

from parity import assert_close, oracle_decode, oracle_extend, out_f64, run_all, say, stored_pools

pytestmark = pytest.mark.gpu

VARIANTS = [(0, "normal"), (100, "peaked"), (200, "needle")]


def every_row(wl):
    return None


def one_in_32(wl):
    e = wl.extend
    toks = set()
    for b in range(e.batch):
        n = int(e.extend_lens[b])
        s0 = int(e.extend_start_loc[b])
        toks |= {s0, s0 + n - 1}
        for t in range(0, n, 32):
            k = (t // 32) % 32
            toks.add(s0 + min(n - 1, t + k))
    return sorted(toks)


def check(cfg, seed_off, variant, rows):
    spec = W.CONFIGS[cfg]
    seed = W.TIMING_SEEDS[cfg] + seed_off
    say(f"{spec.name} seed {seed} {variant}: generating")
    wl = W.make_workload(spec, seed, variant)
    say("running kv_store + extend + decode")
    dw, outs = run_all(wl)
    got_e = out_f64(outs["extend"]) if "extend" in outs else None
    got_d = out_f64(outs["decode"]) if "decode" in outs else None
    del dw, outs
    torch.cuda.empty_cache()
    kp, vp = stored_pools(wl)
    if got_e is not None:
        toks = rows(wl)
        say(f"oracle: {'all' if toks is None else len(toks)} of {wl.extend.total_tokens} extend rows")
        ref = oracle_extend(wl, kp, vp, tokens=toks)
        assert_close(got_e if toks is None else got_e[toks], ref, "bf16", f"{spec.name}/{variant} extend")
    if got_d is not None:
        say(f"oracle: all {wl.decode.batch} decode requests")
        assert_close(got_d, oracle_decode(wl, kp, vp), "bf16", f"{spec.name}/{variant} decode")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("seed_off,variant", VARIANTS)
def test_shared_prefix_batch(seed_off, variant):
    check(3, seed_off, variant, every_row)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("seed_off,variant", VARIANTS)
def test_mixed_chunk_batch(seed_off, variant):
    check(4, seed_off, variant, every_row)


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("seed_off,variant", VARIANTS)
def test_long_context_batch(seed_off, variant):
    check(5, seed_off, variant, one_in_32)
