"""Full-size parity on the mixed chunked-prefill and long-context workloads, in the launch
configuration the benchmark times (kv_store, then EXTEND and DECODE on one pool).

The oracle computes sampled rows one by one: the first, last and tile-boundary suffix rows plus
a seeded random sample, and a seeded sample of DECODE requests (all requests for the
long-context batch). Long contexts make plain outputs tiny (~1e-3), so the needle and peaked
variants run too: there a wrong or missing key range moves outputs by O(1).
"""

import numpy as np
import pytest
import torch

from prefix_cached_paged_amd import workloads as W

from parity import assert_close, oracle_decode, oracle_extend, out_f64, run_all, say, stored_pools

pytestmark = pytest.mark.gpu


def sampled_tokens(wl, n_random, rng):
    e = wl.extend
    toks = []
    for b in range(e.batch):
        n = int(e.extend_lens[b])
        s0 = int(e.extend_start_loc[b])
        pick = {0, 1, n - 1, n - 2, min(n - 1, 63), min(n - 1, 64), min(n - 1, 255), min(n - 1, 256)}
        pick |= set(rng.choice(n, size=min(n, n_random), replace=False).tolist())
        toks += [s0 + i for i in sorted(pick) if 0 <= i < n]
    return toks


def check(cfg, seed, variant, n_tok, n_req):
    spec = W.CONFIGS[cfg]
    say(f"{spec.name} seed {seed} {variant}: generating")
    wl = W.make_workload(spec, seed, variant)
    say("running kv_store + extend + decode")
    dw, outs = run_all(wl)
    got_e = out_f64(outs["extend"])
    got_d = out_f64(outs["decode"])
    del dw, outs
    torch.cuda.empty_cache()
    kp, vp = stored_pools(wl)
    rng = np.random.default_rng(seed)
    toks = sampled_tokens(wl, n_tok, rng)
    say(f"oracle: {len(toks)} extend rows")
    assert_close(got_e[toks], oracle_extend(wl, kp, vp, tokens=toks), "bf16", f"config{cfg}/{variant} extend")
    B = wl.decode.batch
    reqs = sorted(rng.choice(B, size=min(B, n_req), replace=False).tolist())
    say(f"oracle: {len(reqs)} decode requests")
    assert_close(got_d[reqs], oracle_decode(wl, kp, vp, requests=reqs), "bf16", f"config{cfg}/{variant} decode")


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("seed_off,variant", [(0, "normal"), (100, "peaked")])
def test_mixed_chunk_batch(seed_off, variant):
    check(4, W.TIMING_SEEDS[4] + seed_off, variant, n_tok=24, n_req=24)


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("seed_off,variant", [(0, "normal"), (100, "needle")])
def test_long_context_batch(seed_off, variant):
    check(5, W.TIMING_SEEDS[5] + seed_off, variant, n_tok=6, n_req=8)
