"""HIP graph capture of one step of the path: kv_store, EXTEND and DECODE on one stream.

The calls allocate nothing and clear nothing with memsets (the DECODE workspace is the
caller's), so a step can be captured once and replayed. The EXTEND of the step-replay test
splits its keys (3 requests x 8 kv heads x 5 row tiles = 120 workgroups: two splits and a
merge); its workspace comes from the binding, through torch's allocator, which serves it from
the graph's pool during capture. Every replay is checked bit for bit against an eager run of
the same step, with eager work and synchronisations between replays, and the inputs are
changed between replays to show that the graph reads the live buffers.
"""

import pytest
import torch

from prefix_cached_paged_amd import rax as R
from prefix_cached_paged_amd import workloads as W
from prefix_cached_paged_amd.device import upload

from parity import assert_close, oracle_decode, oracle_extend, out_f64, say, stored_pools

pytestmark = pytest.mark.gpu


def step(dw, wl, ws):
    R.kv_store(dw.k_new, dw.v_new, dw.store_loc, dw.k_pool, dw.v_pool)
    e = dw.ext
    R.extend_attention(e["q"], e["o"], dw.k_pool, dw.v_pool, dw.req_to_token, e["req_pool_indices"],
                       e["prefix_lens"], e["extend_lens"], e["extend_start_loc"], e["max_extend_len"],
                       e["max_seq_len"], wl.sm_scale)
    d = dw.dec
    R.decode_attention(d["q"], d["o"], dw.k_pool, dw.v_pool, dw.req_to_token, d["req_pool_indices"],
                       d["seq_lens"], d["max_seq_len"], wl.sm_scale, workspace=ws)


def bits(t):
    return t.view(torch.int16).clone()


# batch 40 computes the DECODE plan inside the split kernel; batch 1,500 runs the plan kernel.
@pytest.mark.parametrize("batch,ctx", [(40, (1, 2000)), (1500, (1, 150))])
def test_graph_replays_match_eager(batch, ctx):
    spec = W.Spec("graph", "bf16", 32, 8, 128, 400000, extend_prefix=(1000, 0, 3000),
                  extend_lens=(300, 64, 129), decode_batch=batch, decode_range=ctx)
    wl = W.make_workload(spec, 611)
    dw = upload(wl)
    d = dw.dec
    ws = torch.empty(max(1, R.decode_workspace_bytes(R.BF16, d["q"].shape[0], d["max_seq_len"], spec.n_q_heads,
                                                     spec.n_kv_heads, spec.head_dim)),
                     dtype=torch.uint8, device="cuda")
    say(f"graph test: decode batch {batch}")
    step(dw, wl, ws)
    torch.cuda.synchronize()
    ref_e, ref_d = bits(dw.ext["o"]), bits(d["o"])
    kp, vp = stored_pools(wl)
    assert_close(out_f64(dw.ext["o"]), oracle_extend(wl, kp, vp), "bf16", "eager extend")
    assert_close(out_f64(d["o"]), oracle_decode(wl, kp, vp), "bf16", "eager decode")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(dw, wl, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(dw, wl, ws)
    torch.cuda.synchronize()

    for r in range(3):
        dw.ext["o"].fill_(float("nan"))
        d["o"].zero_()
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(dw.ext["o"]), ref_e), f"replay {r}: extend differs from eager"
        assert torch.equal(bits(d["o"]), ref_d), f"replay {r}: decode differs from eager"

    # new queries: the replay must see them, and agree with an eager step on the same inputs
    dw.ext["q"].mul_(-2)
    d["q"].mul_(2)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    got_e, got_d = bits(dw.ext["o"]), bits(d["o"])
    assert not torch.equal(got_d, ref_d)
    step(dw, wl, ws)
    torch.cuda.synchronize()
    assert torch.equal(bits(dw.ext["o"]), got_e), "replay with new queries differs from eager"
    assert torch.equal(bits(d["o"]), got_d), "replay with new queries differs from eager"


def test_graph_replays_fp8_paged_ragged():
    """The FP8, page-table and ragged (fused store) entry points under capture: three replays,
    each bit for bit equal to the eager calls."""
    spec = W.Spec("graph-x", "bf16", 32, 8, 128, 131072, extend_prefix=(1000, 0, 3000),
                  extend_lens=(300, 64, 129), decode_batch=40, decode_range=(1, 2000), page_size=16)
    wl = W.make_workload(spec, 612)
    dw = upload(wl)
    e, d = dw.ext, dw.dec
    n = wl.extend.total_tokens
    pt = torch.from_numpy(wl.page_table).cuda()
    ks = vs = 4.0 * spec.sigma / 448
    k8 = torch.empty(dw.k_pool.shape, dtype=torch.uint8, device="cuda")
    v8 = torch.empty_like(k8)
    R.kv_store(dw.k_new, dw.v_new, dw.store_loc, dw.k_pool, dw.v_pool)     # every used row of the bf16 pool
    used = torch.unique(torch.from_numpy(wl.req_to_token[wl.req_to_token >= 0]).long()).int().cuda()
    R.kv_store_fp8(dw.k_pool[used.long()], dw.v_pool[used.long()], used, k8, v8, ks, vs)
    ws = torch.empty(R.decode_workspace_bytes(R.BF16, d["q"].shape[0], d["max_seq_len"], spec.n_q_heads,
                                              spec.n_kv_heads, spec.head_dim), dtype=torch.uint8, device="cuda")
    outs = {k: torch.empty_like(e["q"]) for k in ("e8", "ep", "er")}
    outs.update({k: torch.empty_like(d["q"]) for k in ("d8", "dp")})
    rest = (dw.req_to_token, e["req_pool_indices"], e["prefix_lens"], e["extend_lens"], e["extend_start_loc"],
            e["max_extend_len"], e["max_seq_len"], wl.sm_scale)

    def step():
        R.kv_store_fp8(dw.k_new, dw.v_new, dw.store_loc, k8, v8, ks, vs)
        R.extend_attention_fp8(e["q"], outs["e8"], k8, v8, *rest, ks, vs)
        R.decode_attention_fp8(d["q"], outs["d8"], k8, v8, dw.req_to_token, d["req_pool_indices"], d["seq_lens"],
                               d["max_seq_len"], wl.sm_scale, ks, vs, workspace=ws)
        R.extend_attention_paged(e["q"], outs["ep"], dw.k_pool, dw.v_pool, pt, spec.page_size, *rest[1:])
        R.decode_attention_paged(d["q"], outs["dp"], dw.k_pool, dw.v_pool, pt, spec.page_size,
                                 d["req_pool_indices"], d["seq_lens"], d["max_seq_len"], wl.sm_scale, workspace=ws)
        R.extend_attention_ragged(e["q"], outs["er"], dw.k_new[:n], dw.v_new[:n], dw.k_pool, dw.v_pool, *rest,
                                  store_loc=dw.store_loc[:n])

    step()
    torch.cuda.synchronize()
    ref = {k: bits(v) for k, v in outs.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        for v in outs.values():
            v.fill_(float("nan"))
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(bits(v), ref[k]), f"replay {r}: {k} differs from eager"
