"""CPU checks of the C ABI: the library loads, exports what the header declares, and rejects bad
arguments on the host before anything is launched (no compute call is made here)."""

import ctypes
import os
import subprocess

import pytest

from prefix_cached_paged_amd import rax as R

pytestmark = pytest.mark.skipif(not os.path.exists(R.library_path()), reason="librax.so not built")

FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def lib():
    return R.load()


def test_every_declared_symbol_is_exported():
    names = R.declared_symbols()
    assert set(names) == {"rax_version", "rax_status_str", "rax_kv_store", "rax_extend_workspace_bytes",
                          "rax_extend_attention", "rax_decode_workspace_bytes", "rax_decode_attention",
                          "rax_decode_num_splits", "rax_kv_store_fp8", "rax_extend_attention_fp8",
                          "rax_decode_attention_fp8", "rax_extend_attention_ragged",
                          "rax_extend_attention_paged", "rax_decode_attention_paged",
                          "rax_extend_attention_paged_fp8", "rax_decode_attention_paged_fp8",
                          "rax_extend_attention_ragged_paged",
                          "rax_check_workspace_bytes", "rax_check_kv_store", "rax_check_extend",
                          "rax_check_decode", "rax_decode_attention_noalloc"}
    out = subprocess.run(["nm", "-D", "--defined-only", R.library_path()], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in names:
        assert n in exported, n
        assert hasattr(lib(), n)


def test_version_and_status_names():
    assert lib().rax_version() == 100
    for code, name in enumerate(["RAX_OK", "RAX_ERR_NULL", "RAX_ERR_SHAPE", "RAX_ERR_DTYPE",
                                 "RAX_ERR_UNSUPPORTED", "RAX_ERR_WORKSPACE", "RAX_ERR_LAUNCH",
                                 "RAX_ERR_SCRATCH"]):
        assert lib().rax_status_str(code).decode() == name
    assert lib().rax_status_str(99).decode() == "unknown status"


def kv_store(**kw):
    a = dict(dtype=0, k_new=FAKE, v_new=FAKE, loc=FAKE, n_new=4, k_pool=FAKE, v_pool=FAKE, num_slots=16,
             n_kv_heads=2, head_dim=128, stream=None)
    a.update(kw)
    return lib().rax_kv_store(*a.values())


def test_kv_store_validation():
    assert kv_store(dtype=7) == 3
    assert kv_store(n_new=-1) == 2
    assert kv_store(n_new=17) == 2
    assert kv_store(num_slots=0) == 2
    assert kv_store(n_kv_heads=0) == 2
    assert kv_store(head_dim=96) == 4
    assert kv_store(k_pool=None) == 1
    assert kv_store(loc=None) == 1
    assert kv_store(n_new=0, k_pool=None) == 0  # empty: no-op, nothing enqueued


def extend(**kw):
    a = dict(dtype=0, q=FAKE, o=FAKE, k_pool=FAKE, v_pool=FAKE, num_slots=1024, r2t=FAKE, r2t_stride=512,
             rpi=FAKE, prefix=FAKE, ext=FAKE, start=FAKE, batch=2, total=64, max_ext=40, max_seq=300, hq=8,
             hkv=2, d=128, scale=0.088, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return lib().rax_extend_attention(*a.values())


def test_extend_validation():
    assert extend(dtype=2) == 3
    assert extend(batch=-1) == 2
    assert extend(max_seq=600) == 2          # beyond the table row
    assert extend(max_ext=301) == 2          # an extend longer than the longest sequence
    assert extend(max_ext=65, total=64) == 2
    assert extend(hq=6, hkv=4) == 2          # not a multiple
    assert extend(d=96) == 4
    assert extend(hq=6, hkv=2, batch=0, q=None) == 0     # group 3: the run-time group kernel
    assert extend(hq=128, hkv=2, batch=0, q=None) == 0   # group 64: 4 tokens per 256-row tile
    assert extend(hq=514, hkv=2) == 4        # group 257: not one token's heads per tile
    assert extend(d=32) == 4                 # head_dim 64 or 128 only
    assert extend(d=64, batch=0, q=None) == 0  # bf16 EXTEND: head_dim 64 too
    assert extend(dtype=1, d=64, batch=0, q=None) == 0           # fp32: head_dim 64 ...
    assert extend(dtype=1, hq=6, hkv=2, batch=0, q=None) == 0    # ... and any group
    assert extend(scale=float("nan")) == 2
    assert extend(q=None) == 1
    assert extend(start=None) == 1
    assert extend(batch=0, q=None) == 0      # empty batch
    assert extend(total=0, max_ext=0, q=None) == 0
    # few row tiles over a long context: the key splits need a workspace, and a missing or short
    # one is refused before any launch (the fp32 path needs none)
    big = dict(r2t_stride=16384, max_seq=16000, num_slots=1 << 20)
    need = lib().rax_extend_workspace_bytes(0, 2, 64, 40, 16000, 8, 2, 128)
    assert need > 0
    assert extend(**big) == 5
    assert extend(ws=FAKE, ws_bytes=need - 1, **big) == 5
    assert extend(dtype=1, batch=0, q=None, **big) == 0


def decode(**kw):
    a = dict(dtype=0, q=FAKE, o=FAKE, k_pool=FAKE, v_pool=FAKE, num_slots=1024, r2t=FAKE, r2t_stride=512,
             rpi=FAKE, seq=FAKE, batch=3, max_seq=300, hq=8, hkv=2, d=128, scale=0.088, ws=None, ws_bytes=0,
             stream=None)
    a.update(kw)
    return lib().rax_decode_attention(*a.values())


def test_decode_validation():
    assert decode(dtype=5) == 3
    assert decode(max_seq=513) == 2
    assert decode(max_seq=0) == 2
    assert decode(hq=8, hkv=3) == 2
    assert decode(d=32) == 4
    assert decode(hq=34, hkv=2, batch=0, q=None) == 0   # group 17: two waves of heads per kv head
    assert decode(hq=2 * 257, hkv=2) == 4    # group 257 has no kernel
    assert decode(dtype=1, hq=34, hkv=2, batch=0, q=None) == 0   # fp32: any group
    assert decode(d=64, batch=0, q=None) == 0                     # bf16 DECODE: head_dim 64 too
    assert decode(seq=None) == 1
    # workspace: bf16 needs one, too small or missing is refused before any launch
    need = lib().rax_decode_workspace_bytes(0, 3, 300, 8, 2, 128)
    assert need > 0
    assert decode(ws=None, ws_bytes=0) == 5
    assert decode(ws=FAKE, ws_bytes=need - 1) == 5
    assert decode(batch=0, q=None) == 0


def a256(x):
    return (x + 255) // 256 * 256


def test_decode_workspace_size():
    # ranges per kv-head group: one resident round (768 workgroups of 4 kv heads, 3 per CU, for
    # bf16 and FP8 pools alike), or enough 4096-key ranges for every request at max_seq_len,
    # whichever is larger
    # (one wave per kv head and 16 query heads: wave heads = hkv * ceil(G / 16))
    for B, L, hq, hkv in [(64, 4096, 32, 8), (8, 131072, 64, 8), (1, 1, 4, 4), (128, 8192, 32, 8),
                          (4096, 32768, 32, 8), (16, 1000, 64, 32), (8, 4096, 16, 1), (8, 4096, 32, 1),
                          (4, 1000, 8, 2), (4, 1000, 48, 1)]:
        for dtype, resident in ((0, 768), (2, 768)):
            wheads = hkv * ((hq // hkv + 15) // 16)
            groups = (wheads + 3) // 4
            worst = B * ((L + 63) // 64 * 64)
            grid = max(max(1, resident // groups), (worst + 4095) // 4096)
            assert lib().rax_decode_num_splits(dtype, B, L, wheads) == grid
            parts = (B + grid) * hq
            want = 256 + a256((B + 1) * 8) + a256(grid * 4) + a256(parts * 128 * 4) + parts * 4
            assert lib().rax_decode_workspace_bytes(dtype, B, L, hq, hkv, 128) == want
    assert lib().rax_decode_workspace_bytes(1, 64, 4096, 32, 8, 128) == 0   # fp32 path needs none
    assert lib().rax_extend_workspace_bytes(0, 1, 2048, 2048, 16384, 32, 8, 128) == 0
    # few row tiles: S key splits of fp32 partial rows and log2-sum-exps (S = floor(256 / (pairs
    # x row tiles)), at most 16 and at most one per 512 keys of max_seq_len), over bf16 and FP8
    # pools alike; none for the fp32 path
    for B, N, E, L, hq, hkv, d in [(1, 100, 100, 10100, 32, 8, 128), (1, 100, 100, 10100, 8, 1, 128),
                                    (2, 137, 100, 12100, 32, 8, 64), (1, 2048, 2048, 4096, 32, 4, 128),
                                    (1, 64, 64, 700, 32, 8, 128), (1, 2048, 2048, 16384, 28, 4, 128),
                                    (1, 2048, 2048, 16384, 16, 1, 128)]:
        bq = 256 // (hq // hkv)
        work = B * hkv * ((E + bq - 1) // bq)
        S = 1 if work >= 256 else max(1, min(256 // work, (L + 63) // 64 // 8, 16))
        want = 0 if S == 1 else a256(S * N * hq * d * 4) + S * N * hq * 4
        assert lib().rax_extend_workspace_bytes(0, B, N, E, L, hq, hkv, d) == want, (B, N, E, L, hq, hkv, d)
        assert lib().rax_extend_workspace_bytes(2, B, N, E, L, hq, hkv, d) == want
        assert lib().rax_extend_workspace_bytes(1, B, N, E, L, hq, hkv, d) == 0


def test_fp8_calls_check_scales_and_shapes_before_launching():
    L = lib()
    # kv_store_fp8(k_new, v_new, loc, n_new, k_pool, v_pool, num_slots, Hkv, D, k_scale, v_scale, stream)
    st = lambda **kw: L.rax_kv_store_fp8(kw.get("k", FAKE), FAKE, FAKE, kw.get("n", 4), FAKE, FAKE,
                                         kw.get("S", 100), 2, kw.get("D", 128), kw.get("ks", 1.0),
                                         kw.get("vs", 1.0), None)
    assert st(n=0) == 0
    assert st(ks=0.0) == 2 and st(vs=-1.0) == 2 and st(ks=float("nan")) == 2 and st(vs=float("inf")) == 2
    assert st(D=96) == 4
    assert st(n=200) == 2
    assert st(k=None) == 1
    # decode_attention_fp8(q, o, kp, vp, S, r2t, stride, rpi, seq, B, L, Hq, Hkv, D, sm, ks, vs, ws, wsb, stream)
    need = L.rax_decode_workspace_bytes(2, 3, 300, 8, 2, 128)
    # FP8 pools keep fewer split workgroups resident (wider iterations), so need at most as much
    assert 0 < need <= L.rax_decode_workspace_bytes(0, 3, 300, 8, 2, 128)
    dec = lambda **kw: L.rax_decode_attention_fp8(FAKE, FAKE, FAKE, FAKE, 1000, FAKE, 512, FAKE, FAKE,
                                                  kw.get("B", 3), 300, 8, 2, 128, 0.1, kw.get("ks", 1.0),
                                                  kw.get("vs", 1.0), kw.get("ws", FAKE), kw.get("wsb", need),
                                                  None)
    assert dec(ks=0.0) == 2 and dec(vs=float("nan")) == 2
    assert dec(B=0) == 0
    assert dec(ws=None, wsb=0) == 5
    # extend_attention_fp8(q, o, kp, vp, S, r2t, stride, rpi, pre, ext, start, B, N, maxe, maxL, Hq, Hkv, D,
    #                      sm, ks, vs, ws, wsb, stream)
    ext = lambda **kw: L.rax_extend_attention_fp8(FAKE, FAKE, FAKE, FAKE, 1000, FAKE, 512, FAKE, FAKE, FAKE,
                                                  FAKE, kw.get("B", 3), 100, 50, 300, kw.get("Hq", 8), 2,
                                                  kw.get("D", 128), 0.1, kw.get("ks", 1.0), kw.get("vs", 1.0),
                                                  None, 0, None)
    assert ext(ks=-2.0) == 2 and ext(vs=float("inf")) == 2 and ext(ks=float("nan")) == 2
    assert ext(B=0) == 0
    assert ext(D=32) == 4          # head_dim 64 or 128 only
    assert ext(Hq=6, B=0) == 0     # group 3: the run-time group kernel
    assert ext(Hq=2 * 257) == 4    # group 257 has no kernel
    assert L.rax_extend_workspace_bytes(2, 3, 100, 50, 300, 8, 2, 128) == 0


def test_ragged_extend_checks_before_launching():
    L = lib()
    # (dtype, q, o, k_new, v_new, store_loc, kp, vp, S, r2t, stride, rpi, pre, ext, start, B, N, maxe, maxL,
    #  Hq, Hkv, D, sm, ws, wsb, stream)
    rag = lambda **kw: L.rax_extend_attention_ragged(kw.get("dt", 0), FAKE, FAKE, kw.get("kn", FAKE), FAKE,
                                                     kw.get("loc", None), FAKE, FAKE, kw.get("S", 1000), FAKE,
                                                     512, FAKE, FAKE, FAKE, FAKE, kw.get("B", 3), kw.get("N", 100),
                                                     50, 300, 8, 2, kw.get("D", 128), 0.1, None, 0, None)
    assert rag(kn=None) == 1                 # no new rows
    assert rag(B=0) == 0 and rag(kn=None, B=0) == 0
    assert rag(dt=7) == 3
    assert rag(D=96) == 4
    assert rag(loc=FAKE, S=60, N=100) == 2   # more rows to store than slots


def test_paged_calls_check_page_size_and_table_width():
    L = lib()
    # (dtype, q, o, kp, vp, S, pt, pt_stride, P, rpi, pre, ext, start, B, N, maxe, maxL, Hq, Hkv, D, sm, ws, wsb, st)
    ext = lambda **kw: L.rax_extend_attention_paged(0, FAKE, FAKE, FAKE, FAKE, 4096, kw.get("pt", FAKE),
                                                    kw.get("stride", 32), kw.get("P", 16), FAKE, FAKE, FAKE, FAKE,
                                                    kw.get("B", 3), 100, 50, kw.get("L", 300), 8, 2, 128, 0.1,
                                                    None, 0, None)
    for bad in (0, 3, 12, -16, 1 << 21):
        assert ext(P=bad) == 2, bad
    assert ext(L=600) == 2               # 32 pages of 16 cover 512 positions only
    assert ext(B=0) == 0
    assert ext(pt=None) == 1
    # (dtype, q, o, kp, vp, S, pt, pt_stride, P, rpi, seq, B, maxL, Hq, Hkv, D, sm, ws, wsb, stream)
    dec = lambda **kw: L.rax_decode_attention_paged(0, FAKE, FAKE, FAKE, FAKE, 4096, kw.get("pt", FAKE),
                                                    kw.get("stride", 8), kw.get("P", 64), FAKE, FAKE,
                                                    kw.get("B", 3), kw.get("L", 512), 8, 2, 128, 0.1, FAKE,
                                                    1 << 30, None)
    assert dec(P=48) == 2
    assert dec(L=513) == 2               # 8 pages of 64
    assert dec(B=0) == 0
    assert dec(pt=None) == 1


def test_paged_fp8_calls_check_page_size_scales_and_table_width():
    L = lib()
    # (q, o, kp, vp, S, pt, pt_stride, P, rpi, pre, ext, start, B, N, maxe, maxL, Hq, Hkv, D, sm, ks, vs, ws, wsb,
    #  stream)
    ext = lambda **kw: L.rax_extend_attention_paged_fp8(FAKE, FAKE, FAKE, FAKE, 4096, kw.get("pt", FAKE),
                                                        kw.get("stride", 32), kw.get("P", 16), FAKE, FAKE, FAKE,
                                                        FAKE, kw.get("B", 3), 100, 50, kw.get("L", 300), 8, 2,
                                                        kw.get("D", 128), 0.1, kw.get("ks", 1.0), 1.0, None, 0,
                                                        None)
    for bad in (0, 3, 12, -16, 1 << 21):
        assert ext(P=bad) == 2, bad
    assert ext(L=600) == 2               # 32 pages of 16 cover 512 positions only
    assert ext(ks=0.0) == 2 and ext(ks=float("inf")) == 2
    assert ext(D=32) == 4
    assert ext(B=0) == 0
    assert ext(pt=None) == 1
    # (q, o, kp, vp, S, pt, pt_stride, P, rpi, seq, B, maxL, Hq, Hkv, D, sm, ks, vs, ws, wsb, stream)
    dec = lambda **kw: L.rax_decode_attention_paged_fp8(FAKE, FAKE, FAKE, FAKE, 4096, kw.get("pt", FAKE),
                                                        kw.get("stride", 8), kw.get("P", 64), FAKE, FAKE,
                                                        kw.get("B", 3), kw.get("L", 512), 8, 2, 128, 0.1, 1.0,
                                                        kw.get("vs", 1.0), FAKE, 1 << 30, None)
    assert dec(P=48) == 2
    assert dec(L=513) == 2               # 8 pages of 64
    assert dec(vs=-1.0) == 2
    assert dec(B=0) == 0
    assert dec(pt=None) == 1


def test_binding_checks_what_the_abi_cannot_see():
    """The C calls take one head_dim, one row count and the per-request arrays' length from the
    batch size; the binding compares the tensors' own shapes first (host tensors suffice: the
    checks run before any device pointer is taken)."""
    import torch
    bf = torch.bfloat16
    q = torch.zeros(6, 8, 128, dtype=bf)
    kp = torch.zeros(32, 2, 128, dtype=bf)
    r2t = torch.zeros(2, 16, dtype=torch.int32)
    ints = lambda n: torch.zeros(n, dtype=torch.int32)
    ext = lambda q, o, kp, vp, per: R.extend_attention(q, o, kp, vp, r2t, *per, 3, 16, 0.1)
    with pytest.raises(ValueError, match="head_dim"):
        ext(q, torch.zeros_like(q), torch.zeros(32, 2, 64, dtype=bf), torch.zeros(32, 2, 64, dtype=bf), [ints(2)] * 4)
    with pytest.raises(ValueError, match="q and o"):
        ext(q, torch.zeros(6, 8, 64, dtype=bf), kp, torch.zeros_like(kp), [ints(2)] * 4)
    with pytest.raises(ValueError, match="k_pool and v_pool"):
        ext(q, torch.zeros_like(q), kp, torch.zeros(31, 2, 128, dtype=bf), [ints(2)] * 4)
    with pytest.raises(ValueError, match="per-request"):
        ext(q, torch.zeros_like(q), kp, torch.zeros_like(kp), [ints(2), ints(2), ints(3), ints(2)])
    with pytest.raises(ValueError, match="2-D"):
        R.decode_attention(q, torch.zeros_like(q), kp, torch.zeros_like(kp), ints(16), ints(6), ints(6), 16, 0.1)
    with pytest.raises(ValueError, match="per-request"):
        R.decode_attention(q, torch.zeros_like(q), kp, torch.zeros_like(kp), r2t, ints(6), ints(5), 16, 0.1)
    with pytest.raises(ValueError, match="loc"):
        R.kv_store(torch.zeros(3, 2, 128, dtype=bf), torch.zeros(3, 2, 128, dtype=bf), ints(4), kp, torch.zeros_like(kp))
    with pytest.raises(ValueError, match="head_dim"):
        R.kv_store(torch.zeros(3, 2, 64, dtype=bf), torch.zeros(3, 2, 64, dtype=bf), ints(3), kp, torch.zeros_like(kp))
    with pytest.raises(ValueError, match="store_loc"):
        R.extend_attention_ragged(q, torch.zeros_like(q), torch.zeros(6, 2, 128, dtype=bf),
                                  torch.zeros(6, 2, 128, dtype=bf), kp, torch.zeros_like(kp), r2t, ints(2), ints(2),
                                  ints(2), ints(2), 3, 16, 0.1, store_loc=ints(5))


def test_check_calls_validate_before_launching():
    L = lib()
    assert L.rax_check_workspace_bytes(1) == 4 and L.rax_check_workspace_bytes(33) == 8
    assert L.rax_check_workspace_bytes(0) == 0
    ws = L.rax_check_workspace_bytes(1024)
    # kv_store: shapes, counts, workspace
    assert L.rax_check_kv_store(FAKE, -1, 1024, FAKE, ws, FAKE, None) == 2
    assert L.rax_check_kv_store(FAKE, 4, 0, FAKE, ws, FAKE, None) == 2
    assert L.rax_check_kv_store(FAKE, 4, 1024, FAKE, ws, None, None) == 1
    assert L.rax_check_kv_store(None, 4, 1024, FAKE, ws, FAKE, None) == 1
    assert L.rax_check_kv_store(FAKE, 4, 1024, FAKE, ws - 1, FAKE, None) == 5
    assert L.rax_check_kv_store(FAKE, 4, 1024, None, ws, FAKE, None) == 5

    def ext(**kw):
        a = dict(table=FAKE, rows=4, stride=512, page=1, rpi=FAKE, p=FAKE, e=FAKE, s=FAKE, batch=3, total=64,
                 max_ext=64, max_seq=300, slots=1024, ragged=0, store=None, ws=None, ws_bytes=0, counts=FAKE,
                 stream=None)
        a.update(kw)
        return L.rax_check_extend(*a.values())

    assert ext(page=3) == 2                      # not a power of two
    assert ext(page=1 << 21) == 2
    assert ext(max_seq=513) == 2                 # past the table row
    assert ext(page=4, stride=64, max_seq=257) == 2
    assert ext(rows=0) == 2
    assert ext(store=FAKE) == 2                  # a store without the ragged call
    assert ext(counts=None) == 1
    assert ext(e=None) == 1
    assert ext(ragged=1, store=FAKE) == 5        # the overlap check needs the bitmap
    assert ext(ragged=1, store=FAKE, ws=FAKE, ws_bytes=ws - 1) == 5

    def dec(**kw):
        a = dict(table=FAKE, rows=4, stride=512, page=1, rpi=FAKE, seq=FAKE, batch=3, max_seq=300, slots=1024,
                 counts=FAKE, stream=None)
        a.update(kw)
        return L.rax_check_decode(*a.values())

    assert dec(page=0) == 2
    assert dec(max_seq=600) == 2
    assert dec(slots=0) == 2
    assert dec(seq=None) == 1
    assert dec(counts=None) == 1


def decode_noalloc(**kw):
    a = dict(dtype=0, q=FAKE, o=FAKE, k_pool=FAKE, v_pool=FAKE, num_slots=1 << 20, r2t=FAKE, r2t_stride=8192,
             rpi=FAKE, seq=FAKE, batch=64, max_seq=4096, hq=32, hkv=8, d=128, scale=0.088, stream=None)
    a.update(kw)
    return lib().rax_decode_attention_noalloc(*a.values())


def test_noalloc_decode_checks_before_looking_up_its_scratch():
    """Host validation (as rax_decode_attention) and the scratch limit are decided before the
    static array is looked up or anything is enqueued: no GPU is needed for these."""
    assert R.DECODE_SCRATCH_BYTES == 32 << 20
    assert decode_noalloc(dtype=7) == 3
    assert decode_noalloc(batch=-1) == 2
    assert decode_noalloc(max_seq=9000) == 2           # beyond the table row
    assert decode_noalloc(hq=6, hkv=4) == 2
    assert decode_noalloc(d=96) == 4
    assert decode_noalloc(q=None) == 1
    assert decode_noalloc(batch=0) == 0                # empty: no-op
    # 1,000 requests of up to 8,192 keys need about 47 MiB of partials: refused
    nb = lib().rax_decode_workspace_bytes(0, 1000, 8192, 32, 8, 128)
    assert nb > R.DECODE_SCRATCH_BYTES
    assert decode_noalloc(batch=1000, max_seq=8192) == 7
    assert lib().rax_status_str(7).decode() == "RAX_ERR_SCRATCH"
    # the workload shapes fit: 64 requests of up to 4,096 keys, 8 of up to 131,072 with 64 q heads
    assert lib().rax_decode_workspace_bytes(0, 64, 4096, 32, 8, 128) <= R.DECODE_SCRATCH_BYTES
    assert lib().rax_decode_workspace_bytes(0, 8, 131072, 64, 8, 128) <= R.DECODE_SCRATCH_BYTES
