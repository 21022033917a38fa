"""Pins of the oracle's FP8 E4M3 KV pool (decode of each byte, the store's encoding, and where
the per-pool scales enter attention). CPU only.

Independent references: torch's float8_e4m3fn conversions (a library implementation of the
same OCP format), values fixed by the format's definition, and closed forms of attention.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as F

ALL = np.arange(256, dtype=np.uint8)


def test_decode_matches_torch_for_every_byte():
    ours = oracle.e4m3_bits_to_f64(ALL)
    ref = torch.from_numpy(ALL).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x30, 0.5),
    (0x38, 1.0), (0x39, 1.125), (0x40, 2.0), (0x4C, 6.0), (0x77, 240.0), (0x7E, 448.0),
    (0xB8, -1.0), (0xFE, -448.0)])
def test_decode_closed_forms(code, value):
    assert oracle.e4m3_bits_to_f64(np.array([code], np.uint8))[0] == value


def test_decode_specials_and_symmetry():
    v = oracle.e4m3_bits_to_f64(ALL)
    assert math.isnan(v[0x7F]) and math.isnan(v[0xFF])
    assert np.sum(np.isnan(v)) == 2
    assert v[0x80] == 0.0 and np.signbit(v[0x80]) and not np.signbit(v[0x00])
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)                      # codes 0..126 increase
    assert np.array_equal(v[0x80:0xFF], -pos)            # sign bit mirrors


def test_round_trip_of_every_finite_byte():
    v = oracle.e4m3_bits_to_f64(ALL)
    fin = ~np.isnan(v)
    assert np.array_equal(oracle.e4m3_round(v[fin]), ALL[fin])


def test_ties_go_to_the_even_code_and_neighbours_to_the_nearest():
    v = oracle.e4m3_bits_to_f64(np.arange(127, dtype=np.uint8))
    lo, hi = v[:-1], v[1:]
    mid = 0.5 * (lo + hi)
    codes = np.arange(126)
    want_mid = np.where(codes % 2 == 0, codes, codes + 1)
    assert np.array_equal(oracle.e4m3_round(mid), want_mid)
    assert np.array_equal(oracle.e4m3_round(-mid), want_mid | 0x80)
    up = np.nextafter(mid, np.inf)
    down = np.nextafter(mid, -np.inf)
    assert np.array_equal(oracle.e4m3_round(up), codes + 1)
    assert np.array_equal(oracle.e4m3_round(down), codes)


def nearest_by_search(x):
    """Brute force: the E4M3 value nearest to each x (ties to the even code), by comparing with
    every finite code's value."""
    v = oracle.e4m3_bits_to_f64(np.arange(127, dtype=np.uint8))
    a = np.abs(np.asarray(x, np.float64))[:, None]
    d = np.abs(v[None, :] - a)
    best = d.min(axis=1, keepdims=True)
    cand = np.where(d == best, np.arange(127)[None, :], 10 ** 6)
    even = np.where((cand % 2 == 0) & (cand < 10 ** 6), cand, 10 ** 6).min(axis=1)
    code = np.where(even < 10 ** 6, even, cand.min(axis=1))
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def test_rounding_matches_a_brute_force_nearest_search():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.uniform(-448, 448, 4000), rng.normal(0, 0.02, 4000), rng.normal(0, 3, 4000),
                        rng.uniform(-2.0 ** -5, 2.0 ** -5, 4000)])
    v = oracle.e4m3_bits_to_f64(np.arange(127, dtype=np.uint8))
    mids = 0.5 * (v[:-1] + v[1:])
    x = np.concatenate([x, mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9)])
    assert np.array_equal(oracle.e4m3_round(x), nearest_by_search(x))


def test_encode_matches_torch_in_range():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.normal(0, 1, 20000), rng.normal(0, 100, 20000), rng.uniform(-448, 448, 20000),
                        rng.normal(0, 0.01, 20000)]).astype(np.float32)
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_round(x.astype(np.float64)), ref)


def bf16(x):
    """bfloat16 bits of float32 values that are exactly representable in bf16."""
    b = np.asarray(x, np.float32).view(np.uint32)
    assert np.all(b & 0xFFFF == 0)
    return (b >> 16).astype(np.uint16)


def test_quantize_scales_clamps_and_keeps_sign_of_zero():
    assert list(oracle.quantize_bf16(bf16([3.0, -3.0, 0.0, -0.0]), 0.5)) == [0x4C, 0xCC, 0x00, 0x80]
    assert list(oracle.quantize_bf16(bf16([2.0 ** 20, -2.0 ** 20, 2.0 ** -20]), 1.0)) == [0x7E, 0xFE, 0x00]
    assert list(oracle.quantize_bf16(bf16([-2.0 ** -20]), 1.0)) == [0x80]
    # the multiplier is the float32 reciprocal of the scale: 1/3 rounds in float32
    y = np.float32(1.5) * np.float32(1.0 / 3.0)
    assert oracle.quantize_bf16(bf16([1.5]), 3.0)[0] == oracle.e4m3_round(np.array([float(y)]))[0]
    with pytest.raises(ValueError):
        oracle.quantize_bf16(bf16([1.0]), 0.0)
    with pytest.raises(ValueError):
        oracle.quantize_bf16(np.array([0x7FC0], np.uint16), 1.0)   # NaN input


def test_store_writes_only_the_named_rows():
    rng = np.random.default_rng(8)
    S, H, D, n = 20, 2, 8, 5
    kp = rng.integers(0, 0x7F, (S, H, D), dtype=np.uint8)
    vp = rng.integers(0x80, 0xFF, (S, H, D), dtype=np.uint8)
    kn = bf16(np.round(rng.normal(0, 2, (n, H, D)) * 8) / 8)
    vn = bf16(np.round(rng.normal(0, 2, (n, H, D)) * 8) / 8)
    loc = np.array([3, 17, 0, 9, 11])
    k2, v2 = oracle.kv_store_fp8(kp, vp, kn, vn, loc, 0.25, 0.5)
    other = np.setdiff1d(np.arange(S), loc)
    assert np.array_equal(k2[other], kp[other]) and np.array_equal(v2[other], vp[other])
    assert np.array_equal(k2[loc], oracle.quantize_bf16(kn, 0.25))
    assert np.array_equal(v2[loc], oracle.quantize_bf16(vn, 0.5))
    with pytest.raises(ValueError):
        oracle.kv_store_fp8(kp, vp, kn, vn, np.array([3, 3, 0, 9, 11]))


def _one_request(k_bytes, v_bytes, q):
    L, D = k_bytes.shape
    kp = k_bytes.reshape(L, 1, D).astype(np.uint8)
    vp = v_bytes.reshape(L, 1, D).astype(np.uint8)
    r2t = np.arange(L, dtype=np.int32)[None, :]
    return kp, vp, r2t, np.zeros(1, np.int32), np.array([L], np.int32), np.asarray(q, np.float64)[None, None, :]


def test_v_scale_multiplies_the_output():
    """q = 0: uniform weights, so the output is v_scale times the mean of the decoded V rows."""
    rng = np.random.default_rng(9)
    kb = rng.integers(0, 0x7E, (6, 8)).astype(np.uint8)
    vb = rng.integers(0, 0x7E, (6, 8)).astype(np.uint8)
    kp, vp, r2t, rpi, sl, q = _one_request(kb, vb, np.zeros(8))
    o = oracle.decode_attention(q, kp, vp, r2t, rpi, sl, 1, 0.3, k_scale=5.0, v_scale=0.75)
    want = 0.75 * oracle.e4m3_bits_to_f64(vb).mean(axis=0)
    assert np.allclose(o[0, 0], want, rtol=1e-14, atol=0)


def test_k_scale_multiplies_the_scores():
    """Two keys, one all-zero: weight of the other is 1 / (1 + exp(-c)), c = sm_scale k_scale q.k."""
    kb = np.zeros((2, 4), np.uint8)
    kb[0] = [0x38, 0x40, 0x30, 0x00]                    # 1, 2, 0.5, 0
    vb = np.zeros((2, 4), np.uint8)
    vb[0, 0] = 0x38                                     # V row 0 = (1, 0, 0, 0), row 1 = 0
    q = np.array([0.5, -0.25, 1.0, 3.0])
    kp, vp, r2t, rpi, sl, qq = _one_request(kb, vb, q)
    for ks in (0.5, 1.0, 3.0):
        o = oracle.decode_attention(qq, kp, vp, r2t, rpi, sl, 1, 0.7, k_scale=ks, v_scale=1.0)
        c = 0.7 * ks * (0.5 * 1 - 0.25 * 2 + 1.0 * 0.5)
        assert abs(o[0, 0, 0] - 1.0 / (1.0 + math.exp(-c))) < 1e-15
