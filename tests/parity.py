"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI, compute the oracle
on the same seeded inputs, compare.

Tolerances (element by element, in float64 of the difference):
* bf16: |gpu - oracle| <= 1e-2 + half_ulp_bf16(|oracle|) element by element, and
  ||gpu - oracle||_2 / ||oracle||_2 <= 1e-2.
  Inputs are exact bf16 values on both sides. The 1e-2 absolute bound is the arithmetic's
  budget; the output itself is delivered in bf16, and rounding a value to bf16 moves it by up
  to half a unit in the last place of its binade, 2^(floor(log2 |o|) - 8) (0.0078 for
  |o| in [2, 4), 0.0156 in [4, 8)), so exactly that much is added per element. The GPU also
  rounds P to bf16 before P V (relative 2^-9 per weight). The relative RMS bound keeps the
  check meaningful on long contexts where outputs are tiny.
* fp32: max-abs <= 1e-5 and relative RMS <= 1e-6 (fp32 accumulation over <= a few thousand
  terms, no reduced-precision step).
"""

from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle
from prefix_cached_paged_amd import rax as R
from prefix_cached_paged_amd.device import to_host_bits, upload

TOL = {"bf16": dict(max_abs=1e-2, half_ulp=True, rel_rms=1e-2),
       "fp32": dict(max_abs=1e-5, half_ulp=False, rel_rms=1e-6)}


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Half a bf16 unit in the last place of |x|'s binade: 2^(floor(log2 |x|) - 8); 0 at 0.

    bf16 carries 8 significant bits, so its spacing in [2^k, 2^(k+1)) is 2^(k-7)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(a)                 # a = f 2^e with f in [0.5, 1): floor(log2 a) = e - 1
    return np.where(a > 0, np.ldexp(1.0, e - 9), 0.0)


def bound(ref: np.ndarray, dtype: str) -> np.ndarray:
    """Per-element bound on |gpu - oracle|."""
    tol = TOL[dtype]
    return tol["max_abs"] + (half_ulp_bf16(ref) if tol["half_ulp"] else 0.0)


def say(msg: str):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def out_f64(t: torch.Tensor) -> np.ndarray:
    return oracle.to_f64(to_host_bits(t))


def errors(got: np.ndarray, ref: np.ndarray) -> dict:
    d = got - ref
    nref = float(np.sqrt(np.sum(ref * ref)))
    return dict(max_abs=float(np.max(np.abs(d))) if d.size else 0.0,
                max_ref=float(np.max(np.abs(ref))) if ref.size else 0.0,
                rel_rms=float(np.sqrt(np.sum(d * d)) / nref) if nref > 0 else 0.0,
                finite=bool(np.all(np.isfinite(got))))


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str):
    e = errors(got, ref)
    say(f"{what}: max_abs={e['max_abs']:.3e} max|ref|={e['max_ref']:.3e} rel_rms={e['rel_rms']:.3e}")
    tol = TOL[dtype]
    assert e["finite"], f"{what}: non-finite output"
    excess = float(np.max(np.abs(got - ref) - bound(ref, dtype))) if ref.size else -1.0
    assert excess <= 0.0, f"{what}: error above {tol['max_abs']} (+ bf16 half-ulp) by {excess:.3e}: {e}"
    assert e["rel_rms"] <= tol["rel_rms"], f"{what}: {e}"
    return e


def store(dw, stream=None):
    R.kv_store(dw.k_new, dw.v_new, dw.store_loc, dw.k_pool, dw.v_pool, stream=stream)


def extend(dw, wl, stream=None):
    x = dw.ext
    R.extend_attention(x["q"], x["o"], dw.k_pool, dw.v_pool, dw.req_to_token, x["req_pool_indices"],
                       x["prefix_lens"], x["extend_lens"], x["extend_start_loc"], x["max_extend_len"],
                       x["max_seq_len"], wl.sm_scale, stream=stream)
    return x["o"]


def decode(dw, wl, stream=None):
    x = dw.dec
    R.decode_attention(x["q"], x["o"], dw.k_pool, dw.v_pool, dw.req_to_token, x["req_pool_indices"],
                       x["seq_lens"], x["max_seq_len"], wl.sm_scale, stream=stream)
    return x["o"]


def stored_pools(wl):
    return oracle.kv_store(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.store_loc)


def oracle_extend(wl, kp, vp, tokens=None):
    e = wl.extend
    return oracle.extend_attention(e.q, kp, vp, wl.req_to_token, e.req_pool_indices, e.prefix_lens,
                                   e.extend_lens, e.extend_start_loc, wl.spec.n_kv_heads, wl.sm_scale,
                                   tokens=tokens)


def oracle_decode(wl, kp, vp, requests=None):
    d = wl.decode
    return oracle.decode_attention(d.q, kp, vp, wl.req_to_token, d.req_pool_indices, d.seq_lens,
                                   wl.spec.n_kv_heads, wl.sm_scale, requests=requests)


def run_all(wl, do_extend=True, do_decode=True):
    """Upload, store the new rows, run EXTEND and DECODE; return (device workload, outputs)."""
    dw = upload(wl)
    store(dw)
    outs = {}
    if do_extend and dw.ext is not None:
        outs["extend"] = extend(dw, wl)
    if do_decode and dw.dec is not None:
        outs["decode"] = decode(dw, wl)
    torch.cuda.synchronize()
    return dw, outs
