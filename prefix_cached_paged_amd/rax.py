"""Thin ctypes binding over librax.so (argument marshalling only).

Every function takes torch tensors that already live on the GPU, reads their data pointers
and shapes, and calls the C entry point of the same name on the current (or given) HIP stream.
No arithmetic of the method happens here. Tensors of ``torch.bfloat16`` or ``torch.float32``
select the element format. Raises ``RaxError`` with the library's status name on any error
status, and ``RuntimeError`` if the library has not been built.
"""

from __future__ import annotations

import ctypes
import os
import re

import torch  # imported before the library so that one HIP runtime serves the process

__all__ = [
    "RaxError", "BF16", "FP32", "load", "version", "kv_store", "extend_attention",
    "decode_attention", "decode_attention_noalloc", "DECODE_SCRATCH_BYTES", "extend_workspace_bytes",
    "decode_workspace_bytes", "decode_num_splits",
    "library_path", "declared_symbols", "FP8_E4M3", "kv_store_fp8", "decode_attention_fp8",
    "extend_attention_fp8", "extend_attention_ragged", "extend_attention_paged", "decode_attention_paged",
    "CHECK_ITEMS", "check_kv_store", "check_extend", "check_decode",
]

BF16 = 0
FP32 = 1
FP8_E4M3 = 2   # pool element of the *_fp8 calls (uint8 tensors)
DECODE_SCRATCH_BYTES = 32 << 20   # RAX_DECODE_SCRATCH_BYTES: the no-allocation DECODE's static scratch
_PKG = os.path.dirname(os.path.abspath(__file__))
_HEADER = os.path.join(os.path.dirname(_PKG), "include", "librax.h")
_lib = None

_c_i32, _c_i64, _c_sz, _c_f, _c_p = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p

_SIGS = {
    "rax_version": (ctypes.c_int, []),
    "rax_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "rax_kv_store": (ctypes.c_int, [ctypes.c_int, _c_p, _c_p, _c_p, _c_i64, _c_p, _c_p, _c_i64, _c_i32,
                                    _c_i32, _c_p]),
    "rax_extend_workspace_bytes": (_c_sz, [ctypes.c_int, _c_i32, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32,
                                           _c_i32]),
    "rax_extend_attention": (ctypes.c_int, [ctypes.c_int, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_p, _c_i64,
                                            _c_p, _c_p, _c_p, _c_p, _c_i32, _c_i64, _c_i32, _c_i32,
                                            _c_i32, _c_i32, _c_i32, _c_f, _c_p, _c_sz, _c_p]),
    "rax_extend_attention_ragged": (ctypes.c_int, [ctypes.c_int, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                                   _c_i64, _c_p, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_i32,
                                                   _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_f,
                                                   _c_p, _c_sz, _c_p]),
    "rax_extend_attention_paged": (ctypes.c_int, [ctypes.c_int, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_p, _c_i64,
                                                  _c_i32, _c_p, _c_p, _c_p, _c_p, _c_i32, _c_i64, _c_i32,
                                                  _c_i32, _c_i32, _c_i32, _c_i32, _c_f, _c_p, _c_sz, _c_p]),
    "rax_decode_attention_paged": (ctypes.c_int, [ctypes.c_int, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_p, _c_i64,
                                                  _c_i32, _c_p, _c_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                                  _c_f, _c_p, _c_sz, _c_p]),
    "rax_decode_workspace_bytes": (_c_sz, [ctypes.c_int, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32]),
    "rax_decode_attention": (ctypes.c_int, [ctypes.c_int, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_p, _c_i64,
                                            _c_p, _c_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_f,
                                            _c_p, _c_sz, _c_p]),
    "rax_decode_attention_noalloc": (ctypes.c_int, [ctypes.c_int, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_p, _c_i64,
                                                    _c_p, _c_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_f,
                                                    _c_p]),
    "rax_decode_num_splits": (_c_i32, [ctypes.c_int, _c_i32, _c_i32, _c_i32]),
    "rax_kv_store_fp8": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_i64, _c_p, _c_p, _c_i64, _c_i32, _c_i32, _c_f,
                                        _c_f, _c_p]),
    "rax_extend_attention_fp8": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_p, _c_i64, _c_p, _c_p,
                                                _c_p, _c_p, _c_i32, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32,
                                                _c_i32, _c_f, _c_f, _c_f, _c_p, _c_sz, _c_p]),
    "rax_decode_attention_fp8": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_p, _c_i64, _c_p, _c_p,
                                                _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_f, _c_f, _c_f,
                                                _c_p, _c_sz, _c_p]),
    "rax_extend_attention_ragged_paged": (ctypes.c_int, [ctypes.c_int, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                                         _c_p, _c_i64, _c_p, _c_i64, _c_i32, _c_p, _c_p, _c_p,
                                                         _c_p, _c_i32, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32,
                                                         _c_i32, _c_f, _c_p, _c_sz, _c_p]),
    "rax_extend_attention_paged_fp8": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_p, _c_i64, _c_i32,
                                                      _c_p, _c_p, _c_p, _c_p, _c_i32, _c_i64, _c_i32, _c_i32,
                                                      _c_i32, _c_i32, _c_i32, _c_f, _c_f, _c_f, _c_p, _c_sz,
                                                      _c_p]),
    "rax_decode_attention_paged_fp8": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_p, _c_i64, _c_i32,
                                                      _c_p, _c_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_f,
                                                      _c_f, _c_f, _c_p, _c_sz, _c_p]),
    "rax_check_workspace_bytes": (_c_sz, [_c_i64]),
    "rax_check_kv_store": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_sz, _c_p, _c_p]),
    "rax_check_extend": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_i32, _c_p, _c_p, _c_p, _c_p, _c_i32, _c_i64,
                                        _c_i32, _c_i32, _c_i64, _c_i32, _c_p, _c_p, _c_sz, _c_p, _c_p]),
    "rax_check_decode": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_i32, _c_p, _c_p, _c_i32, _c_i32, _c_i64, _c_p,
                                        _c_p]),
}


class RaxError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        name = load().rax_status_str(status).decode()
        super().__init__(f"{where}: {name} ({status})")


def library_path() -> str:
    return os.path.join(_PKG, "librax.so")


def declared_symbols() -> list[str]:
    """Names of the functions include/librax.h declares."""
    text = open(_HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[A-Za-z_][\w\s\*]*?)\b(rax_\w+)\s*\(", text, flags=re.M)))


def load():
    """Load librax.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m prefix_cached_paged_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def version() -> int:
    return load().rax_version()


def _dtype(*ts) -> int:
    dt = ts[0].dtype
    for t in ts:
        if t.dtype != dt:
            raise TypeError("all float tensors of one call must share a dtype")
    if dt == torch.bfloat16:
        return BF16
    if dt == torch.float32:
        return FP32
    raise TypeError(f"unsupported dtype {dt}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("librax takes device tensors")
    if not t.is_contiguous():
        raise ValueError("librax takes contiguous tensors")
    return t.data_ptr()


def _idx(t):
    if t.dtype != torch.int32:
        raise TypeError("index tensors must be int32")
    return _ptr(t)


def _stream(stream, device=None):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return s.cuda_stream


def _expect(ok: bool, what: str):
    if not ok:
        raise ValueError(what)


def _same_device(*ts):
    dev = ts[0].device
    _expect(all(t is None or t.device == dev for t in ts), "all tensors of one call must be on one device")


def _attn_shapes(q, o, k_pool, v_pool):
    """Shapes the C entry points cannot see (they take one head_dim and the pool's slot count):
    q and o alike, K and V pools alike, one head_dim, every tensor on q's device."""
    _expect(q.dim() == 3 and o.shape == q.shape, "q and o must be [rows, n_q_heads, head_dim] alike")
    _expect(k_pool.dim() == 3 and v_pool.shape == k_pool.shape,
            "k_pool and v_pool must be [num_slots, n_kv_heads, head_dim] alike")
    _expect(k_pool.shape[2] == q.shape[2], "the pools' head_dim differs from q's")
    _same_device(q, o, k_pool, v_pool)
    N, Hq, D = q.shape
    S, Hkv, _ = k_pool.shape
    return N, Hq, D, S, Hkv


def _per_request(B, *ts):
    _expect(all(t.dim() == 1 and t.shape[0] == B for t in ts), f"per-request arrays must have {B} entries")


def _table(t):
    _expect(t.dim() == 2, "the request / page table must be 2-D [rows, stride]")
    return t.shape[1]


def _rows(k_new, v_new, loc, k_pool, v_pool):
    _expect(k_new.dim() == 3 and v_new.shape == k_new.shape,
            "k_new and v_new must be [n, n_kv_heads, head_dim] alike")
    _expect(k_pool.dim() == 3 and v_pool.shape == k_pool.shape and tuple(k_new.shape[1:]) == tuple(k_pool.shape[1:]),
            "k_pool and v_pool must be [num_slots, n_kv_heads, head_dim] alike, with the rows' heads and head_dim")
    _expect(loc.dim() == 1 and loc.shape[0] <= k_new.shape[0], "loc must be 1-D with at most one entry per row")
    _same_device(k_new, v_new, loc, k_pool, v_pool)


def _check(status: int, where: str):
    if status != 0:
        raise RaxError(status, where)


def kv_store(k_new, v_new, loc, k_pool, v_pool, stream=None):
    """k_pool[loc[i]] = k_new[i]; v_pool[loc[i]] = v_new[i] (in place)."""
    _rows(k_new, v_new, loc, k_pool, v_pool)
    S, Hkv, D = k_pool.shape
    _check(load().rax_kv_store(_dtype(k_new, v_new, k_pool, v_pool), _ptr(k_new), _ptr(v_new), _idx(loc),
                               loc.shape[0], _ptr(k_pool), _ptr(v_pool), S, Hkv, D, _stream(stream, k_pool.device)),
           "rax_kv_store")


def extend_workspace_bytes(dtype: int, batch, total_tokens, max_extend_len, max_seq_len, n_q_heads,
                           n_kv_heads, head_dim) -> int:
    return load().rax_extend_workspace_bytes(dtype, batch, total_tokens, max_extend_len, max_seq_len,
                                             n_q_heads, n_kv_heads, head_dim)


def decode_workspace_bytes(dtype: int, batch, max_seq_len, n_q_heads, n_kv_heads, head_dim) -> int:
    return load().rax_decode_workspace_bytes(dtype, batch, max_seq_len, n_q_heads, n_kv_heads, head_dim)


def decode_num_splits(dtype: int, batch, max_seq_len, n_kv_heads) -> int:
    return load().rax_decode_num_splits(dtype, batch, max_seq_len, n_kv_heads)


def _workspace(nbytes, workspace, device, stream=None):
    """The caller's workspace, or a new one. A new block is tied to the launch stream
    (``record_stream``): the caching allocator then does not hand it to other work until that
    stream has passed the kernels that write and read it, although the tensor itself is dropped
    when the call returns."""
    if nbytes == 0:
        return workspace
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        workspace.record_stream(stream if stream is not None else torch.cuda.current_stream(device))
    return workspace


def extend_attention(q, o, k_pool, v_pool, req_to_token, req_pool_indices, prefix_lens, extend_lens,
                     extend_start_loc, max_extend_len, max_seq_len, sm_scale, workspace=None,
                     stream=None):
    """EXTEND attention of the suffix rows ``q`` into ``o`` (same shape), keys from the pool."""
    N, Hq, D, S, Hkv = _attn_shapes(q, o, k_pool, v_pool)
    dt = _dtype(q, o, k_pool, v_pool)
    B = prefix_lens.shape[0]
    _per_request(B, req_pool_indices, prefix_lens, extend_lens, extend_start_loc)
    _table(req_to_token)
    need = extend_workspace_bytes(dt, B, N, max_extend_len, max_seq_len, Hq, Hkv, D)
    workspace = _workspace(need, workspace, q.device, stream)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().rax_extend_attention(dt, _ptr(q), _ptr(o), _ptr(k_pool), _ptr(v_pool), S, _idx(req_to_token),
                                       req_to_token.shape[1], _idx(req_pool_indices), _idx(prefix_lens),
                                       _idx(extend_lens), _idx(extend_start_loc), B, N, int(max_extend_len),
                                       int(max_seq_len), Hq, Hkv, D, float(sm_scale), _ptr(workspace), wbytes,
                                       _stream(stream, q.device)),
           "rax_extend_attention")


def extend_attention_ragged(q, o, k_new, v_new, k_pool, v_pool, req_to_token, req_pool_indices, prefix_lens,
                            extend_lens, extend_start_loc, max_extend_len, max_seq_len, sm_scale, store_loc=None,
                            workspace=None, stream=None):
    """EXTEND with the suffix K/V read from ``k_new`` / ``v_new`` (rows in ``q``'s order); with
    ``store_loc`` the rows are also written to those pool slots."""
    N, Hq, D, S, Hkv = _attn_shapes(q, o, k_pool, v_pool)
    dt = _dtype(q, o, k_pool, v_pool)
    if _dtype(k_new, v_new) != dt or k_new.shape != (N, Hkv, D) or v_new.shape != k_new.shape:
        raise ValueError("k_new / v_new must be [tokens, n_kv_heads, head_dim] in the pool's dtype")
    _expect(store_loc is None or (store_loc.dim() == 1 and store_loc.shape[0] == N),
            "store_loc must hold one slot per suffix row")
    _same_device(q, k_new, v_new, store_loc)
    B = prefix_lens.shape[0]
    _per_request(B, req_pool_indices, prefix_lens, extend_lens, extend_start_loc)
    _table(req_to_token)
    need = extend_workspace_bytes(dt, B, N, max_extend_len, max_seq_len, Hq, Hkv, D)
    workspace = _workspace(need, workspace, q.device, stream)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().rax_extend_attention_ragged(dt, _ptr(q), _ptr(o), _ptr(k_new), _ptr(v_new),
                                              _idx(store_loc) if store_loc is not None else None, _ptr(k_pool),
                                              _ptr(v_pool), S, _idx(req_to_token), req_to_token.shape[1],
                                              _idx(req_pool_indices), _idx(prefix_lens), _idx(extend_lens),
                                              _idx(extend_start_loc), B, N, int(max_extend_len), int(max_seq_len),
                                              Hq, Hkv, D, float(sm_scale), _ptr(workspace), wbytes,
                                              _stream(stream, q.device)),
           "rax_extend_attention_ragged")


def extend_attention_ragged_paged(q, o, k_new, v_new, k_pool, v_pool, page_table, page_size, req_pool_indices,
                                  prefix_lens, extend_lens, extend_start_loc, max_extend_len, max_seq_len, sm_scale,
                                  store_loc=None, workspace=None, stream=None):
    """Ragged EXTEND (suffix K/V from ``k_new`` / ``v_new``, optional fused store) with the prefix
    read through a page table of ``page_size`` slots per page."""
    N, Hq, D, S, Hkv = _attn_shapes(q, o, k_pool, v_pool)
    dt = _dtype(q, o, k_pool, v_pool)
    if _dtype(k_new, v_new) != dt or k_new.shape != (N, Hkv, D) or v_new.shape != k_new.shape:
        raise ValueError("k_new / v_new must be [tokens, n_kv_heads, head_dim] in the pool's dtype")
    _expect(store_loc is None or (store_loc.dim() == 1 and store_loc.shape[0] == N),
            "store_loc must hold one slot per suffix row")
    _same_device(q, k_new, v_new, store_loc)
    B = prefix_lens.shape[0]
    _per_request(B, req_pool_indices, prefix_lens, extend_lens, extend_start_loc)
    _table(page_table)
    need = extend_workspace_bytes(dt, B, N, max_extend_len, max_seq_len, Hq, Hkv, D)
    workspace = _workspace(need, workspace, q.device, stream)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().rax_extend_attention_ragged_paged(dt, _ptr(q), _ptr(o), _ptr(k_new), _ptr(v_new),
                                                    _idx(store_loc) if store_loc is not None else None,
                                                    _ptr(k_pool), _ptr(v_pool), S, _idx(page_table),
                                                    page_table.shape[1], int(page_size), _idx(req_pool_indices),
                                                    _idx(prefix_lens), _idx(extend_lens), _idx(extend_start_loc),
                                                    B, N, int(max_extend_len), int(max_seq_len), Hq, Hkv, D,
                                                    float(sm_scale), _ptr(workspace), wbytes,
                                                    _stream(stream, q.device)),
           "rax_extend_attention_ragged_paged")


def extend_attention_paged(q, o, k_pool, v_pool, page_table, page_size, req_pool_indices, prefix_lens,
                           extend_lens, extend_start_loc, max_extend_len, max_seq_len, sm_scale, workspace=None,
                           stream=None):
    """EXTEND with keys addressed through a page table of ``page_size`` slots per page."""
    N, Hq, D, S, Hkv = _attn_shapes(q, o, k_pool, v_pool)
    dt = _dtype(q, o, k_pool, v_pool)
    B = prefix_lens.shape[0]
    _per_request(B, req_pool_indices, prefix_lens, extend_lens, extend_start_loc)
    _table(page_table)
    need = extend_workspace_bytes(dt, B, N, max_extend_len, max_seq_len, Hq, Hkv, D)
    workspace = _workspace(need, workspace, q.device, stream)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().rax_extend_attention_paged(dt, _ptr(q), _ptr(o), _ptr(k_pool), _ptr(v_pool), S,
                                             _idx(page_table), page_table.shape[1], int(page_size),
                                             _idx(req_pool_indices), _idx(prefix_lens), _idx(extend_lens),
                                             _idx(extend_start_loc), B, N, int(max_extend_len), int(max_seq_len),
                                             Hq, Hkv, D, float(sm_scale), _ptr(workspace), wbytes,
                                             _stream(stream, q.device)),
           "rax_extend_attention_paged")


def decode_attention_paged(q, o, k_pool, v_pool, page_table, page_size, req_pool_indices, seq_lens, max_seq_len,
                           sm_scale, workspace=None, stream=None):
    """DECODE with keys addressed through a page table of ``page_size`` slots per page."""
    B, Hq, D, S, Hkv = _attn_shapes(q, o, k_pool, v_pool)
    dt = _dtype(q, o, k_pool, v_pool)
    _per_request(B, req_pool_indices, seq_lens)
    _table(page_table)
    need = decode_workspace_bytes(dt, B, max_seq_len, Hq, Hkv, D)
    workspace = _workspace(need, workspace, q.device, stream)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().rax_decode_attention_paged(dt, _ptr(q), _ptr(o), _ptr(k_pool), _ptr(v_pool), S,
                                             _idx(page_table), page_table.shape[1], int(page_size),
                                             _idx(req_pool_indices), _idx(seq_lens), B, int(max_seq_len), Hq, Hkv,
                                             D, float(sm_scale), _ptr(workspace), wbytes, _stream(stream, q.device)),
           "rax_decode_attention_paged")


def decode_attention(q, o, k_pool, v_pool, req_to_token, req_pool_indices, seq_lens, max_seq_len, sm_scale,
                     workspace=None, stream=None):
    """DECODE attention of one query per request ``q`` [B, Hq, D] into ``o``."""
    B, Hq, D, S, Hkv = _attn_shapes(q, o, k_pool, v_pool)
    dt = _dtype(q, o, k_pool, v_pool)
    _per_request(B, req_pool_indices, seq_lens)
    _table(req_to_token)
    need = decode_workspace_bytes(dt, B, max_seq_len, Hq, Hkv, D)
    workspace = _workspace(need, workspace, q.device, stream)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().rax_decode_attention(dt, _ptr(q), _ptr(o), _ptr(k_pool), _ptr(v_pool), S, _idx(req_to_token),
                                       req_to_token.shape[1], _idx(req_pool_indices), _idx(seq_lens), B,
                                       int(max_seq_len), Hq, Hkv, D, float(sm_scale), _ptr(workspace), wbytes,
                                       _stream(stream, q.device)),
           "rax_decode_attention")


def decode_attention_noalloc(q, o, k_pool, v_pool, req_to_token, req_pool_indices, seq_lens, max_seq_len,
                             sm_scale, stream=None):
    """decode_attention without a workspace: the plan and partials go to the library's static
    per-device scratch (no allocation at all; calls on one GPU must not overlap)."""
    B, Hq, D, S, Hkv = _attn_shapes(q, o, k_pool, v_pool)
    dt = _dtype(q, o, k_pool, v_pool)
    _per_request(B, req_pool_indices, seq_lens)
    _table(req_to_token)
    _check(load().rax_decode_attention_noalloc(dt, _ptr(q), _ptr(o), _ptr(k_pool), _ptr(v_pool), S,
                                               _idx(req_to_token), req_to_token.shape[1], _idx(req_pool_indices),
                                               _idx(seq_lens), B, int(max_seq_len), Hq, Hkv, D, float(sm_scale),
                                               _stream(stream, q.device)),
           "rax_decode_attention_noalloc")


def _fp8_pool(t):
    if t.dtype != torch.uint8:
        raise TypeError("FP8 pools are uint8 tensors of E4M3 bytes")
    return _ptr(t)


def _bf16(t):
    if t.dtype != torch.bfloat16:
        raise TypeError("q, o and the new rows of the FP8 calls are bfloat16")
    return _ptr(t)


def kv_store_fp8(k_new, v_new, loc, k_pool, v_pool, k_scale=1.0, v_scale=1.0, stream=None):
    """Write bf16 rows into FP8 E4M3 pools at ``loc`` (scale 1.0 when the caller has none)."""
    _rows(k_new, v_new, loc, k_pool, v_pool)
    S, Hkv, D = k_pool.shape
    _check(load().rax_kv_store_fp8(_bf16(k_new), _bf16(v_new), _idx(loc), loc.shape[0], _fp8_pool(k_pool),
                                   _fp8_pool(v_pool), S, Hkv, D, float(k_scale), float(v_scale),
                                   _stream(stream, k_pool.device)),
           "rax_kv_store_fp8")


def extend_attention_fp8(q, o, k_pool, v_pool, req_to_token, req_pool_indices, prefix_lens, extend_lens,
                         extend_start_loc, max_extend_len, max_seq_len, sm_scale, k_scale=1.0, v_scale=1.0,
                         workspace=None, stream=None):
    """EXTEND attention over FP8 E4M3 pools (bf16 ``q`` and ``o``)."""
    N, Hq, D, S, Hkv = _attn_shapes(q, o, k_pool, v_pool)
    B = prefix_lens.shape[0]
    _per_request(B, req_pool_indices, prefix_lens, extend_lens, extend_start_loc)
    _table(req_to_token)
    need = extend_workspace_bytes(FP8_E4M3, B, N, max_extend_len, max_seq_len, Hq, Hkv, D)
    workspace = _workspace(need, workspace, q.device, stream)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().rax_extend_attention_fp8(_bf16(q), _bf16(o), _fp8_pool(k_pool), _fp8_pool(v_pool), S,
                                           _idx(req_to_token), req_to_token.shape[1], _idx(req_pool_indices),
                                           _idx(prefix_lens), _idx(extend_lens), _idx(extend_start_loc), B, N,
                                           int(max_extend_len), int(max_seq_len), Hq, Hkv, D, float(sm_scale),
                                           float(k_scale), float(v_scale), _ptr(workspace), wbytes,
                                           _stream(stream, q.device)),
           "rax_extend_attention_fp8")


def decode_attention_fp8(q, o, k_pool, v_pool, req_to_token, req_pool_indices, seq_lens, max_seq_len, sm_scale,
                         k_scale=1.0, v_scale=1.0, workspace=None, stream=None):
    """DECODE attention over FP8 E4M3 pools (bf16 ``q`` and ``o``)."""
    B, Hq, D, S, Hkv = _attn_shapes(q, o, k_pool, v_pool)
    _per_request(B, req_pool_indices, seq_lens)
    _table(req_to_token)
    need = decode_workspace_bytes(FP8_E4M3, B, int(max_seq_len), Hq, Hkv, D)
    workspace = _workspace(need, workspace, q.device, stream)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().rax_decode_attention_fp8(_bf16(q), _bf16(o), _fp8_pool(k_pool), _fp8_pool(v_pool), S,
                                           _idx(req_to_token), req_to_token.shape[1], _idx(req_pool_indices),
                                           _idx(seq_lens), B, int(max_seq_len), Hq, Hkv, D, float(sm_scale),
                                           float(k_scale), float(v_scale), _ptr(workspace), wbytes,
                                           _stream(stream, q.device)),
           "rax_decode_attention_fp8")


def extend_attention_paged_fp8(q, o, k_pool, v_pool, page_table, page_size, req_pool_indices, prefix_lens,
                               extend_lens, extend_start_loc, max_extend_len, max_seq_len, sm_scale, k_scale=1.0,
                               v_scale=1.0, workspace=None, stream=None):
    """EXTEND over FP8 E4M3 pools with keys addressed through a page table of ``page_size`` slots."""
    N, Hq, D, S, Hkv = _attn_shapes(q, o, k_pool, v_pool)
    B = prefix_lens.shape[0]
    _per_request(B, req_pool_indices, prefix_lens, extend_lens, extend_start_loc)
    _table(page_table)
    need = extend_workspace_bytes(FP8_E4M3, B, N, max_extend_len, max_seq_len, Hq, Hkv, D)
    workspace = _workspace(need, workspace, q.device, stream)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().rax_extend_attention_paged_fp8(_bf16(q), _bf16(o), _fp8_pool(k_pool), _fp8_pool(v_pool), S,
                                                 _idx(page_table), page_table.shape[1], int(page_size),
                                                 _idx(req_pool_indices), _idx(prefix_lens), _idx(extend_lens),
                                                 _idx(extend_start_loc), B, N, int(max_extend_len),
                                                 int(max_seq_len), Hq, Hkv, D, float(sm_scale), float(k_scale),
                                                 float(v_scale), _ptr(workspace), wbytes,
                                                 _stream(stream, q.device)),
           "rax_extend_attention_paged_fp8")


def decode_attention_paged_fp8(q, o, k_pool, v_pool, page_table, page_size, req_pool_indices, seq_lens,
                               max_seq_len, sm_scale, k_scale=1.0, v_scale=1.0, workspace=None, stream=None):
    """DECODE over FP8 E4M3 pools with keys addressed through a page table of ``page_size`` slots."""
    B, Hq, D, S, Hkv = _attn_shapes(q, o, k_pool, v_pool)
    _per_request(B, req_pool_indices, seq_lens)
    _table(page_table)
    need = decode_workspace_bytes(FP8_E4M3, B, int(max_seq_len), Hq, Hkv, D)
    workspace = _workspace(need, workspace, q.device, stream)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().rax_decode_attention_paged_fp8(_bf16(q), _bf16(o), _fp8_pool(k_pool), _fp8_pool(v_pool), S,
                                                 _idx(page_table), page_table.shape[1], int(page_size),
                                                 _idx(req_pool_indices), _idx(seq_lens), B, int(max_seq_len), Hq,
                                                 Hkv, D, float(sm_scale), float(k_scale), float(v_scale),
                                                 _ptr(workspace), wbytes, _stream(stream, q.device)),
           "rax_decode_attention_paged_fp8")


# Debug checks of the device-side contracts: counts per kind (order of rax_check_item).
CHECK_ITEMS = ("length", "row", "slot", "duplicate", "overlap")


def _counts_dict(counts):
    return dict(zip(CHECK_ITEMS, (int(x) for x in counts.cpu().tolist())))  # waits for the stream


def _check_bitmap(num_slots, device):
    return torch.empty(load().rax_check_workspace_bytes(int(num_slots)), dtype=torch.uint8, device=device)


def check_kv_store(loc, num_slots, stream=None):
    """Counts of ``loc`` entries outside [0, num_slots) ("slot") and repeats ("duplicate")."""
    _expect(loc.dim() == 1, "loc must be 1-D")
    counts = torch.empty(len(CHECK_ITEMS), dtype=torch.int32, device=loc.device)
    ws = _check_bitmap(num_slots, loc.device)
    _check(load().rax_check_kv_store(_idx(loc), loc.shape[0], int(num_slots), _ptr(ws), ws.numel(), _ptr(counts),
                                     _stream(stream, loc.device)),
           "rax_check_kv_store")
    return _counts_dict(counts)


def check_extend(table, req_pool_indices, prefix_lens, extend_lens, extend_start_loc, total_tokens, max_extend_len,
                 max_seq_len, num_slots, page_size=1, ragged=False, store_loc=None, stream=None):
    """Contract breaks in the index arrays of an EXTEND call (token or page ``table``; the ragged
    call reads only the prefix from the pool, and ``store_loc`` adds the duplicate / overlap
    checks of its store)."""
    B = prefix_lens.shape[0]
    _per_request(B, req_pool_indices, prefix_lens, extend_lens, extend_start_loc)
    _expect(store_loc is None or (store_loc.dim() == 1 and store_loc.shape[0] == int(total_tokens)),
            "store_loc must hold one slot per suffix row")
    _same_device(table, req_pool_indices, prefix_lens, extend_lens, extend_start_loc, store_loc)
    stride = _table(table)
    counts = torch.empty(len(CHECK_ITEMS), dtype=torch.int32, device=table.device)
    ws = _check_bitmap(num_slots, table.device) if store_loc is not None else None
    _check(load().rax_check_extend(_idx(table), table.shape[0], stride, int(page_size), _idx(req_pool_indices),
                                   _idx(prefix_lens), _idx(extend_lens), _idx(extend_start_loc), B, int(total_tokens),
                                   int(max_extend_len), int(max_seq_len), int(num_slots), int(bool(ragged)),
                                   _idx(store_loc) if store_loc is not None else None, _ptr(ws),
                                   ws.numel() if ws is not None else 0, _ptr(counts), _stream(stream, table.device)),
           "rax_check_extend")
    return _counts_dict(counts)


def check_decode(table, req_pool_indices, seq_lens, max_seq_len, num_slots, page_size=1, stream=None):
    """Contract breaks in the index arrays of a DECODE call (token or page ``table``)."""
    B = seq_lens.shape[0]
    _per_request(B, req_pool_indices, seq_lens)
    _same_device(table, req_pool_indices, seq_lens)
    stride = _table(table)
    counts = torch.empty(len(CHECK_ITEMS), dtype=torch.int32, device=table.device)
    _check(load().rax_check_decode(_idx(table), table.shape[0], stride, int(page_size), _idx(req_pool_indices),
                                   _idx(seq_lens), B, int(max_seq_len), int(num_slots), _ptr(counts),
                                   _stream(stream, table.device)),
           "rax_check_decode")
    return _counts_dict(counts)
