"""Move a seeded workload's host arrays to device tensors, and outputs back (plumbing only).

bfloat16 data travels as its raw 16-bit patterns, so the device sees the same bits the
host generated.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from .workloads import Workload


def to_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy with the stored bits (uint16 for bfloat16)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


@dataclass
class DeviceWorkload:
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    req_to_token: torch.Tensor
    store_loc: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    ext: dict | None
    dec: dict | None


def upload(wl: Workload, device="cuda") -> DeviceWorkload:
    ext = dec = None
    if wl.extend is not None:
        e = wl.extend
        ext = dict(q=to_dev(e.q, device), req_pool_indices=to_dev(e.req_pool_indices, device),
                   prefix_lens=to_dev(e.prefix_lens, device), extend_lens=to_dev(e.extend_lens, device),
                   extend_start_loc=to_dev(e.extend_start_loc, device),
                   max_extend_len=e.max_extend_len, max_seq_len=e.max_seq_len)
        ext["o"] = torch.empty_like(ext["q"])
    if wl.decode is not None:
        d = wl.decode
        dec = dict(q=to_dev(d.q, device), req_pool_indices=to_dev(d.req_pool_indices, device),
                   seq_lens=to_dev(d.seq_lens, device), max_seq_len=d.max_seq_len)
        dec["o"] = torch.empty_like(dec["q"])
    return DeviceWorkload(to_dev(wl.k_pool, device), to_dev(wl.v_pool, device), to_dev(wl.req_to_token, device),
                          to_dev(wl.store_loc, device), to_dev(wl.k_new, device), to_dev(wl.v_new, device),
                          ext, dec)
