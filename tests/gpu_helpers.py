"""Shared helpers for the GPU parity tests: moving seeded numpy inputs to the
device and computing oracle references on token subsets."""

import numpy as np
import torch

import oracle as O

DEV = "cuda:0"


def gpu_available() -> bool:
    return torch.cuda.is_available()


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 bit patterns on the host."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return bits(t)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cpu().numpy()
    return t.cpu().numpy()


def bf16_ulp_diff(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance in bf16 ulps between two arrays of finite bf16 bit patterns
    (sign-magnitude mapped to a monotone integer line)."""
    def line(u):
        u = u.astype(np.int32)
        return np.where(u & 0x8000, -(u & 0x7FFF), u & 0x7FFF)
    return np.abs(line(a_bits) - line(b_bits))


def oracle_combine_subset(x_bits, send_token_idx, token_row, w, tokens):
    """Oracle combine of an identity expert over the send layout, for a
    subset of tokens: expert output row r is hidden row send_token_idx[r]."""
    tokens = np.asarray(tokens, dtype=np.int64)
    rows = token_row[tokens]
    uniq, inv = np.unique(rows[rows >= 0], return_inverse=True)
    local = np.full(rows.shape, -1, dtype=np.int32)
    local[rows >= 0] = inv.astype(np.int32)
    y = O.dispatch_permute(x_bits, send_token_idx[uniq]) if len(uniq) else \
        np.zeros((0, x_bits.shape[1]), np.uint16)
    return O.combine(y, local, w[tokens])


def run_send_path(x, idx, w, P, El, cap=None, fp8=False, chunks=1):
    """Counts -> layout -> permute on the GPU for one chunk of tokens."""
    from combine_ep_send_amd import (ep_build_send_layout, ep_compute_send_counts,
                                     ep_dispatch_permute)
    T, K = idx.shape
    c = ep_compute_send_counts(idx, P, El, chunks)
    if cap is None:
        cap = T * min(K, P)
    lay = ep_build_send_layout(idx, w, c.dest, c.send_counts[0], P, El, cap)
    px = ep_dispatch_permute(x, lay.token_row, cap, fp8=fp8) if x is not None else None
    return c, lay, px
