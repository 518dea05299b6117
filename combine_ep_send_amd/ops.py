"""Thin PyTorch binding of libepdc.so.

The ``ep_*`` functions mirror the C entry points one for one: they check
dtypes, shapes and devices, allocate outputs the caller did not pass, and
call the library on the current (or given) HIP stream.  All arithmetic runs
in the HIP kernels; PyTorch only supplies device memory and streams.
"""

from __future__ import annotations

import ctypes
import functools
from typing import NamedTuple, Optional

import torch

from ._lib import (EP_DTYPE_BF16, EP_DTYPE_FP8_E4M3, EP_SCALE_F32, EP_SCALE_POW2, EP_SCALE_UE8M0,
                   EP_WS_WAIT_GAVE_UP, EpError, check, lib)

__all__ = [
    "Counts",
    "SendLayout",
    "ep_compute_send_counts",
    "ep_build_send_layout",
    "ep_dispatch_layout",
    "ep_dispatch_layout_workspace_bytes",
    "ep_dispatch_layout_noalloc",
    "ep_dispatch_layout_chunked",
    "ep_dispatch_layout_chunked_workspace_bytes",
    "library_scratch_status",
    "ep_dispatch_permute",
    "ep_regroup_by_expert",
    "ep_regroup_workspace_bytes",
    "Regrouped",
    "ep_batched_prepare",
    "ep_batched_prepare_fp8",
    "batched_scale_like",
    "SCALE_FORMATS",
    "ep_combine",
    "ep_counts_workspace_bytes",
    "ep_layout_workspace_bytes",
    "ep_batched_workspace_bytes",
    "workspace_for",
    "ep_workspace_status",
    "check_workspaces",
    "workspace_flags",
    "WaitGaveUpError",
]


class Counts(NamedTuple):
    dest: torch.Tensor                 # int32 [T, K]
    is_in_rank: torch.Tensor           # uint8 [T, P]
    send_counts: torch.Tensor          # int32 [C, P]
    tokens_per_expert: Optional[torch.Tensor]  # int32 [C, E] or None
    diag: torch.Tensor                 # int32 [1]: ids outside [-1, E)


class SendLayout(NamedTuple):
    send_token_idx: torch.Tensor       # int32 [cap]
    send_rank: torch.Tensor            # int32 [cap]
    send_idx: torch.Tensor             # int32 [cap, K]
    send_w: torch.Tensor               # float32 [cap, K]
    token_row: torch.Tensor            # int32 [T, K]


class Regrouped(NamedTuple):
    perm_x: torch.Tensor               # bf16 [cap, H]
    perm_src: torch.Tensor             # int32 [cap]: received row, -1 on padding
    perm_w: Optional[torch.Tensor]     # float32 [cap]: the slot's weight
    tokens_per_expert: torch.Tensor    # int32 [E_local]
    expert_offsets: torch.Tensor       # int32 [E_local + 1]
    row_map: torch.Tensor              # int32 [R, K]


def _vp(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _on_stream(fn):
    """An entry point given ``stream`` runs with that stream current, so the
    outputs it allocates belong to it: the caching allocator then hands their
    memory out again only after the work enqueued there."""
    @functools.wraps(fn)
    def call(*args, stream=None, **kw):
        if stream is None:
            return fn(*args, **kw)
        with torch.cuda.stream(stream):
            return fn(*args, stream=stream, **kw)
    return call


def _gpu(t: torch.Tensor, name: str, dtype, ndim: Optional[int] = None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")
    return t


def _shape(t: torch.Tensor, name: str, shape) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def ep_counts_workspace_bytes(num_tokens: int, num_ranks: int, num_local_experts: int,
                              num_chunks: int = 1) -> int:
    return int(lib().ep_counts_workspace_bytes(int(num_tokens), int(num_ranks),
                                               int(num_local_experts), int(num_chunks)))


def ep_layout_workspace_bytes(num_tokens: int, num_bins: int) -> int:
    return int(lib().ep_layout_workspace_bytes(int(num_tokens), int(num_bins)))


def ep_batched_workspace_bytes(num_tokens: int, num_local_experts: int, max_num_tokens: int) -> int:
    return int(lib().ep_batched_workspace_bytes(int(num_tokens), int(num_local_experts),
                                                int(max_num_tokens)))


_WORKSPACES = {}      # (device index, stream handle, kind) -> (workspace, stream)


def workspace_for(nbytes: int, device: torch.device, stream=None,
                  kind: str = "scan") -> torch.Tensor:
    """A zero-initialised workspace of at least ``nbytes``, cached per
    (device, stream, kind).  The kernels leave it ready for the next call, so
    one workspace serves every call of that kind enqueued on its stream.
    ``kind`` is "counts" (ep_compute_send_counts), "scan" (the layout and
    batched scans, which share one protocol) or "fused" (ep_dispatch_layout)."""
    s = stream if stream is not None else torch.cuda.current_stream(device)
    key = (device.index if device.index is not None else torch.cuda.current_device(),
           s.cuda_stream, kind)
    ws = _WORKSPACES.get(key, (None, None))[0]
    if ws is None or ws.numel() < nbytes:
        if ws is not None:             # kept, so that check_workspaces still sees its flags
            _RETIRED.append((key, _WORKSPACES[key]))
        with torch.cuda.stream(s):
            ws = torch.zeros(max(int(nbytes), 1 << 16), dtype=torch.uint8, device=device)
        _WORKSPACES[key] = (ws, s)
    return ws


_RETIRED = []         # workspaces replaced by larger ones, not yet queried


class WaitGaveUpError(EpError):
    """A bounded wait inside a call (grid barrier or scan lookback) gave up:
    the outputs of the call that waited are undefined."""


def ep_workspace_status(workspace: torch.Tensor, *, stream=None) -> int:
    """The error word a workspace has collected since the previous query
    (bit EP_WS_WAIT_GAVE_UP: a bounded wait gave up), cleared by the query.
    Enqueues the query on ``stream`` (default: the current stream) and waits
    for that stream to reach it."""
    _gpu(workspace, "workspace", torch.uint8)
    s = stream if stream is not None else torch.cuda.current_stream(workspace.device)
    with torch.cuda.stream(s):
        flags = torch.zeros(1, dtype=torch.int32, device=workspace.device)
        st = lib().ep_workspace_status(_vp(workspace), workspace.numel(), _vp(flags), _stream(s))
    check(st, "ep_workspace_status")
    s.synchronize()
    return int(flags.item())


def _raise_on_flags(found):
    bad = [(f, kind, dev) for f, kind, dev in found if f]
    if bad:
        what = ", ".join(f"{kind} workspace on cuda:{dev} (flags {f:#x})" for f, kind, dev in bad)
        raise WaitGaveUpError(f"a bounded wait gave up, so the outputs of a call that used it "
                              f"are undefined: {what}")


def workspace_flags(*workspaces: torch.Tensor):
    """[(flags, kind, device index)] of the given workspaces (default: every
    workspace ``workspace_for`` has handed out, each queried on its own
    stream), each read and cleared by ep_workspace_status.  Synchronizes
    those streams."""
    found = []
    if workspaces:
        for ws in workspaces:
            found.append((ep_workspace_status(ws), "given", ws.device.index))
    else:
        for (dev, _, kind), (ws, s) in list(_WORKSPACES.items()):
            found.append((ep_workspace_status(ws, stream=s), kind, dev))
        while _RETIRED:
            (dev, _, kind), (ws, s) = _RETIRED.pop()
            found.append((ep_workspace_status(ws, stream=s), kind, dev))
    return found


def check_workspaces(*workspaces: torch.Tensor) -> None:
    """Raise WaitGaveUpError if any of the given workspaces (default: all
    that ``workspace_for`` handed out) recorded a give-up since its last
    query (see workspace_flags)."""
    _raise_on_flags(workspace_flags(*workspaces))


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

@_on_stream
def ep_compute_send_counts(topk_idx: torch.Tensor, num_ranks: int, num_local_experts: int,
                           num_chunks: int = 1, *, expert_counts: bool = True,
                           out: Optional[Counts] = None,
                           workspace: Optional[torch.Tensor] = None, stream=None) -> Counts:
    _gpu(topk_idx, "topk_idx", torch.int64, 2)
    T, K = topk_idx.shape
    P, El, C = int(num_ranks), int(num_local_experts), int(num_chunks)
    E = P * El
    dev = topk_idx.device
    if out is None:
        out = Counts(
            dest=torch.empty((T, K), dtype=torch.int32, device=dev),
            is_in_rank=torch.empty((T, P), dtype=torch.uint8, device=dev),
            send_counts=torch.empty((C, P), dtype=torch.int32, device=dev),
            tokens_per_expert=(torch.empty((C, E), dtype=torch.int32, device=dev)
                               if expert_counts else None),
            diag=torch.empty(1, dtype=torch.int32, device=dev))
    _shape(_gpu(out.dest, "dest", torch.int32), "dest", (T, K))
    _shape(_gpu(out.is_in_rank, "is_in_rank", torch.uint8), "is_in_rank", (T, P))
    _shape(_gpu(out.send_counts, "send_counts", torch.int32), "send_counts", (C, P))
    if out.tokens_per_expert is not None:
        _shape(_gpu(out.tokens_per_expert, "tokens_per_expert", torch.int32),
               "tokens_per_expert", (C, E))
    _shape(_gpu(out.diag, "diag", torch.int32), "diag", (1,))
    if workspace is None:
        workspace = workspace_for(ep_counts_workspace_bytes(T, P, El, C), dev, stream, "counts")
    _gpu(workspace, "workspace", torch.uint8)
    st = lib().ep_compute_send_counts(
        _vp(topk_idx), T, K, P, El, C, _vp(out.dest), _vp(out.is_in_rank), _vp(out.send_counts),
        _vp(out.tokens_per_expert), _vp(out.diag), _vp(workspace), workspace.numel(),
        _stream(stream))
    check(st, "ep_compute_send_counts")
    return out


@_on_stream
def ep_build_send_layout(topk_idx: torch.Tensor, topk_weights: torch.Tensor,
                         dest: torch.Tensor, send_counts: torch.Tensor, num_ranks: int,
                         num_local_experts: int, num_send_capacity: int, *,
                         out: Optional[SendLayout] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> SendLayout:
    _gpu(topk_idx, "topk_idx", torch.int64, 2)
    T, K = topk_idx.shape
    P, El, cap = int(num_ranks), int(num_local_experts), int(num_send_capacity)
    _shape(_gpu(topk_weights, "topk_weights", torch.float32), "topk_weights", (T, K))
    _shape(_gpu(dest, "dest", torch.int32), "dest", (T, K))
    _gpu(send_counts, "send_counts", torch.int32)
    if send_counts.numel() != P:
        raise ValueError("send_counts must hold P counts (one chunk)")
    dev = topk_idx.device
    if out is None:
        out = SendLayout(
            send_token_idx=torch.empty(cap, dtype=torch.int32, device=dev),
            send_rank=torch.empty(cap, dtype=torch.int32, device=dev),
            send_idx=torch.empty((cap, K), dtype=torch.int32, device=dev),
            send_w=torch.empty((cap, K), dtype=torch.float32, device=dev),
            token_row=torch.empty((T, K), dtype=torch.int32, device=dev))
    for name, t, dt in (("send_token_idx", out.send_token_idx, torch.int32),
                        ("send_rank", out.send_rank, torch.int32),
                        ("send_idx", out.send_idx, torch.int32),
                        ("send_w", out.send_w, torch.float32)):
        _gpu(t, name, dt)
        if t.shape[0] < cap:
            raise ValueError(f"{name} holds fewer than {cap} rows")
    if out.send_idx.dim() != 2 or out.send_idx.shape[1] != K or out.send_w.shape[1:] != (K,):
        raise ValueError("send_idx / send_w must be [cap, K]")
    _shape(_gpu(out.token_row, "token_row", torch.int32), "token_row", (T, K))
    nbytes = ep_layout_workspace_bytes(T, P)
    if workspace is None:
        workspace = workspace_for(nbytes, dev, stream)
    _gpu(workspace, "workspace", torch.uint8)
    st = lib().ep_build_send_layout(
        _vp(topk_idx), _vp(topk_weights), _vp(dest), _vp(send_counts), T, K, P, El, cap,
        _vp(out.send_token_idx), _vp(out.send_rank), _vp(out.send_idx), _vp(out.send_w),
        _vp(out.token_row), _vp(workspace), workspace.numel(), _stream(stream))
    check(st, "ep_build_send_layout")
    return out


def ep_dispatch_layout_workspace_bytes(num_tokens: int, num_ranks: int,
                                       num_local_experts: int) -> int:
    return int(lib().ep_dispatch_layout_workspace_bytes(int(num_tokens), int(num_ranks),
                                                        int(num_local_experts)))


@_on_stream
def ep_dispatch_layout(topk_idx: torch.Tensor, topk_weights: torch.Tensor, num_ranks: int,
                       num_local_experts: int, num_send_capacity: int, *,
                       expert_counts: bool = True, counts: Optional[Counts] = None,
                       out: Optional[SendLayout] = None,
                       workspace: Optional[torch.Tensor] = None, stream=None):
    """Counts and send layout in one launch.  Returns (Counts with C = 1,
    SendLayout), identical to ep_compute_send_counts followed by
    ep_build_send_layout."""
    _gpu(topk_idx, "topk_idx", torch.int64, 2)
    T, K = topk_idx.shape
    P, El, cap = int(num_ranks), int(num_local_experts), int(num_send_capacity)
    E = P * El
    _shape(_gpu(topk_weights, "topk_weights", torch.float32), "topk_weights", (T, K))
    dev = topk_idx.device
    if counts is None:
        counts = Counts(
            dest=torch.empty((T, K), dtype=torch.int32, device=dev),
            is_in_rank=torch.empty((T, P), dtype=torch.uint8, device=dev),
            send_counts=torch.empty((1, P), dtype=torch.int32, device=dev),
            tokens_per_expert=(torch.empty((1, E), dtype=torch.int32, device=dev)
                               if expert_counts else None),
            diag=torch.empty(1, dtype=torch.int32, device=dev))
    _shape(_gpu(counts.dest, "dest", torch.int32), "dest", (T, K))
    _shape(_gpu(counts.is_in_rank, "is_in_rank", torch.uint8), "is_in_rank", (T, P))
    _gpu(counts.send_counts, "send_counts", torch.int32)
    if counts.send_counts.numel() != P:
        raise ValueError("send_counts must hold P counts (one chunk)")
    if counts.tokens_per_expert is not None:
        _gpu(counts.tokens_per_expert, "tokens_per_expert", torch.int32)
        if counts.tokens_per_expert.numel() != E:
            raise ValueError("tokens_per_expert must hold E counts")
    _shape(_gpu(counts.diag, "diag", torch.int32), "diag", (1,))
    if out is None:
        out = SendLayout(
            send_token_idx=torch.empty(cap, dtype=torch.int32, device=dev),
            send_rank=torch.empty(cap, dtype=torch.int32, device=dev),
            send_idx=torch.empty((cap, K), dtype=torch.int32, device=dev),
            send_w=torch.empty((cap, K), dtype=torch.float32, device=dev),
            token_row=torch.empty((T, K), dtype=torch.int32, device=dev))
    for name, t, dt in (("send_token_idx", out.send_token_idx, torch.int32),
                        ("send_rank", out.send_rank, torch.int32),
                        ("send_idx", out.send_idx, torch.int32),
                        ("send_w", out.send_w, torch.float32)):
        _gpu(t, name, dt)
        if t.shape[0] < cap:
            raise ValueError(f"{name} holds fewer than {cap} rows")
    if out.send_idx.dim() != 2 or out.send_idx.shape[1] != K or out.send_w.shape[1:] != (K,):
        raise ValueError("send_idx / send_w must be [cap, K]")
    _shape(_gpu(out.token_row, "token_row", torch.int32), "token_row", (T, K))
    if workspace is None:
        workspace = workspace_for(ep_dispatch_layout_workspace_bytes(T, P, El), dev, stream,
                                  "fused")
    _gpu(workspace, "workspace", torch.uint8)
    st = lib().ep_dispatch_layout(
        _vp(topk_idx), _vp(topk_weights), T, K, P, El, cap, _vp(counts.dest),
        _vp(counts.is_in_rank), _vp(counts.send_counts), _vp(counts.tokens_per_expert),
        _vp(counts.diag), _vp(out.send_token_idx), _vp(out.send_rank), _vp(out.send_idx),
        _vp(out.send_w), _vp(out.token_row), _vp(workspace), workspace.numel(),
        _stream(stream))
    check(st, "ep_dispatch_layout")
    return counts, out


@_on_stream
def ep_dispatch_layout_noalloc(topk_idx: torch.Tensor, topk_weights: torch.Tensor,
                               num_ranks: int, num_local_experts: int, num_send_capacity: int,
                               *, counts: Counts, out: SendLayout, stream=None):
    """ep_dispatch_layout on the library's own scratch (no workspace, no
    allocation): the caller passes every output (``counts`` with C = 1 and
    ``out``), as ep_dispatch_layout takes them."""
    _gpu(topk_idx, "topk_idx", torch.int64, 2)
    T, K = topk_idx.shape
    P, El, cap = int(num_ranks), int(num_local_experts), int(num_send_capacity)
    E = P * El
    _shape(_gpu(topk_weights, "topk_weights", torch.float32), "topk_weights", (T, K))
    _shape(_gpu(counts.dest, "dest", torch.int32), "dest", (T, K))
    _shape(_gpu(counts.is_in_rank, "is_in_rank", torch.uint8), "is_in_rank", (T, P))
    _gpu(counts.send_counts, "send_counts", torch.int32)
    if counts.send_counts.numel() != P:
        raise ValueError("send_counts must hold P counts (one chunk)")
    if counts.tokens_per_expert is not None:
        _gpu(counts.tokens_per_expert, "tokens_per_expert", torch.int32)
        if counts.tokens_per_expert.numel() != E:
            raise ValueError("tokens_per_expert must hold E counts")
    _shape(_gpu(counts.diag, "diag", torch.int32), "diag", (1,))
    for name, t, dt in (("send_token_idx", out.send_token_idx, torch.int32),
                        ("send_rank", out.send_rank, torch.int32),
                        ("send_idx", out.send_idx, torch.int32),
                        ("send_w", out.send_w, torch.float32)):
        _gpu(t, name, dt)
        if t.shape[0] < cap:
            raise ValueError(f"{name} holds fewer than {cap} rows")
    if out.send_idx.dim() != 2 or out.send_idx.shape[1] != K or out.send_w.shape[1:] != (K,):
        raise ValueError("send_idx / send_w must be [cap, K]")
    _shape(_gpu(out.token_row, "token_row", torch.int32), "token_row", (T, K))
    st = lib().ep_dispatch_layout_noalloc(
        _vp(topk_idx), _vp(topk_weights), T, K, P, El, cap, _vp(counts.dest),
        _vp(counts.is_in_rank), _vp(counts.send_counts), _vp(counts.tokens_per_expert),
        _vp(counts.diag), _vp(out.send_token_idx), _vp(out.send_rank), _vp(out.send_idx),
        _vp(out.send_w), _vp(out.token_row), _stream(stream))
    check(st, "ep_dispatch_layout_noalloc")
    return counts, out


def library_scratch_status(*, stream=None) -> int:
    """ep_workspace_status of the library's own scratch on the current device
    (the one ep_dispatch_layout_noalloc uses), read back after ``stream``."""
    s = stream if stream is not None else torch.cuda.current_stream()
    with torch.cuda.stream(s):
        flags = torch.zeros(1, dtype=torch.int32, device=torch.device("cuda", s.device.index))
        st = lib().ep_workspace_status(None, 0, _vp(flags), _stream(s))
    check(st, "ep_workspace_status")
    s.synchronize()
    return int(flags.item())


def ep_dispatch_layout_chunked_workspace_bytes(num_tokens: int, num_ranks: int,
                                               num_chunks: int) -> int:
    return int(lib().ep_dispatch_layout_chunked_workspace_bytes(int(num_tokens), int(num_ranks),
                                                                int(num_chunks)))


@_on_stream
def ep_dispatch_layout_chunked(topk_idx: torch.Tensor, topk_weights: torch.Tensor,
                               num_ranks: int, num_local_experts: int, num_chunks: int,
                               chunk_capacity: int, *, counts: Optional[Counts] = None,
                               out: Optional[SendLayout] = None,
                               workspace: Optional[torch.Tensor] = None, stream=None):
    """Counts of every chunk and every chunk's send layout in one launch.
    Returns (Counts with C chunks and no expert counts, SendLayout whose
    send arrays hold C * chunk_capacity rows, chunk c's from row
    c * chunk_capacity, and whose token_row holds chunk-local rows)."""
    _gpu(topk_idx, "topk_idx", torch.int64, 2)
    T, K = topk_idx.shape
    P, El, C, cap = int(num_ranks), int(num_local_experts), int(num_chunks), int(chunk_capacity)
    rows = C * cap
    _shape(_gpu(topk_weights, "topk_weights", torch.float32), "topk_weights", (T, K))
    dev = topk_idx.device
    if counts is None:
        counts = Counts(
            dest=torch.empty((T, K), dtype=torch.int32, device=dev),
            is_in_rank=torch.empty((T, P), dtype=torch.uint8, device=dev),
            send_counts=torch.empty((C, P), dtype=torch.int32, device=dev),
            tokens_per_expert=None,
            diag=torch.empty(1, dtype=torch.int32, device=dev))
    if counts.tokens_per_expert is not None:
        raise ValueError("ep_dispatch_layout_chunked gives no expert counts")
    _shape(_gpu(counts.dest, "dest", torch.int32), "dest", (T, K))
    _shape(_gpu(counts.is_in_rank, "is_in_rank", torch.uint8), "is_in_rank", (T, P))
    _shape(_gpu(counts.send_counts, "send_counts", torch.int32), "send_counts", (C, P))
    _shape(_gpu(counts.diag, "diag", torch.int32), "diag", (1,))
    if out is None:
        out = SendLayout(
            send_token_idx=torch.empty(rows, dtype=torch.int32, device=dev),
            send_rank=torch.empty(rows, dtype=torch.int32, device=dev),
            send_idx=torch.empty((rows, K), dtype=torch.int32, device=dev),
            send_w=torch.empty((rows, K), dtype=torch.float32, device=dev),
            token_row=torch.empty((T, K), dtype=torch.int32, device=dev))
    for name, t, dt in (("send_token_idx", out.send_token_idx, torch.int32),
                        ("send_rank", out.send_rank, torch.int32),
                        ("send_idx", out.send_idx, torch.int32),
                        ("send_w", out.send_w, torch.float32)):
        _gpu(t, name, dt)
        if t.shape[0] < rows:
            raise ValueError(f"{name} holds fewer than {rows} rows")
    if out.send_idx.dim() != 2 or out.send_idx.shape[1] != K or out.send_w.shape[1:] != (K,):
        raise ValueError("send_idx / send_w must be [rows, K]")
    _shape(_gpu(out.token_row, "token_row", torch.int32), "token_row", (T, K))
    if workspace is None:
        workspace = workspace_for(ep_dispatch_layout_chunked_workspace_bytes(T, P, C), dev,
                                  stream, "fused")
    _gpu(workspace, "workspace", torch.uint8)
    st = lib().ep_dispatch_layout_chunked(
        _vp(topk_idx), _vp(topk_weights), T, K, P, El, C, cap, _vp(counts.dest),
        _vp(counts.is_in_rank), _vp(counts.send_counts), _vp(counts.diag),
        _vp(out.send_token_idx), _vp(out.send_rank), _vp(out.send_idx), _vp(out.send_w),
        _vp(out.token_row), _vp(workspace), workspace.numel(), _stream(stream))
    check(st, "ep_dispatch_layout_chunked")
    return counts, out


def ep_regroup_workspace_bytes(num_rows: int, num_bins: int) -> int:
    return int(lib().ep_regroup_workspace_bytes(int(num_rows), int(num_bins)))


@_on_stream
def ep_regroup_by_expert(recv_x: torch.Tensor, recv_idx: torch.Tensor,
                         recv_w: Optional[torch.Tensor], num_local_experts: int,
                         align: int = 1, capacity: Optional[int] = None, *,
                         row_group: Optional[torch.Tensor] = None, num_groups: int = 1,
                         out: Optional[Regrouped] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> Regrouped:
    """Received rows regrouped by local expert, each expert's segment padded
    to a multiple of ``align``; with ``row_group`` ([R] int32, values in
    [0, num_groups)) the rows are several receive buffers end to end and the
    bins are (group, expert).  The default capacity is the worst case
    R*min(K, E_local) + bins*(align-1); the real row count is
    ``expert_offsets[-1]``."""
    _gpu(recv_x, "recv_x", torch.bfloat16, 2)
    R, H = recv_x.shape
    _gpu(recv_idx, "recv_idx", torch.int32, 2)
    if recv_idx.shape[0] != R:
        raise ValueError("recv_idx must be [R, K]")
    K = recv_idx.shape[1]
    El, A, G = int(num_local_experts), int(align), int(num_groups)
    B = G * El
    if recv_w is not None:
        _shape(_gpu(recv_w, "recv_w", torch.float32), "recv_w", (R, K))
    if row_group is not None:
        _shape(_gpu(row_group, "row_group", torch.int32), "row_group", (R,))
    elif G != 1:
        raise ValueError("num_groups > 1 needs row_group")
    cap = R * min(K, El) + B * (A - 1) if capacity is None else int(capacity)
    dev = recv_x.device
    if out is None:
        out = Regrouped(
            perm_x=torch.empty((cap, H), dtype=torch.bfloat16, device=dev),
            perm_src=torch.empty(cap, dtype=torch.int32, device=dev),
            perm_w=(torch.empty(cap, dtype=torch.float32, device=dev)
                    if recv_w is not None else None),
            tokens_per_expert=torch.empty(B, dtype=torch.int32, device=dev),
            expert_offsets=torch.empty(B + 1, dtype=torch.int32, device=dev),
            row_map=torch.empty((R, K), dtype=torch.int32, device=dev))
    _gpu(out.perm_x, "perm_x", torch.bfloat16, 2)
    if out.perm_x.shape[0] < cap or out.perm_x.shape[1] != H:
        raise ValueError(f"perm_x must be [>= {cap}, {H}]")
    _gpu(out.perm_src, "perm_src", torch.int32)
    if out.perm_src.numel() < cap:
        raise ValueError("perm_src holds fewer rows than the capacity")
    if out.perm_w is not None:
        _gpu(out.perm_w, "perm_w", torch.float32)
        if out.perm_w.numel() < cap:
            raise ValueError("perm_w holds fewer rows than the capacity")
    _shape(_gpu(out.tokens_per_expert, "tokens_per_expert", torch.int32), "tokens_per_expert",
           (B,))
    _shape(_gpu(out.expert_offsets, "expert_offsets", torch.int32), "expert_offsets", (B + 1,))
    _shape(_gpu(out.row_map, "row_map", torch.int32), "row_map", (R, K))
    if workspace is None:
        workspace = workspace_for(ep_regroup_workspace_bytes(R, B), dev, stream, "fused")
    _gpu(workspace, "workspace", torch.uint8)
    st = lib().ep_regroup_by_expert(
        _vp(recv_x), _vp(recv_idx), _vp(recv_w), _vp(row_group), G, R, K, H, El, A, cap,
        _vp(out.perm_x),
        _vp(out.perm_src), _vp(out.perm_w), _vp(out.tokens_per_expert),
        _vp(out.expert_offsets), _vp(out.row_map), _vp(workspace), workspace.numel(),
        _stream(stream))
    check(st, "ep_regroup_by_expert")
    return out


@_on_stream
def ep_dispatch_permute(x: torch.Tensor, token_row: torch.Tensor, num_send_capacity: int, *,
                        fp8: bool = False, out: Optional[torch.Tensor] = None,
                        out_scale: Optional[torch.Tensor] = None, stream=None):
    """bf16: returns send_x [cap, H] bf16.  fp8: returns (send_x [cap, H]
    float8_e4m3fn, send_scale [cap, H/128] float32)."""
    _gpu(x, "x", torch.bfloat16, 2)
    T, H = x.shape
    _gpu(token_row, "token_row", torch.int32, 2)
    if token_row.shape[0] != T:
        raise ValueError("token_row must be [T, K]")
    K = token_row.shape[1]
    cap = int(num_send_capacity)
    dev = x.device
    if fp8:
        if out is None:
            out = torch.empty((cap, H), dtype=torch.float8_e4m3fn, device=dev)
        if out_scale is None:
            out_scale = torch.empty((cap, H // 128), dtype=torch.float32, device=dev)
        _gpu(out, "send_x", torch.float8_e4m3fn)
        _gpu(out_scale, "send_scale", torch.float32)
        if out.shape[0] < cap or out.shape[1:] != (H,) or out_scale.shape[0] < cap \
                or out_scale.shape[1:] != (H // 128,):
            raise ValueError("send_x / send_scale too small")
    else:
        if out is None:
            out = torch.empty((cap, H), dtype=torch.bfloat16, device=dev)
        _gpu(out, "send_x", torch.bfloat16)
        if out.shape[0] < cap or out.shape[1:] != (H,):
            raise ValueError("send_x too small")
    st = lib().ep_dispatch_permute(
        _vp(x), T, H, _vp(token_row), K, cap, EP_DTYPE_FP8_E4M3 if fp8 else EP_DTYPE_BF16,
        _vp(out), _vp(out_scale) if fp8 else None, _stream(stream))
    check(st, "ep_dispatch_permute")
    return (out, out_scale) if fp8 else out


@_on_stream
def ep_batched_prepare(x: torch.Tensor, topk_idx: torch.Tensor, first_expert: int,
                       num_local_experts: int, max_num_tokens: int, *,
                       out: Optional[torch.Tensor] = None,
                       tokens_per_expert: Optional[torch.Tensor] = None,
                       token_row: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, stream=None):
    """Returns (b_x [E_local, max, H] bf16, tokens_per_expert [E_local] int32,
    token_row [T, K] int32)."""
    _gpu(x, "x", torch.bfloat16, 2)
    _gpu(topk_idx, "topk_idx", torch.int64, 2)
    T, H = x.shape
    if topk_idx.shape[0] != T:
        raise ValueError("topk_idx must be [T, K]")
    K = topk_idx.shape[1]
    El, M = int(num_local_experts), int(max_num_tokens)
    dev = x.device
    if out is None:
        out = torch.empty((El, M, H), dtype=torch.bfloat16, device=dev)
    if tokens_per_expert is None:
        tokens_per_expert = torch.empty(El, dtype=torch.int32, device=dev)
    if token_row is None:
        token_row = torch.empty((T, K), dtype=torch.int32, device=dev)
    _shape(_gpu(out, "b_x", torch.bfloat16), "b_x", (El, M, H))
    _shape(_gpu(tokens_per_expert, "tokens_per_expert", torch.int32), "tokens_per_expert", (El,))
    _shape(_gpu(token_row, "token_row", torch.int32), "token_row", (T, K))
    nbytes = ep_batched_workspace_bytes(T, El, M)
    if workspace is None:
        workspace = workspace_for(nbytes, dev, stream)
    _gpu(workspace, "workspace", torch.uint8)
    st = lib().ep_batched_prepare(
        _vp(x), _vp(topk_idx), T, K, H, int(first_expert), El, M, _vp(out),
        _vp(tokens_per_expert), _vp(token_row), _vp(workspace), workspace.numel(),
        _stream(stream))
    check(st, "ep_batched_prepare")
    return out, tokens_per_expert, token_row


SCALE_FORMATS = {"f32": EP_SCALE_F32, "pow2": EP_SCALE_POW2, "ue8m0": EP_SCALE_UE8M0}


def batched_scale_like(num_local_experts: int, max_num_tokens: int, hidden: int,
                       scale_fmt: str = "f32", col_major: bool = False,
                       device=None) -> torch.Tensor:
    """An empty scale tensor for ep_batched_prepare_fp8: [E_local, max, H/128]
    float32, or [E_local, max, H/512] int32 for ``ue8m0``; with ``col_major``
    the last two dimensions are stored column-major (a transposed view of
    [E_local, units, max])."""
    units = hidden // (512 if scale_fmt == "ue8m0" else 128)
    dt = torch.int32 if scale_fmt == "ue8m0" else torch.float32
    El, M = int(num_local_experts), int(max_num_tokens)
    if col_major:
        return torch.empty((El, units, M), dtype=dt, device=device).transpose(1, 2)
    return torch.empty((El, M, units), dtype=dt, device=device)


@_on_stream
def ep_batched_prepare_fp8(x: torch.Tensor, topk_idx: torch.Tensor, first_expert: int,
                           num_local_experts: int, max_num_tokens: int, *,
                           scale_fmt: str = "f32", scale_col_major: bool = False,
                           out: Optional[torch.Tensor] = None,
                           out_scale: Optional[torch.Tensor] = None,
                           tokens_per_expert: Optional[torch.Tensor] = None,
                           token_row: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, stream=None):
    """The expert-batched layout with fp8 rows.  Returns (b_q [E_local, max, H]
    float8_e4m3fn, b_scale (see batched_scale_like), tokens_per_expert
    [E_local] int32, token_row [T, K] int32).  ``scale_fmt`` is "f32",
    "pow2" (power-of-two scales) or "ue8m0" (packed UE8M0 bytes)."""
    if scale_fmt not in SCALE_FORMATS:
        raise ValueError(f"scale_fmt must be one of {sorted(SCALE_FORMATS)}")
    _gpu(x, "x", torch.bfloat16, 2)
    _gpu(topk_idx, "topk_idx", torch.int64, 2)
    T, H = x.shape
    if topk_idx.shape[0] != T:
        raise ValueError("topk_idx must be [T, K]")
    K = topk_idx.shape[1]
    El, M = int(num_local_experts), int(max_num_tokens)
    dev = x.device
    if out is None:
        out = torch.empty((El, M, H), dtype=torch.float8_e4m3fn, device=dev)
    if out_scale is None:
        out_scale = batched_scale_like(El, M, H, scale_fmt, scale_col_major, dev)
    if tokens_per_expert is None:
        tokens_per_expert = torch.empty(El, dtype=torch.int32, device=dev)
    if token_row is None:
        token_row = torch.empty((T, K), dtype=torch.int32, device=dev)
    _shape(_gpu(out, "b_q", torch.float8_e4m3fn), "b_q", (El, M, H))
    like = batched_scale_like(El, M, H, scale_fmt, scale_col_major, "meta")
    if out_scale.device != dev or out_scale.dtype != like.dtype or \
            tuple(out_scale.shape) != tuple(like.shape) or \
            (out_scale.numel() and out_scale.stride() != like.stride()):
        raise ValueError(f"b_scale must be {like.dtype} {tuple(like.shape)} with strides "
                         f"{like.stride()} on {dev}")
    _shape(_gpu(tokens_per_expert, "tokens_per_expert", torch.int32), "tokens_per_expert", (El,))
    _shape(_gpu(token_row, "token_row", torch.int32), "token_row", (T, K))
    nbytes = ep_batched_workspace_bytes(T, El, M)
    if workspace is None:
        workspace = workspace_for(nbytes, dev, stream)
    _gpu(workspace, "workspace", torch.uint8)
    st = lib().ep_batched_prepare_fp8(
        _vp(x), _vp(topk_idx), T, K, H, int(first_expert), El, M, SCALE_FORMATS[scale_fmt],
        1 if scale_col_major else 0, _vp(out), out_scale.data_ptr() if out_scale.numel() else None,
        _vp(tokens_per_expert), _vp(token_row), _vp(workspace), workspace.numel(),
        _stream(stream))
    check(st, "ep_batched_prepare_fp8")
    return out, out_scale, tokens_per_expert, token_row


@_on_stream
def ep_combine(y: torch.Tensor, token_row: torch.Tensor,
               topk_weights: Optional[torch.Tensor], *, bias=None,
               out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """out [T, H] bf16 = fp32 sum over k of w[t, k] * y[token_row[t, k]], or
    with ``topk_weights=None`` the sum of each distinct row of t once (the
    per-destination partial outputs), plus ``bias`` (a [T, H] bf16 tensor or
    a pair of them).  ``y`` is [R, H] or any contiguous bf16 tensor whose last
    dim is H (e.g. the batched buffer [E_local, max, H], read as E_local*max
    rows)."""
    _gpu(y, "y", torch.bfloat16)
    if y.dim() < 2:
        raise ValueError("y must be [rows, H]")
    H = y.shape[-1]
    R = y.numel() // H if H else 0
    _gpu(token_row, "token_row", torch.int32, 2)
    T, K = token_row.shape
    if topk_weights is not None:
        _shape(_gpu(topk_weights, "topk_weights", torch.float32), "topk_weights", (T, K))
    biases = () if bias is None else (tuple(bias) if isinstance(bias, (tuple, list)) else (bias,))
    if len(biases) > 2:
        raise ValueError("bias is one [T, H] tensor or a pair")
    for i, b in enumerate(biases):
        _shape(_gpu(b, f"bias[{i}]", torch.bfloat16), f"bias[{i}]", (T, H))
    b0 = biases[0] if len(biases) > 0 else None
    b1 = biases[1] if len(biases) > 1 else None
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    _shape(_gpu(out, "out", torch.bfloat16), "out", (T, H))
    st = lib().ep_combine(_vp(y), R, _vp(token_row), _vp(topk_weights), T, K, H, _vp(b0),
                          _vp(b1), _vp(out), _stream(stream))
    check(st, "ep_combine")
    return out
