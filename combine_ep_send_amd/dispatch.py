"""Dispatcher-level API named after the axolotl "torch_dispatch" page and
vLLM's BatchedPrepareAndFinalize, built on the ``ep_*`` entry points.

This is the collective-free local path: the P destinations are segments of
one send buffer on this GPU (the page's ``group=None`` case), so dispatch
returns the whole send layout and combine reads it back.
"""

from __future__ import annotations

from typing import Callable, List, NamedTuple, Optional, Tuple

import torch

from .ops import (Regrouped, ep_batched_prepare, ep_batched_prepare_fp8, ep_build_send_layout,
                  ep_combine,
                  ep_compute_send_counts, ep_dispatch_layout, ep_dispatch_permute,
                  ep_regroup_by_expert)

__all__ = [
    "chunk_bounds",
    "to_host",
    "compute_send_counts",
    "build_send_layout",
    "DispatchHandle",
    "dispatch",
    "combine",
    "dispatch_chunked_forward",
    "batched_prepare",
    "batched_finalize",
    "permute_by_expert",
    "restore_by_expert",
]


def chunk_bounds(num_tokens: int, chunks: int) -> List[Tuple[int, int]]:
    """``chunks`` contiguous [start, end) token ranges; all but the last hold
    num_tokens // chunks tokens and the last takes the remainder (axolotl
    "torch_dispatch": chunk_bounds), so leading chunks are empty when
    num_tokens < chunks.  The same split is what ep_compute_send_counts uses
    for its per-chunk counts."""
    if chunks < 1:
        raise ValueError("chunks must be >= 1")
    size = num_tokens // chunks
    return [(i * size, num_tokens if i == chunks - 1 else (i + 1) * size)
            for i in range(chunks)]


def to_host(x: torch.Tensor) -> torch.Tensor:
    """Device-to-host copy of split counts into pinned memory, waited on
    (axolotl "torch_dispatch": to_host).  This is the one sync of a dispatch
    that asks for exact counts."""
    host = torch.empty(x.shape, dtype=x.dtype, pin_memory=True)
    host.copy_(x, non_blocking=True)
    torch.cuda.current_stream(x.device).synchronize()
    return host


def compute_send_counts(topk_idx: torch.Tensor, num_ranks: int, num_local_experts: int):
    """(dest [T,K], is_in_rank [T,P], send_counts [P]) (axolotl
    compute_send_counts)."""
    c = ep_compute_send_counts(topk_idx, num_ranks, num_local_experts, 1, expert_counts=False)
    return c.dest, c.is_in_rank, c.send_counts[0]


def build_send_layout(topk_idx: torch.Tensor, topk_weights: torch.Tensor, dest: torch.Tensor,
                      is_in_rank: torch.Tensor, num_send: int, num_local_experts: int, *,
                      send_counts: Optional[torch.Tensor] = None):
    """(send_token_idx [N], send_rank [N], send_idx [N,K], send_w [N,K],
    token_row [T,K]) (axolotl build_send_layout, plus the inverse map
    token_row that combine uses).  ``num_send`` must equal is_in_rank.sum()."""
    P = is_in_rank.shape[1]
    if send_counts is None:
        send_counts = ep_compute_send_counts(topk_idx, P, num_local_experts, 1,
                                             expert_counts=False).send_counts[0]
    lay = ep_build_send_layout(topk_idx, topk_weights, dest, send_counts.reshape(-1), P,
                               num_local_experts, int(num_send))
    return lay


class DispatchHandle(NamedTuple):
    """What combine needs to return expert outputs to their tokens (the
    page's TorchEPHandle, local form)."""
    num_tokens: int
    token_row: torch.Tensor            # [T, K] send row of each slot's owner
    topk_weights: torch.Tensor         # [T, K] fp32
    send_token_idx: torch.Tensor       # [N]
    send_rank: torch.Tensor            # [N]
    send_counts: torch.Tensor          # [P] (device)
    num_send: int


def dispatch(x: torch.Tensor, topk_idx: torch.Tensor, topk_weights: torch.Tensor, *,
             num_local_experts: int, num_ranks: int, fp8: bool = False,
             num_send: Optional[int] = None):
    """Send each token once to every destination owning one of its experts
    (axolotl dispatch, group=None).  Returns (recv_x, recv_idx, recv_w,
    handle); recv_x is bf16 [N,H], or (e4m3 [N,H], fp32 scales [N,H/128])
    with ``fp8``.  Without ``num_send`` the counts are copied to the host
    once to size the buffers exactly; with it (a capacity, e.g. the worst
    case T*min(K, P)) counts and layout run as one launch."""
    T, K = topk_idx.shape
    if num_send is None:
        # exact sizing: counts, one host copy, then the layout
        c = ep_compute_send_counts(topk_idx, num_ranks, num_local_experts, 1,
                                   expert_counts=False)
        num_send = int(to_host(c.send_counts).sum())
        lay = ep_build_send_layout(topk_idx, topk_weights, c.dest, c.send_counts[0], num_ranks,
                                   num_local_experts, num_send)
    else:
        # given capacity: counts and layout in one launch, no host sync
        c, lay = ep_dispatch_layout(topk_idx, topk_weights, num_ranks, num_local_experts,
                                    num_send, expert_counts=False)
    recv_x = ep_dispatch_permute(x, lay.token_row, num_send, fp8=fp8)
    handle = DispatchHandle(T, lay.token_row, topk_weights, lay.send_token_idx, lay.send_rank,
                            c.send_counts[0], int(num_send))
    return recv_x, lay.send_idx, lay.send_w, handle


def combine(local_out: torch.Tensor, handle: DispatchHandle,
            out: Optional[torch.Tensor] = None, *, weighted: bool = True,
            bias=None) -> torch.Tensor:
    """Per-token sum of the expert outputs [N,H] back onto the source tokens.
    ``weighted``: each slot's row times its top-k weight (Buffer.combine with
    topk_weights).  Otherwise the local kernel has already weighted and
    summed over its slots, and each destination's partial row is added once
    (axolotl combine).  ``bias``: a [T,H] bf16 tensor or a pair, added
    before the one rounding to bf16 (Buffer.combine bias)."""
    return ep_combine(local_out, handle.token_row, handle.topk_weights if weighted else None,
                      bias=bias, out=out)


def dispatch_chunked_forward(x: torch.Tensor, topk_idx: torch.Tensor, topk_weights: torch.Tensor,
                             local_kernel: Callable, *, num_local_experts: int, num_ranks: int,
                             chunks: int, fp8: bool = False, streams: Optional[list] = None,
                             exact_counts: bool = True) -> torch.Tensor:
    """dispatch -> local_kernel -> combine over ``chunks`` token ranges,
    alternating over HIP streams (axolotl dispatch_chunked_forward).

    One count pass covers every chunk; with ``exact_counts`` its [C,P] counts
    reach the host in one copy and size each chunk's buffers, otherwise each
    chunk gets the worst case T_c * min(K, P) rows.  ``local_kernel(recv_x,
    recv_idx, recv_w)`` returns the bf16 expert output [rows, H]; it runs on
    the chunk's stream.  Every chunk's layout is enqueued before chunk 0's
    expert kernel, and chunk c+1's permute before chunk c's combine result is
    needed, so the streams overlap; the latency-bound layouts of chunks >= 1
    run on the second stream while chunk 0's rows stream on the first."""
    T, K = topk_idx.shape
    H = x.shape[1]
    P = int(num_ranks)
    dev = x.device
    main = torch.cuda.current_stream(dev)
    if streams is None:
        streams = [torch.cuda.Stream(device=dev) for _ in range(2)]
    bounds = chunk_bounds(T, chunks)
    s0 = streams[0]
    s0.wait_stream(main)
    c = ep_compute_send_counts(topk_idx, P, num_local_experts, chunks, expert_counts=False,
                               stream=s0)
    if exact_counts:
        with torch.cuda.stream(s0):
            caps = [int(v) for v in to_host(c.send_counts).sum(dim=1)]
    else:
        caps = [(e - s) * min(K, P) for s, e in bounds]
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ready = torch.cuda.Event()
    ready.record(s0)
    for st in streams[1:]:
        st.wait_event(ready)
    # Layouts: chunk 0's on stream 0, the later chunks' back to back on
    # stream 1 while chunk 0's permute runs (they are latency-bound).
    lays, laid = [], []
    for i, (s, e) in enumerate(bounds):
        st = s0 if i == 0 or len(streams) == 1 else streams[1]
        lay = None
        if e > s:
            lay = ep_build_send_layout(topk_idx[s:e], topk_weights[s:e], c.dest[s:e],
                                       c.send_counts[i], P, num_local_experts, caps[i],
                                       stream=st)
        ev = torch.cuda.Event()
        ev.record(st)
        lays.append(lay)
        laid.append(ev)
    for i, (s, e) in enumerate(bounds):
        if e == s:
            continue
        st = streams[i % len(streams)]
        st.wait_event(laid[i])
        with torch.cuda.stream(st):
            lay = lays[i]
            recv_x = ep_dispatch_permute(x[s:e], lay.token_row, caps[i], fp8=fp8, stream=st)
            y = local_kernel(recv_x, lay.send_idx, lay.send_w)
            ep_combine(y, lay.token_row, topk_weights[s:e], out=out[s:e], stream=st)
    for st in streams:
        done = torch.cuda.Event()
        done.record(st)
        main.wait_event(done)
    return out


def batched_prepare(a1: torch.Tensor, topk_ids: torch.Tensor, *, num_local_experts: int,
                    rank: int, max_num_tokens: int, quant: Optional[str] = None,
                    scale_col_major: bool = False):
    """vLLM BatchedPrepareAndFinalize.prepare.  Unquantized: returns (b_a1
    [E_local, max, H] bf16, tokens_per_expert [E_local], token_row [T,K]).
    With ``quant`` = "f32", "pow2" or "ue8m0" the rows are fp8 e4m3 with one
    scale per token per 128 channels (NeMo uccl_ep Buffer.low_latency_dispatch
    use_fp8 / round_scale / use_ue8m0), and the return value is (b_q,
    b_scale, tokens_per_expert, token_row)."""
    first = int(rank) * int(num_local_experts)
    if quant is None:
        return ep_batched_prepare(a1, topk_ids, first, num_local_experts, max_num_tokens)
    return ep_batched_prepare_fp8(a1, topk_ids, first, num_local_experts, max_num_tokens,
                                  scale_fmt=quant, scale_col_major=scale_col_major)


def batched_finalize(fused_expert_output: torch.Tensor, topk_weights: torch.Tensor,
                     token_row: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """vLLM BatchedPrepareAndFinalize.finalize: weight by topk_weights and sum
    the local experts' outputs per token (fp32 accumulation)."""
    return ep_combine(fused_expert_output, token_row, topk_weights, out=out)


def permute_by_expert(recv_x: torch.Tensor, recv_idx: torch.Tensor,
                      recv_w: Optional[torch.Tensor], *, num_local_experts: int,
                      pad_multiple: int = 1, row_group: Optional[torch.Tensor] = None,
                      num_groups: int = 1) -> Regrouped:
    """The received rows regrouped so that each local expert's rows are
    contiguous, each expert padded to ``pad_multiple`` rows (NeMo
    get_permuted_hidden_states_by_experts / dispatch_postprocess with
    moe_router_expert_pad_multiple; Buffer.dispatch expert_alignment).
    ``recv_idx`` holds local expert ids (-1 elsewhere), e.g. the send_idx of
    one destination's segment; an int64 tensor is converted.  With
    ``row_group`` (e.g. the send layout's send_rank) every destination's
    segment is regrouped at once, one after the other."""
    if recv_idx.dtype != torch.int32:
        recv_idx = recv_idx.to(torch.int32)
    return ep_regroup_by_expert(recv_x, recv_idx.contiguous(), recv_w, num_local_experts,
                                pad_multiple, row_group=row_group, num_groups=num_groups)


def restore_by_expert(expert_out: torch.Tensor, regrouped: Regrouped,
                      recv_w: Optional[torch.Tensor], out: Optional[torch.Tensor] = None
                      ) -> torch.Tensor:
    """Expert outputs [rows, H] in the regrouped order back onto the received
    rows (NeMo get_restored_hidden_states_by_experts): weighted by ``recv_w``
    and summed over each row's local slots, or, with ``recv_w=None``, summed
    unweighted."""
    return ep_combine(expert_out, regrouped.row_map, recv_w, out=out)
