"""Dispatcher-level API named after the axolotl "torch_dispatch" page and
vLLM's BatchedPrepareAndFinalize, built on the ``ep_*`` entry points.

This is the collective-free local path: the P destinations are segments of
one send buffer on this GPU (the page's ``group=None`` case), so dispatch
returns the whole send layout and combine reads it back.
"""

from __future__ import annotations

from typing import Callable, List, NamedTuple, Optional, Tuple

import torch

from .ops import (Counts, Regrouped, SendLayout, ep_batched_prepare, ep_batched_prepare_fp8,
                  ep_build_send_layout, ep_combine, ep_compute_send_counts,
                  ep_counts_workspace_bytes, ep_dispatch_layout, ep_dispatch_layout_chunked,
                  ep_dispatch_layout_chunked_workspace_bytes, ep_dispatch_permute,
                  ep_layout_workspace_bytes, ep_regroup_by_expert, workspace_for)

__all__ = [
    "chunk_bounds",
    "to_host",
    "compute_send_counts",
    "build_send_layout",
    "DispatchHandle",
    "dispatch",
    "combine",
    "dispatch_chunked_forward",
    "ChunkedDispatcher",
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


class ChunkedDispatcher:
    """dispatch -> local kernel -> combine over contiguous token chunks,
    alternating over HIP streams (axolotl "torch_dispatch":
    dispatch_chunked_forward, chunk_bounds).

    Everything a forward touches is allocated once, for one shape (T, K, H,
    P, E_local, chunks): the counts, each chunk's send layout and send
    buffer (bf16, or fp8 codes + per-128-channel scales), the side streams
    and (on first use) the workspaces, so repeated forwards allocate nothing
    but events.

    ``streams`` S counts the caller's stream: stream 0 is the stream current
    at each forward (so the first chunk waits for nothing), and S - 1 side
    streams are created here; chunk c runs on stream c mod S.  One forward,
    in enqueue order:
      1. without ``exact_counts``: the counts of every chunk and all the
         chunks' send layouts in ONE launch on the caller's stream
         (ep_dispatch_layout_chunked), each chunk with its worst case
         T_c * min(K, P) rows, so nothing waits on the host;
         with ``exact_counts``: one count pass over every chunk ([C, P]) on
         the caller's stream, the counts reach the host in ONE copy and size
         each chunk exactly, then the send layouts, the first chunk's on its
         own stream and the later chunks' back to back on the next stream
         (latency-bound, they run while the first chunk's rows stream);
      2. chunk 0's row permute; then for each chunk c, on its stream: chunk
         c+1's row permute (on chunk c+1's stream, after its layout),
         ``local_kernel(c, recv_x, recv_idx, recv_w)`` (bf16 expert output
         [rows, H], enqueued on chunk c's stream), then chunk c's weighted
         combine into out[start:end];
      3. the caller's stream waits for the side streams.
    So chunk c+1's dispatch is issued before chunk c's local kernel, and
    chunk c's combine is enqueued after chunk c+1's dispatch.
    ``timer`` (start(name, stream) / stop(token)) brackets every launch with
    events; ``serialize`` puts all of it on the caller's stream."""

    def __init__(self, num_tokens: int, num_topk: int, hidden: int, *, num_local_experts: int,
                 num_ranks: int, chunks: int, fp8: bool = False, streams: int = 2,
                 exact_counts: bool = False, device=None):
        self.T, self.K, self.H = int(num_tokens), int(num_topk), int(hidden)
        self.P, self.El, self.C = int(num_ranks), int(num_local_experts), int(chunks)
        self.fp8, self.exact_counts = bool(fp8), bool(exact_counts)
        dev = torch.device(device) if device is not None else torch.device(
            "cuda", torch.cuda.current_device())
        if dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        if int(streams) < 1:
            raise ValueError("at least one stream")
        self.side_streams = [torch.cuda.Stream(device=dev) for _ in range(int(streams) - 1)]
        self.bounds = chunk_bounds(self.T, self.C)
        # one row stride for every chunk: the largest chunk's worst case
        self.stride = max((e - s) * min(self.K, self.P) for s, e in self.bounds)
        self.caps = [self.stride] * self.C
        T, K, P, H = self.T, self.K, self.P, self.H
        self.counts = Counts(
            dest=torch.empty((T, K), dtype=torch.int32, device=dev),
            is_in_rank=torch.empty((T, P), dtype=torch.uint8, device=dev),
            send_counts=torch.empty((self.C, P), dtype=torch.int32, device=dev),
            tokens_per_expert=None,
            diag=torch.empty(1, dtype=torch.int32, device=dev))
        # every chunk's layout in one set of arrays (chunk c's rows from row
        # c * stride), each chunk's layout a view of it
        cap, rows = self.stride, self.stride * self.C
        self.all_layouts = SendLayout(
            send_token_idx=torch.empty(rows, dtype=torch.int32, device=dev),
            send_rank=torch.empty(rows, dtype=torch.int32, device=dev),
            send_idx=torch.empty((rows, K), dtype=torch.int32, device=dev),
            send_w=torch.empty((rows, K), dtype=torch.float32, device=dev),
            token_row=torch.empty((T, K), dtype=torch.int32, device=dev))
        L = self.all_layouts
        self.layouts, self.recv = [], []
        for i, (a, b) in enumerate(self.bounds):
            r = slice(i * cap, (i + 1) * cap)
            self.layouts.append(SendLayout(L.send_token_idx[r], L.send_rank[r], L.send_idx[r],
                                           L.send_w[r], L.token_row[a:b]))
            if self.fp8:
                self.recv.append((torch.empty((cap, H), dtype=torch.float8_e4m3fn, device=dev),
                                  torch.empty((cap, H // 128), dtype=torch.float32, device=dev)))
            else:
                self.recv.append(torch.empty((cap, H), dtype=torch.bfloat16, device=dev))
        self.layout_ws_bytes = ep_layout_workspace_bytes(max(e - s for s, e in self.bounds) or 1,
                                                         P)

    def chunk_stream_index(self, i: int, nstreams: int) -> int:
        """Index of chunk i's stream among ``nstreams`` (0 = the caller's)."""
        return i % nstreams

    def forward(self, x: torch.Tensor, topk_idx: torch.Tensor, topk_weights: torch.Tensor,
                local_kernel: Callable, *, out: Optional[torch.Tensor] = None, timer=None,
                serialize: bool = False) -> torch.Tensor:
        T, K, P, El, H = self.T, self.K, self.P, self.El, self.H
        if tuple(x.shape) != (T, H) or tuple(topk_idx.shape) != (T, K) or \
                tuple(topk_weights.shape) != (T, K):
            raise ValueError(f"inputs must be x [{T}, {H}], topk_idx / topk_weights [{T}, {K}]")
        if out is None:
            out = torch.empty((T, H), dtype=torch.bfloat16, device=self.device)
        main = torch.cuda.current_stream(self.device)
        streams = [main] if serialize else [main] + self.side_streams
        S = len(streams)
        chunk_st = [streams[self.chunk_stream_index(i, S)] for i in range(self.C)]

        def mark(name, st):
            return timer.start(name, st) if timer is not None else None

        def done(tok):
            if tok is not None:
                timer.stop(tok)

        side_started = set()      # side streams that this forward has ordered after the caller

        def join(st):
            """A side stream's first work waits for what the caller enqueued."""
            if st is not main and st not in side_started:
                st.wait_stream(main)
                side_started.add(st)

        laid = []
        if not self.exact_counts:
            # counts and every chunk's layout in one launch, no host sync
            ws = workspace_for(ep_dispatch_layout_chunked_workspace_bytes(T, P, self.C),
                               self.device, main, "fused")
            tk = mark("dispatch_layout", main)
            ep_dispatch_layout_chunked(topk_idx, topk_weights, P, El, self.C, self.stride,
                                       counts=self.counts, out=self.all_layouts, workspace=ws,
                                       stream=main)
            done(tk)
            ready = None
            if any(st is not main for st in chunk_st):
                ready = torch.cuda.Event()
                ready.record(main)
            laid = [(ready, main)] * self.C
        else:
            ws = workspace_for(ep_counts_workspace_bytes(T, P, El, self.C), self.device, main,
                               "counts")
            tk = mark("counts", main)
            ep_compute_send_counts(topk_idx, P, El, self.C, expert_counts=False,
                                   out=self.counts, workspace=ws, stream=main)
            done(tk)
            self.caps = [int(v) for v in to_host(self.counts.send_counts).sum(dim=1)]
            first = next((i for i, (a, b) in enumerate(self.bounds) if b > a), 0)
            lead = chunk_st[first]
            rest = streams[(streams.index(lead) + 1) % S]
            for i, (a, b) in enumerate(self.bounds):
                st = lead if i <= first else rest
                if b > a:
                    join(st)
                    lws = workspace_for(self.layout_ws_bytes, self.device, st)
                    tk = mark("layout", st)
                    ep_build_send_layout(topk_idx[a:b], topk_weights[a:b], self.counts.dest[a:b],
                                         self.counts.send_counts[i], P, El, self.caps[i],
                                         out=self.layouts[i], workspace=lws, stream=st)
                    done(tk)
                ev = torch.cuda.Event()
                ev.record(st)
                laid.append((ev, st))

        def dispatch_chunk(i):
            """Chunk i's row permute on its stream, after its layout."""
            a, b = self.bounds[i]
            st = chunk_st[i]
            ev, lst = laid[i]
            if lst is not st:      # the layout ran on another stream (after the caller's work)
                st.wait_event(ev)
                if st is not main:
                    side_started.add(st)
            lay = self.layouts[i]
            tk = mark("permute_fp8" if self.fp8 else "permute", st)
            if self.fp8:
                q, sc = self.recv[i]
                ep_dispatch_permute(x[a:b], lay.token_row, self.caps[i], fp8=True, out=q,
                                    out_scale=sc, stream=st)
                recv_x = (q, sc)
            else:
                recv_x = ep_dispatch_permute(x[a:b], lay.token_row, self.caps[i],
                                             out=self.recv[i], stream=st)
            done(tk)
            return recv_x

        # Chunk i+1's dispatch is issued before chunk i's local kernel, so on
        # separate streams the next chunk's rows stream while this chunk's
        # expert runs; every chunk has its own send buffer, so nothing waits
        # for the buffer to be read.  Empty chunks have no work.
        live = [i for i, (a, b) in enumerate(self.bounds) if b > a]
        recv = {live[0]: dispatch_chunk(live[0])} if live else {}
        for n, i in enumerate(live):
            if n + 1 < len(live):
                recv[live[n + 1]] = dispatch_chunk(live[n + 1])
            a, b = self.bounds[i]
            st = chunk_st[i]
            lay = self.layouts[i]
            with torch.cuda.stream(st):
                y = local_kernel(i, recv.pop(i), lay.send_idx, lay.send_w)
            tk = mark("combine", st)
            ep_combine(y, lay.token_row, topk_weights[a:b], out=out[a:b], stream=st)
            done(tk)
        for st in side_started:
            main.wait_stream(st)
        return out


def dispatch_chunked_forward(x: torch.Tensor, topk_idx: torch.Tensor, topk_weights: torch.Tensor,
                             local_kernel: Callable, *, num_local_experts: int, num_ranks: int,
                             chunks: int, fp8: bool = False, streams=None,
                             exact_counts: bool = True) -> torch.Tensor:
    """dispatch -> local_kernel -> combine over ``chunks`` token ranges,
    alternating over HIP streams (axolotl dispatch_chunked_forward): one
    ChunkedDispatcher forward.  ``local_kernel(recv_x, recv_idx, recv_w)``
    returns the bf16 expert output [rows, H] of one chunk (recv_x is
    (e4m3 rows, scales) with ``fp8``); it runs on the chunk's stream.  With
    ``exact_counts`` (the default, as on the page) the split counts of every
    chunk reach the host in one copy; otherwise each chunk gets the worst
    case T_c * min(K, P) rows and nothing waits on the host."""
    T, K = topk_idx.shape
    d = ChunkedDispatcher(T, K, x.shape[1], num_local_experts=num_local_experts,
                          num_ranks=num_ranks, chunks=chunks, fp8=fp8,
                          streams=streams if streams is not None else 2,
                          exact_counts=exact_counts, device=x.device)
    return d.forward(x, topk_idx, topk_weights,
                     lambda i, rx, ri, rw: local_kernel(rx, ri, rw))


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
