#!/usr/bin/env python3
"""Throughput of MoE token dispatch + combine on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch of seeded synthetic
routing, with inputs already resident in HBM:
  send layouts:  counts + send layout (one launch) -> row permute -> combine
  batched:       batched prepare (zero-padded) -> combine
  fp8 chunked:   counts and every chunk's send layout (one launch), then per
                 chunk: fp8 quantize-permute -> combine, on one stream or
                 alternating over ``--streams`` HIP streams
The identity expert sits between dispatch and combine: combine reads the send
rows themselves (bf16), or the dequantized fp8 rows prepared before timing.

Every step, warm-up included, starts after a 512 MiB scratch read that clears
the 256 MB Infinity Cache, so each step reads its inputs from HBM, and the
cache holds only clean lines (a clearing write would leave up to 256 MB of
its own dirty lines for the step to write back).  A step is charged for the
lines it leaves dirty: its time runs to the end of the next clearing read,
which writes them back, minus the time that read takes on a clean cache.
``--back-to-back`` times K uninterrupted steps instead.

Prints ONE JSON line.  ``value`` is algorithmic HBM bytes per step / step
time (GB/s); tokens/s and the fraction of the 8 TB/s HBM peak ride along.
``roofline`` describes the dominant kernel, timed with HIP events on its own
stream; ``cpu_baseline`` times the CPU oracle on a bounded token sample.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "dispatch+combine HBM GB/s (% of peak) + tokens/s, T=16384 H=7168 E=256 K=8"
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "skewed_t16384"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic bytes (the minimum each kernel must move)
# ---------------------------------------------------------------------------

def bytes_counts(T, K, P, E, C):
    return 8 * T * K + 4 * T * K + T * P + 4 * C * (P + E)


def bytes_layout(T, K, P, N):
    return (8 + 4 + 4) * T * K + 4 * P + N * (8 + 8 * K) + 4 * T * K


def bytes_dispatch_layout(T, K, P, E, N):
    # reads ids + weights, writes dest, is_in_rank, counts, the send rows' metadata, token_row
    return 12 * T * K + 4 * T * K + T * P + 4 * (P + E) + N * (8 + 8 * K) + 4 * T * K


def bytes_dispatch_layout_chunked(T, K, P, C, N):
    # counts of C chunks and every chunk's layout in one launch: reads ids +
    # weights, writes dest, is_in_rank, the [C, P] counts, the send rows'
    # metadata and token_row (no expert counts)
    return 12 * T * K + 4 * T * K + T * P + 4 * C * P + N * (8 + 8 * K) + 4 * T * K


def bytes_permute(H, U, N):
    return 2 * H * U + 2 * H * N


def bytes_permute_fp8(H, U, N):
    return 2 * H * U + N * (H + 4 * (H // 128))


def bytes_combine(H, T, K, R):
    return 2 * H * R + 8 * T * K + 2 * H * T


def bytes_batched(H, T, K, El, M, U_local):
    return 2 * H * U_local + 8 * T * K + 2 * H * El * M + 4 * El + 4 * T * K


def bytes_batched_fp8(H, T, K, El, M, U_local, units):
    # bf16 rows of the local tokens and the ids in; e4m3 rows, one 32-bit
    # scale word per unit (128 channels, or 512 with UE8M0), counts and
    # token_row out, padding included
    return 2 * H * U_local + 8 * T * K + H * El * M + 4 * units * El * M + 4 * El + 4 * T * K


# ---------------------------------------------------------------------------

class Timer:
    """HIP events around each kernel launch, on the launching stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def start(self, name, stream):
        ev = self.torch.cuda.Event(enable_timing=True)
        ev.record(stream)
        return (name, ev, stream)

    def stop(self, tok):
        name, ev0, stream = tok
        ev1 = self.torch.cuda.Event(enable_timing=True)
        ev1.record(stream)
        self.pairs.setdefault(name, []).append((ev0, ev1))

    def averages_us(self):
        return {k: 1000.0 * float(np.mean([a.elapsed_time(b) for a, b in v]))
                for k, v in self.pairs.items()}


def build_send_step(torch, ep, s, d_idx, d_w, d_x):
    T, K, P, El, H = s.T, s.K, s.P, s.E_local, s.H
    cap = T * min(K, P)
    dev = d_x.device
    counts, lay = ep.ep_dispatch_layout(d_idx, d_w, P, El, cap)
    send_x = torch.empty((cap, H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ws = ep.workspace_for(ep.ep_dispatch_layout_workspace_bytes(T, P, El), dev, kind="fused")

    def step(timer=None):
        st = torch.cuda.current_stream()
        # counts + send layout in one launch (worst-case capacity, no host sync)
        tk = timer.start("dispatch_layout", st) if timer else None
        ep.ep_dispatch_layout(d_idx, d_w, P, El, cap, counts=counts, out=lay, workspace=ws)
        if timer:
            timer.stop(tk)
            tk = timer.start("permute", st)
        ep.ep_dispatch_permute(d_x, lay.token_row, cap, out=send_x)
        if timer:
            timer.stop(tk)
            tk = timer.start("combine", st)
        ep.ep_combine(send_x, lay.token_row, d_w, out=out)
        if timer:
            timer.stop(tk)

    step()
    torch.cuda.synchronize()
    N = int(counts.send_counts.sum().item())
    U = int(((d_idx >= 0).any(dim=1)).sum().item())
    kb = {
        "dispatch_layout": bytes_dispatch_layout(T, K, P, s.E, N),
        "permute": bytes_permute(H, U, N),
        "combine": bytes_combine(H, T, K, N),
    }
    info = {"num_send": N, "routed_tokens": U, "capacity": cap,
            "send_counts": counts.send_counts[0].tolist()}
    return step, kb, info


def bytes_regroup(H, N, K, M, M_data, B):
    # ids, weights and row groups of the N received rows; row_map, the source
    # and weight of every regrouped row, counts and offsets; rows: each
    # received row read once, every regrouped row (padding included) written
    return (4 + 4) * N * K + 4 * N + 4 * N * K + 8 * M + 4 * (2 * B + 1) + 2 * H * N + 2 * H * M


def build_expert_major_step(torch, ep, s, d_idx, d_w, d_x):
    """Dispatch, then every destination's received rows regrouped by local
    expert (aligned), an identity expert, the weighted restore onto the send
    rows, and the unweighted combine of the per-destination partials.  The
    receivers' row count N is known on the host, as after a count exchange
    (routing is fixed, so it is taken once in the setup)."""
    T, K, P, El, H, A = s.T, s.K, s.P, s.E_local, s.H, s.align
    cap = T * min(K, P)
    B = P * El
    cap_m = T * K + B * (A - 1)        # one row per routed slot, plus padding
    dev = d_x.device
    counts, lay = ep.ep_dispatch_layout(d_idx, d_w, P, El, cap)
    torch.cuda.synchronize()
    N = int(counts.send_counts.sum().item())
    send_x = torch.empty((cap, H), dtype=torch.bfloat16, device=dev)
    y_send = torch.empty((N, H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    reg = ep.Regrouped(
        perm_x=torch.empty((cap_m, H), dtype=torch.bfloat16, device=dev),
        perm_src=torch.empty(cap_m, dtype=torch.int32, device=dev),
        perm_w=torch.empty(cap_m, dtype=torch.float32, device=dev),
        tokens_per_expert=torch.empty(B, dtype=torch.int32, device=dev),
        expert_offsets=torch.empty(B + 1, dtype=torch.int32, device=dev),
        row_map=torch.empty((N, K), dtype=torch.int32, device=dev))
    ws = ep.workspace_for(ep.ep_dispatch_layout_workspace_bytes(T, P, El), dev, kind="fused")
    ws_r = ep.workspace_for(ep.ep_regroup_workspace_bytes(N, B), dev, kind="regroup")
    recv_x, recv_idx, recv_w, recv_rank = send_x[:N], lay.send_idx[:N], lay.send_w[:N], \
        lay.send_rank[:N]

    def step(timer=None):
        st = torch.cuda.current_stream()
        tk = timer.start("dispatch_layout", st) if timer else None
        ep.ep_dispatch_layout(d_idx, d_w, P, El, cap, counts=counts, out=lay, workspace=ws)
        if timer:
            timer.stop(tk)
            tk = timer.start("permute", st)
        ep.ep_dispatch_permute(d_x, lay.token_row, cap, out=send_x)
        if timer:
            timer.stop(tk)
            tk = timer.start("regroup", st)
        ep.ep_regroup_by_expert(recv_x, recv_idx, recv_w, El, A, cap_m, row_group=recv_rank,
                                num_groups=P, out=reg, workspace=ws_r)
        if timer:
            timer.stop(tk)
            tk = timer.start("restore", st)
        ep.ep_combine(reg.perm_x, reg.row_map, recv_w, out=y_send)
        if timer:
            timer.stop(tk)
            tk = timer.start("combine", st)
        ep.ep_combine(y_send, lay.token_row, None, out=out)
        if timer:
            timer.stop(tk)

    step()
    torch.cuda.synchronize()
    U = int(((d_idx >= 0).any(dim=1)).sum().item())
    M = int(reg.expert_offsets[-1].item())
    M_data = int(reg.tokens_per_expert.sum().item())
    kb = {
        "dispatch_layout": bytes_dispatch_layout(T, K, P, s.E, N),
        "permute": bytes_permute(H, U, N),
        "regroup": bytes_regroup(H, N, K, M, M_data, B),
        "restore": 2 * H * M_data + 8 * N * K + 2 * H * N,
        "combine": 2 * H * N + 4 * T * K + 2 * H * T,
    }
    info = {"num_send": N, "routed_tokens": U, "capacity": cap, "regrouped_rows": M,
            "regrouped_data_rows": M_data, "align": A,
            "send_counts": counts.send_counts[0].tolist()}
    return step, kb, info


def build_batched_step(torch, ep, s, d_idx, d_w, d_x):
    T, K, El, H, M = s.T, s.K, s.E_local, s.H, s.max_num_tokens
    first = s.first_expert
    dev = d_x.device
    b_x = torch.empty((El, M, H), dtype=torch.bfloat16, device=dev)
    tpe = torch.empty(El, dtype=torch.int32, device=dev)
    trow = torch.empty((T, K), dtype=torch.int32, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ws = ep.workspace_for(ep.ep_batched_workspace_bytes(T, El, M), dev)

    def step(timer=None):
        st = torch.cuda.current_stream()
        tk = timer.start("batched_prepare", st) if timer else None
        ep.ep_batched_prepare(d_x, d_idx, first, El, M, out=b_x, tokens_per_expert=tpe,
                              token_row=trow, workspace=ws)
        if timer:
            timer.stop(tk)
            tk = timer.start("combine", st)
        ep.ep_combine(b_x, trow, d_w, out=out)
        if timer:
            timer.stop(tk)

    step()
    torch.cuda.synchronize()
    local = (d_idx >= first) & (d_idx < first + El)
    U_local = int(local.any(dim=1).sum().item())
    rows = int(tpe.sum().item())
    kb = {
        "batched_prepare": bytes_batched(H, T, K, El, M, U_local),
        "combine": bytes_combine(H, T, K, rows),
    }
    return step, kb, {"rows": rows, "local_tokens": U_local,
                      "tokens_per_expert": tpe.tolist()}


def dequantize_batched(torch, q, sc, scale_fmt):
    """bf16 fl32(decode(q) * scale) of an fp8 batched buffer: the output of an
    identity expert behind fp8, the combine's input (built outside the timed
    region)."""
    El, M, H = q.shape
    if scale_fmt == "ue8m0":
        b = sc.contiguous().view(torch.uint8).to(torch.int32)        # [El, M, H/128] bytes
        scale = torch.ldexp(torch.ones_like(b, dtype=torch.float32), b - 127)
    else:
        scale = sc.contiguous()
    vals = q.float().view(El, M, H // 128, 128) * scale[..., None]
    return vals.view(El, M, H).to(torch.bfloat16)


def build_batched_fp8_step(torch, ep, s, d_idx, d_w, d_x):
    T, K, El, H, M = s.T, s.K, s.E_local, s.H, s.max_num_tokens
    first, fmt, colm = s.first_expert, s.scale_fmt, s.scale_col_major
    dev = d_x.device
    b_q = torch.empty((El, M, H), dtype=torch.float8_e4m3fn, device=dev)
    b_s = ep.batched_scale_like(El, M, H, fmt, colm, dev)
    tpe = torch.empty(El, dtype=torch.int32, device=dev)
    trow = torch.empty((T, K), dtype=torch.int32, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ws = ep.workspace_for(ep.ep_batched_workspace_bytes(T, El, M), dev)
    ep.ep_batched_prepare_fp8(d_x, d_idx, first, El, M, scale_fmt=fmt, scale_col_major=colm,
                              out=b_q, out_scale=b_s, tokens_per_expert=tpe, token_row=trow,
                              workspace=ws)
    y = dequantize_batched(torch, b_q, b_s, fmt)

    def step(timer=None):
        st = torch.cuda.current_stream()
        tk = timer.start("batched_prepare_fp8", st) if timer else None
        ep.ep_batched_prepare_fp8(d_x, d_idx, first, El, M, scale_fmt=fmt,
                                  scale_col_major=colm, out=b_q, out_scale=b_s,
                                  tokens_per_expert=tpe, token_row=trow, workspace=ws)
        if timer:
            timer.stop(tk)
            tk = timer.start("combine", st)
        ep.ep_combine(y, trow, d_w, out=out)
        if timer:
            timer.stop(tk)

    step()
    torch.cuda.synchronize()
    local = (d_idx >= first) & (d_idx < first + El)
    U_local = int(local.any(dim=1).sum().item())
    rows = int(tpe.sum().item())
    units = H // (512 if fmt == "ue8m0" else 128)
    kb = {
        "batched_prepare_fp8": bytes_batched_fp8(H, T, K, El, M, U_local, units),
        "combine": bytes_combine(H, T, K, rows),
    }
    return step, kb, {"rows": rows, "local_tokens": U_local, "scale_fmt": fmt,
                      "scale_col_major": colm, "tokens_per_expert": tpe.tolist()}


def build_fp8_chunked_step(torch, ep, s, d_idx, d_w, d_x):
    """The chunked fp8 workload through the library's ChunkedDispatcher, the
    same object the parity tests run: the counts and every chunk's send
    layout in one launch with the worst-case capacities (no host sync), then
    per chunk the fp8 quantize-permute and the combine, chunk i+1's permute
    issued before chunk i's expert: all on the caller's stream, or chunk c on
    stream c mod S of S streams, the caller's first.  The identity expert
    behind fp8 returns y = bf16(decode(q) * scale), built once before
    timing."""
    T, K, P, El, H, C = s.T, s.K, s.P, s.E_local, s.H, s.chunks
    disp = ep.ChunkedDispatcher(T, K, H, num_local_experts=El, num_ranks=P, chunks=C, fp8=True,
                                streams=s.streams, exact_counts=False, device=d_x.device)
    ys = [None] * C

    def dequantize(i, recv, idx, w):
        q, sc = recv
        n = q.shape[0]
        ys[i] = (q.float().view(n, H // 128, 128) * sc[:, :, None]).view(n, H).to(torch.bfloat16)
        return ys[i]

    out = torch.empty((T, H), dtype=torch.bfloat16, device=d_x.device)
    disp.forward(d_x, d_idx, d_w, dequantize, out=out)
    torch.cuda.synchronize()

    def identity_expert(i, recv, idx, w):
        return ys[i]

    def step(timer=None):
        # The per-kernel timing pass runs every chunk on one stream, so each
        # launch's duration is its own and not shared with the other stream's.
        disp.forward(d_x, d_idx, d_w, identity_expert, out=out, timer=timer,
                     serialize=timer is not None)

    step()
    torch.cuda.synchronize()
    sc_host = disp.counts.send_counts.cpu().numpy()
    kb = {"dispatch_layout": bytes_dispatch_layout_chunked(T, K, P, C, int(sc_host.sum())),
          "permute_fp8": 0, "combine": 0}
    Ns = []
    for i, (a, b) in enumerate(disp.bounds):
        N = int(sc_host[i].sum())
        U = int(((d_idx[a:b] >= 0).any(dim=1)).sum().item())
        Ns.append(N)
        kb["permute_fp8"] += bytes_permute_fp8(H, U, N)
        kb["combine"] += bytes_combine(H, b - a, K, N)
    # per-launch bytes of the per-chunk kernels: averages over the C launches
    per_launch = {k: (v / C if k != "dispatch_layout" else v) for k, v in kb.items()}
    return step, kb, {"num_send_per_chunk": Ns, "per_launch_bytes": per_launch,
                      "send_counts": sc_host.sum(axis=0).tolist(),
                      "kernel_timing": "chunks serialized on one stream in the per-kernel pass"}


# ---------------------------------------------------------------------------

def cpu_baseline(s, budget_tokens):
    """Time the CPU oracle (single-threaded numpy) on the first
    ``budget_tokens`` tokens of the same workload, over the same phases."""
    import oracle as O
    from epgen import make_hidden, make_routing

    sub = s.replace(T=budget_tokens)
    idx, w = make_routing(sub)
    x = make_hidden(sub)
    T, K, H = sub.T, sub.K, sub.H
    t0 = time.perf_counter()
    if s.layout == "expert_major":
        El, P, A = s.E_local, s.P, s.align
        sti, srk, sidx, sw, trow = O.build_send_layout(idx, w, P, El)
        N = len(sti)
        sx = O.dispatch_permute(x, sti)
        px, src, pw, cnt, off, rmap = O.regroup_by_expert(sx, sidx, sw, El, A, row_group=srk,
                                                          num_groups=P)
        y = O.combine(px, rmap, sw)
        O.combine_partials(y, trow)
        U = int((idx >= 0).any(axis=1).sum())
        M, Md = int(off[-1]), int(cnt.sum())
        nbytes = (bytes_dispatch_layout(T, K, P, s.E, N) + bytes_permute(H, U, N) +
                  bytes_regroup(H, N, K, M, Md, P * El) + 2 * H * Md + 8 * N * K + 2 * H * N +
                  2 * H * N + 4 * T * K + 2 * H * T)
    elif s.layout == "batched" and s.fp8:
        # max_num_tokens scaled with the sample, so padding keeps its share
        El, M = s.E_local, -(-s.max_num_tokens * T // s.T)
        bq, bs, tpe, trow = O.batched_prepare_fp8(x, idx, s.first_expert, El, M, s.scale_fmt)
        # the identity expert behind fp8 (untimed, as on the GPU): the used rows dequantized
        t_prep = time.perf_counter()
        used, local = np.unique(trow[trow >= 0], return_inverse=True)
        lrow = np.full(trow.shape, -1, dtype=np.int32)
        lrow[trow >= 0] = local
        scales = bs.reshape(El * M, -1)[used]
        if s.scale_fmt == "ue8m0":
            scales = O.ue8m0_decode(O.unpack_ue8m0(scales))
        y = O.dequantize_rows_fp8(bq.reshape(El * M, H)[used], scales)
        t0 += time.perf_counter() - t_prep
        O.combine(y, lrow, w)
        U_local = int(((idx >= s.first_expert) & (idx < s.first_expert + El)).any(axis=1).sum())
        units = H // (512 if s.scale_fmt == "ue8m0" else 128)
        nbytes = bytes_batched_fp8(H, T, K, El, M, U_local, units) + \
            bytes_combine(H, T, K, int(tpe.sum()))
    elif s.layout == "batched":
        bx, tpe, trow = O.batched_prepare(x, idx, s.first_expert, s.E_local, s.max_num_tokens)
        O.combine(bx.reshape(-1, H), trow, w)
        U_local = int(((idx >= s.first_expert) & (idx < s.first_expert + s.E_local))
                      .any(axis=1).sum())
        nbytes = bytes_batched(H, T, K, s.E_local, s.max_num_tokens, U_local) + \
            bytes_combine(H, T, K, int(tpe.sum()))
    else:
        nbytes, N_all = 0, 0
        for a, b in O.chunk_bounds(T, s.chunks):
            O.compute_send_counts(idx[a:b], s.P, s.E_local, 1)
            sti, srk, sidx, sw, trow = O.build_send_layout(idx[a:b], w[a:b], s.P, s.E_local)
            N = len(sti)
            N_all += N
            U = int((idx[a:b] >= 0).any(axis=1).sum())
            if s.fp8:
                q, sc = O.dispatch_permute_fp8(x[a:b], sti)
                # the identity expert behind fp8 (untimed, as on the GPU)
                t_prep = time.perf_counter()
                y = O.dequantize_rows_fp8(q, sc)
                t0 += time.perf_counter() - t_prep
                nbytes += bytes_permute_fp8(H, U, N)
            else:
                y = O.dispatch_permute(x[a:b], sti)
                nbytes += bytes_permute(H, U, N)
            O.combine(y, trow, w[a:b])
            nbytes += bytes_combine(H, b - a, K, N)
            if s.chunks == 1:    # the GPU step counts the one-launch counts + layout
                nbytes += bytes_dispatch_layout(b - a, K, s.P, s.E, N)
        if s.chunks > 1:         # ... and every chunk's counts and layout in one launch
            nbytes += bytes_dispatch_layout_chunked(T, K, s.P, s.chunks, N_all)
    dt = time.perf_counter() - t0
    return {
        "value": round(nbytes / dt / 1e9, 4),
        "unit": "GB/s",
        "tokens_per_s": round(T / dt, 1),
        "seconds": round(dt, 3),
        "cores": 1,
        "host_cpus": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": (f"the whole {s.name} workload" if T == s.T else
                   f"first {T} tokens of the {s.name} workload") +
                  " (same generator and seed), all phases, numpy single-threaded" +
                  (f", max_num_tokens scaled to {-(-s.max_num_tokens * T // s.T)}"
                   if s.layout == "batched" and s.fp8 else ""),
    }


KERNEL_SOURCES = ("scan.hip", "fused.hip", "rows.hip", "api.hip", "epdc_device.h",
                  "epdc_launch.h")


def kernel_source_digest():
    """SHA-256 over the library's sources (the measured traffic is only
    valid for the code it was measured on)."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "combine_ep_send_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_from_profiles(workload, kernel_name, source_digest):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE
    (each scaled by its reading for a plain 1 GiB copy), if a committed
    summary exists for this workload, kernel and kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}_{kernel_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != source_digest:
        return None
    return rec


def row_skew(info):
    """Rows per destination (send layouts) or per local expert (batched):
    smallest, largest, mean and largest / mean."""
    rows = info.get("send_counts", info.get("tokens_per_expert"))
    if not rows:
        return {}
    r = np.asarray(rows, dtype=np.float64)
    what = "destination" if "send_counts" in info else "local_expert"
    return {f"rows_per_{what}": {"min": int(r.min()), "max": int(r.max()),
                                 "mean": round(float(r.mean()), 2),
                                 "max_over_mean": round(float(r.max() / r.mean()), 3)
                                 if r.mean() > 0 else None}}


class CacheClear:
    """Reads 512 MiB of device memory (a max over 128 Mi floats), which
    evicts everything the 256 MB Infinity Cache held and leaves it clean;
    lines left dirty before it are written back during it."""

    def __init__(self, torch, dev):
        self.torch = torch
        self.buf = torch.ones((512 << 20) // 4, dtype=torch.float32, device=dev)

    def run(self):
        self.buf.max()

    def clean_ms(self, stream, n=12):
        """Median time of the read on an already clean cache."""
        t = self.torch
        self.run()
        ts = []
        for _ in range(n):
            e0 = t.cuda.Event(enable_timing=True)
            e1 = t.cuda.Event(enable_timing=True)
            e0.record(stream)
            self.run()
            e1.record(stream)
            t.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-tokens", type=int, default=None,
                    help="tokens in the CPU-oracle sample (default: sized for ~15 s)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--streams", type=int, default=None,
                    help="HIP streams the chunked workload's chunks alternate over (default: "
                         "the workload's own, 1 for fp8_t32768; 2 runs the pipelined schedule)")
    ap.add_argument("--back-to-back", action="store_true",
                    help="run the timed steps back to back under one pair of events, "
                         "without clearing the Infinity Cache between steps (by default "
                         "every step, warm-up included, follows a 512 MiB scratch read "
                         "outside its events, so no step finds its inputs in the cache)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run five plain 1 GiB device copies (the reference kernel for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the library has no exchange between GPUs)", file=sys.stderr)
        return 2

    import torch

    import combine_ep_send_amd as ep
    from epgen import make_hidden, make_routing, spec

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.copy_calibration:
        n = 1 << 30
        a = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda:0")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                          "launches": 5}), flush=True)
        return 0
    ep.lib()                                   # fail loudly if the library is missing
    s = spec(args.workload)
    if args.streams is not None:
        if args.streams < 1 or s.chunks < 2:
            print("--streams takes a count >= 1 and applies to a chunked workload",
                  file=sys.stderr)
            return 2
        s = s.replace(streams=args.streams)
    log(f"[bench] workload {s.name}: T={s.T} H={s.H} E={s.E} K={s.K} P={s.P} "
        f"layout={s.layout} fp8={s.fp8} chunks={s.chunks}")
    idx, w = make_routing(s)
    x = make_hidden(s)
    dev = torch.device("cuda:0")
    d_idx = torch.from_numpy(idx).to(dev)
    d_w = torch.from_numpy(w).to(dev)
    d_x = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    del x

    if s.layout == "batched" and s.fp8:
        step, kbytes, info = build_batched_fp8_step(torch, ep, s, d_idx, d_w, d_x)
    elif s.layout == "batched":
        step, kbytes, info = build_batched_step(torch, ep, s, d_idx, d_w, d_x)
    elif s.layout == "expert_major":
        step, kbytes, info = build_expert_major_step(torch, ep, s, d_idx, d_w, d_x)
    elif s.fp8:
        step, kbytes, info = build_fp8_chunked_step(torch, ep, s, d_idx, d_w, d_x)
    else:
        step, kbytes, info = build_send_step(torch, ep, s, d_idx, d_w, d_x)
    total_bytes = int(sum(kbytes.values()))
    log(f"[bench] setup done: {info}; algorithmic bytes/step = {total_bytes / 1e9:.4f} GB")

    main_stream = torch.cuda.current_stream()
    # 512 MiB of scratch: twice the Infinity Cache, so reading it evicts every
    # line a previous step left there, and leaves only clean lines behind (a
    # clearing write would leave up to 256 MB of its own dirty lines for the
    # next step to write back: 2 % of the write-heavy batched step).
    scratch = (CacheClear(torch, dev) if not args.back_to_back else None)
    for _ in range(args.warmup):
        if scratch is not None:
            scratch.run()
        step()
    torch.cuda.synchronize()
    log(f"[bench] {args.warmup} warmup steps done")
    if scratch is None:
        # Timed region: K whole steps between two events on the main stream
        # (the chunked workload joins its side streams back into it every step).
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(main_stream)
        for _ in range(args.steps):
            step()
        ev1.record(main_stream)
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / args.steps
        step_ms = [ms]
    else:
        # Each step starts on a cleared cache and is charged for the lines it
        # leaves dirty: its interval runs from before the step to after the
        # next clearing read, which writes those lines back, and the time the
        # same read takes on a clean cache is subtracted.
        clear_ms = scratch.clean_ms(main_stream)
        scratch.run()
        evs = []
        for _ in range(args.steps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e2 = torch.cuda.Event(enable_timing=True)
            e0.record(main_stream)
            step()
            e1.record(main_stream)
            scratch.run()
            e2.record(main_stream)
            evs.append((e0, e1, e2))
        torch.cuda.synchronize()
        step_ms = [a.elapsed_time(c) - clear_ms for a, _, c in evs]
        events_ms = [a.elapsed_time(b) for a, b, _ in evs]
        ms = float(np.mean(step_ms))
    log(f"[bench] {args.steps} timed steps: {ms:.4f} ms/step (events)")

    # Per-kernel durations: the same K steps again, each kernel bracketed by
    # HIP events on the stream it is launched on.  (Events between kernels
    # cost a few microseconds each, so this pass is kept out of the step time.)
    timer = Timer(torch)
    for _ in range(args.steps):
        if scratch is not None:
            scratch.run()
        step(timer)
    torch.cuda.synchronize()
    kern_us = timer.averages_us()
    # every bounded wait of the steps above must have ended normally: a wait
    # that gave up leaves its flag in the workspace, and that step's outputs
    # would be undefined
    ws_errors = sum(1 for f, _, _ in ep.workspace_flags() if f)
    if ws_errors:
        log(f"[bench] {ws_errors} workspace(s) report a bounded wait that gave up")
    per_launch = info.get("per_launch_bytes", kbytes)
    dom = max((k for k in kern_us if k not in ("counts", "layout", "dispatch_layout",
                                                   "regroup")),
              key=lambda k: kern_us[k])
    dom_gbs = per_launch[dom] / (kern_us[dom] * 1e-6) / 1e9
    trec = traffic_from_profiles(s.name, dom, kernel_source_digest())

    gbs = total_bytes / (ms * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "ms_per_step_median": round(float(np.median(step_ms)), 5),
        "ms_per_step_min": round(float(np.min(step_ms)), 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if not s.fp8 else "fp8-e4m3+bf16",
        "data": "synthetic",
        "config": {
            "workload": s.name, "T": s.T, "H": s.H, "E": s.E, "K": s.K, "P": s.P,
            "routing": s.routing + (f"(s={s.zipf_s})" if s.routing == "zipf" else ""),
            "unrouted_frac": s.unrouted_frac, "layout": s.layout, "chunks": s.chunks,
            "streams": s.streams, "seed": s.seed, "parallelism": "single GPU",
            "mall_flush_between_steps": not args.back_to_back,
            **{k: v for k, v in info.items() if k != "per_launch_bytes"},
            **row_skew(info),
        },
        "pct_of_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(s.T / (ms * 1e-3), 1),
        "alg_bytes_per_step": total_bytes,
        "step_timing": ("one event pair around K back-to-back steps" if args.back_to_back else
                        "each step starts on a cache cleared by a 512 MiB read; its time "
                        "runs to the end of the next clearing read (which writes back the "
                        "lines the step left dirty) minus that read's time on a clean cache"),
        **({} if args.back_to_back else {
            "clean_clear_ms": round(clear_ms, 5),
            "ms_per_step_to_last_kernel": round(float(np.mean(events_ms)), 5)}),
        "kernel_avg_us": {k: round(v, 3) for k, v in kern_us.items()},
        "workspace_errors": ws_errors,
        "roofline": {
            "kernel": dom,
            "bound": "hbm",
            "achieved": round(dom_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
            "traffic": (trec["read_bytes_per_launch"] + trec["write_bytes_per_launch"]
                        if trec else None),
            "traffic_read_write": ([trec["read_bytes_per_launch"], trec["write_bytes_per_launch"]]
                                   if trec else None),
            "alg_bytes_per_launch": int(per_launch[dom]),
            "avg_launch_us": round(kern_us[dom], 3),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        whole = {"skewed_t16384": 16384, "uniform_t4096": 4096, "tiny": 256,
                 "batched_t8192": 8192, "fp8_t32768": 6144, "batched_fp8_t8192": 8192,
                 "expert_major_t16384": 16384}
        n = args.cpu_tokens or whole.get(s.name, 1024)
        log(f"[bench] timing the CPU oracle on {n} tokens")
        result["cpu_baseline"] = cpu_baseline(s, n)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
