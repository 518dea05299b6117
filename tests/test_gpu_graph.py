"""The library's calls under HIP graph capture: the send path (counts and
layout in one launch, permute, combine), the batched fp8 layout and the
regroup by expert are captured once and replayed several times, with eager
work and synchronizations between the replays; every replay must equal the
eager result bit for bit.  The calls enqueue kernels only (no memset, no
allocation, no host sync), and their workspaces rearm themselves, so a
replayed barrier or lookback starts from where the last call left it."""

import numpy as np
import pytest
import torch

from epgen import make_hidden, make_routing, spec
from tests.gpu_helpers import to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

import combine_ep_send_amd as ep  # noqa: E402


def _replays(capture_fn, outputs, n=4):
    """Capture capture_fn, then replay it n times; return host copies of the
    outputs after each replay."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        capture_fn()                       # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        capture_fn()
    torch.cuda.synchronize()
    got = []
    for i in range(n):
        for o in outputs:                  # eager work between replays
            o.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got.append([o.view(torch.uint8).cpu().numpy().copy() for o in outputs])
    return got


def test_send_path_graph_replays():
    s = spec("skewed_t16384", T=3000, H=1024)
    idx, w = make_routing(s)
    x = make_hidden(s)
    T, K, P, El, H = s.T, s.K, s.P, s.E_local, s.H
    cap = T * min(K, P)
    d_idx, d_w, d_x = to_dev(idx), to_dev(w), to_dev(x)
    counts, lay = ep.ep_dispatch_layout(d_idx, d_w, P, El, cap)
    send_x = ep.ep_dispatch_permute(d_x, lay.token_row, cap)
    out = ep.ep_combine(send_x, lay.token_row, d_w)
    torch.cuda.synchronize()
    N = int(counts.send_counts.sum().item())
    eager = [lay.token_row.clone(), lay.send_token_idx[:N].clone(), send_x[:N].clone(), out.clone()]
    ws = ep.workspace_for(ep.ep_dispatch_layout_workspace_bytes(T, P, El), d_x.device,
                          kind="graph")

    def step():
        ep.ep_dispatch_layout(d_idx, d_w, P, El, cap, counts=counts, out=lay, workspace=ws)
        ep.ep_dispatch_permute(d_x, lay.token_row, cap, out=send_x)
        ep.ep_combine(send_x, lay.token_row, d_w, out=out)

    outs = [lay.token_row, lay.send_token_idx[:N], send_x[:N], out]
    for rep in _replays(step, outs):
        for got, want in zip(rep, eager):
            assert np.array_equal(got, want.view(torch.uint8).cpu().numpy())
    hdr = ws[:16].view(torch.int32).cpu().numpy()
    assert hdr[3] == 0 and hdr[0] > 0 and hdr[0] == hdr[2]   # no time-out; count handed on


def test_batched_fp8_and_regroup_graph_replays():
    s = spec("batched_t8192", T=2000, H=1536)
    idx, w = make_routing(s)
    x = make_hidden(s)
    T, K, El, H = s.T, s.K, s.E_local, s.H
    d_idx, d_x, d_w = to_dev(idx), to_dev(x), to_dev(w)
    M = 256
    bq, bs, tpe, trow = ep.ep_batched_prepare_fp8(d_x, d_idx, 0, El, M, scale_fmt="ue8m0",
                                                  scale_col_major=True)
    # regroup of this GPU's send buffer (P = 8 destinations) by local expert
    P = s.P
    counts, lay = ep.ep_dispatch_layout(d_idx, d_w, P, El, T * min(K, P))
    N = int(counts.send_counts.sum().item())
    send_x = ep.ep_dispatch_permute(d_x, lay.token_row, T * min(K, P))
    reg = ep.ep_regroup_by_expert(send_x[:N], lay.send_idx[:N], lay.send_w[:N], El, 16,
                                  row_group=lay.send_rank[:N], num_groups=P)
    torch.cuda.synchronize()
    M_r = int(reg.expert_offsets[-1].item())
    bs_mem = bs.transpose(1, 2)           # the scales in memory order (contiguous)
    eager = [bq.clone(), bs_mem.clone(), tpe.clone(), trow.clone(),
             reg.perm_x[:M_r].clone(), reg.row_map.clone(), reg.expert_offsets.clone()]
    ws_b = ep.workspace_for(ep.ep_batched_workspace_bytes(T, El, M), d_x.device, kind="graph_b")
    ws_r = ep.workspace_for(ep.ep_regroup_workspace_bytes(N, P * El), d_x.device, kind="graph_r")

    def step():
        ep.ep_batched_prepare_fp8(d_x, d_idx, 0, El, M, scale_fmt="ue8m0", scale_col_major=True,
                                  out=bq, out_scale=bs, tokens_per_expert=tpe, token_row=trow,
                                  workspace=ws_b)
        ep.ep_regroup_by_expert(send_x[:N], lay.send_idx[:N], lay.send_w[:N], El, 16,
                                row_group=lay.send_rank[:N], num_groups=P, out=reg,
                                workspace=ws_r)

    outs = [bq, bs_mem, tpe, trow, reg.perm_x[:M_r], reg.row_map, reg.expert_offsets]
    for rep in _replays(step, outs):
        for got, want in zip(rep, eager):
            assert np.array_equal(got, want.view(torch.uint8).cpu().numpy())


def test_noalloc_send_path_graph_replays():
    """The send path on the library's own scratch (ep_dispatch_layout_noalloc),
    the use it is for: captured with no allocation, replayed, equal to the
    workspace call's eager result every time."""
    s = spec("skewed_t16384", T=2500, H=512, seed=4)
    idx, w = make_routing(s)
    x = make_hidden(s)
    T, K, P, El = s.T, s.K, s.P, s.E_local
    cap = T * min(K, P)
    d_idx, d_w, d_x = to_dev(idx), to_dev(w), to_dev(x)
    counts, lay = ep.ep_dispatch_layout(d_idx, d_w, P, El, cap)
    send_x = ep.ep_dispatch_permute(d_x, lay.token_row, cap)
    out = ep.ep_combine(send_x, lay.token_row, d_w)
    torch.cuda.synchronize()
    N = int(counts.send_counts.sum().item())
    eager = [lay.token_row.clone(), lay.send_token_idx[:N].clone(), counts.send_counts.clone(),
             send_x[:N].clone(), out.clone()]

    def step():
        ep.ep_dispatch_layout_noalloc(d_idx, d_w, P, El, cap, counts=counts, out=lay)
        ep.ep_dispatch_permute(d_x, lay.token_row, cap, out=send_x)
        ep.ep_combine(send_x, lay.token_row, d_w, out=out)

    outs = [lay.token_row, lay.send_token_idx[:N], counts.send_counts, send_x[:N], out]
    for rep in _replays(step, outs):
        for got, want in zip(rep, eager):
            assert np.array_equal(got, want.view(torch.uint8).cpu().numpy())
    assert ep.library_scratch_status() == 0


def test_chunked_layout_graph_replays():
    """Every chunk's counts and layout in one launch, then each chunk's fp8
    permute and the combine of its dequantized rows, captured and replayed."""
    s = spec("fp8_t32768", T=3000, H=512, seed=6)
    idx, w = make_routing(s)
    x = make_hidden(s)
    T, K, P, El, H, C = s.T, s.K, s.P, s.E_local, s.H, 3
    bounds = ep.chunk_bounds(T, C)
    cap = max((b - a) * min(K, P) for a, b in bounds)
    d_idx, d_w, d_x = to_dev(idx), to_dev(w), to_dev(x)
    counts, lay = ep.ep_dispatch_layout_chunked(d_idx, d_w, P, El, C, cap)
    q = torch.empty((C * cap, H), dtype=torch.float8_e4m3fn, device="cuda")
    sc = torch.empty((C * cap, H // 128), dtype=torch.float32, device="cuda")
    y = torch.zeros((C * cap, H), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ws = ep.workspace_for(ep.ep_dispatch_layout_chunked_workspace_bytes(T, P, C), d_x.device,
                          kind="graph_c")

    def step():
        ep.ep_dispatch_layout_chunked(d_idx, d_w, P, El, C, cap, counts=counts, out=lay,
                                      workspace=ws)
        for i, (a, b) in enumerate(bounds):
            r = slice(i * cap, (i + 1) * cap)
            ep.ep_dispatch_permute(d_x[a:b], lay.token_row[a:b], cap, fp8=True, out=q[r],
                                   out_scale=sc[r])
            y[r] = (q[r].float().view(cap, H // 128, 128) * sc[r][:, :, None]).view(cap, H) \
                .to(torch.bfloat16)
            ep.ep_combine(y[r], lay.token_row[a:b], d_w[a:b], out=out[a:b])

    step()
    torch.cuda.synchronize()
    Ns = counts.send_counts.sum(dim=1).tolist()
    written = [q[i * cap:i * cap + n] for i, n in enumerate(Ns)]   # rows past N untouched
    eager = [lay.token_row.clone(), counts.send_counts.clone(), out.clone()] + \
        [t.view(torch.uint8).clone() for t in written]
    outs = [lay.token_row, counts.send_counts, out] + written
    for rep in _replays(step, outs):
        for got, want in zip(rep, eager):
            assert np.array_equal(got, want.view(torch.uint8).cpu().numpy())
    hdr = ws[:16].view(torch.int32).cpu().numpy()
    assert hdr[3] == 0 and hdr[0] == hdr[2]
