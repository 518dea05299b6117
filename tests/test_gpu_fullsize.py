"""GPU parity at the workloads' full sizes, each run exactly as bench.py
times it, every output element compared with the oracle.

* send workloads (tiny, uniform_t4096, skewed_t16384): counts and layout in
  one launch with the worst-case capacity, the (occupancy-capped) row
  permute and the combine of the send rows (identity expert);
* batched_t8192: the expert-batched fill and the combine over it;
* fp8_t32768: the library's ChunkedDispatcher, 4 chunks, worst-case
  capacities, the fp8 quantize-permute, an identity expert behind fp8
  (y = bf16(decode(q) * scale)) and the combine, on the caller's stream (the
  bench's default) and alternating over 2 streams; run twice, as the bench
  does (the second forward returns the first's expert outputs), and checked
  chunk by chunk.
The oracle's own results are computed on the host from the same seeded
inputs (the full skewed workload in a few seconds)."""

import numpy as np
import pytest
import torch

import oracle as O
from epgen import make_hidden, make_routing, spec
from tests.gpu_helpers import bits, gpu_available, host, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

import combine_ep_send_amd as ep  # noqa: E402


def _load(name, **over):
    s = spec(name, **over)
    print(f"case: full-size {name} T={s.T} H={s.H} E={s.E} K={s.K} P={s.P}", flush=True)
    idx, w = make_routing(s)
    x = make_hidden(s)
    return s, idx, w, x


@pytest.mark.parametrize("name", ["tiny", "uniform_t4096", "skewed_t16384"])
def test_send_workload_full_size(name):
    s, idx, w, x = _load(name)
    T, K, P, El, H = s.T, s.K, s.P, s.E_local, s.H
    cap = T * min(K, P)                      # the bench's no-sync capacity
    d_idx, d_w, d_x = to_dev(idx), to_dev(w), to_dev(x)
    # the bench's step: one-launch counts + layout, permute, combine
    c, lay = ep.ep_dispatch_layout(d_idx, d_w, P, El, cap)
    sx = ep.ep_dispatch_permute(d_x, lay.token_row, cap)
    out = ep.ep_combine(sx, lay.token_row, d_w)
    torch.cuda.synchronize()
    ep.check_workspaces()

    dest, iir, sc, tpe = O.compute_send_counts(idx, P, El, 1)
    assert np.array_equal(host(c.dest), dest)
    assert np.array_equal(host(c.is_in_rank), iir)
    assert np.array_equal(host(c.send_counts), sc)
    assert np.array_equal(host(c.tokens_per_expert), tpe)
    assert int(host(c.diag)[0]) == 0
    sti, srk, sidx, sw, trow = O.build_send_layout(idx, w, P, El)
    N = len(sti)
    print(f"  N={N} send rows", flush=True)
    assert np.array_equal(host(lay.send_token_idx)[:N], sti)
    assert np.array_equal(host(lay.send_rank)[:N], srk)
    assert np.array_equal(host(lay.send_idx)[:N], sidx)
    assert np.array_equal(host(lay.send_w)[:N].view(np.uint32), sw.view(np.uint32))
    assert np.array_equal(host(lay.token_row), trow)
    # every send row, every channel
    ox = O.dispatch_permute(x, sti)
    assert np.array_equal(bits(sx[:N]), ox)
    # every token, every channel (0 ulp; the bar is 1 bf16 ulp)
    ref = O.combine(ox, trow, w)
    del ox
    assert np.array_equal(bits(out), ref)


def test_batched_workload_full_size():
    s, idx, w, x = _load("batched_t8192")
    T, K, H, El, M, first = s.T, s.K, s.H, s.E_local, s.max_num_tokens, s.first_expert
    d_idx, d_w, d_x = to_dev(idx), to_dev(w), to_dev(x)
    bx = torch.full((El, M, H), 1.0, dtype=torch.bfloat16, device="cuda")
    _, tpe, trow = ep.ep_batched_prepare(d_x, d_idx, first, El, M, out=bx)
    out = ep.ep_combine(bx, trow, d_w)
    torch.cuda.synchronize()
    ep.check_workspaces()

    obx, otpe, otrow = O.batched_prepare(x, idx, first, El, M)
    assert np.array_equal(host(tpe), otpe)
    assert np.array_equal(host(trow), otrow)
    print(f"  rows={int(otpe.sum())} max={int(otpe.max())}", flush=True)
    for e in range(El):                      # every row, padding included
        assert np.array_equal(bits(bx[e]), obx[e]), e
    ref = O.combine(obx.reshape(-1, H), otrow, w)
    assert np.array_equal(bits(out), ref)


# ---------------------------------------------------------------------------
# fp8_t32768 as the bench times it
# ---------------------------------------------------------------------------

def _dequantize(q, sc, H):
    n = q.shape[0]
    return (q.float().view(n, H // 128, 128) * sc[:, :, None]).view(n, H).to(torch.bfloat16)


@pytest.fixture(scope="module", params=[1, 2], ids=["1stream", "2streams"])
def fp8_chunked(request):
    s, idx, w, x = _load("fp8_t32768", streams=request.param)
    print(f"  {s.streams} stream(s)", flush=True)
    T, K, P, El, H, C = s.T, s.K, s.P, s.E_local, s.H, s.chunks
    d_idx, d_w, d_x = to_dev(idx), to_dev(w), to_dev(x)
    disp = ep.ChunkedDispatcher(T, K, H, num_local_experts=El, num_ranks=P, chunks=C,
                                fp8=True, streams=s.streams, exact_counts=False)
    ys = [None] * C

    def dequantize(i, recv, ridx, rw):
        ys[i] = _dequantize(recv[0], recv[1], H)
        return ys[i]

    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    disp.forward(d_x, d_idx, d_w, dequantize, out=out)
    first = bits(out)
    out.fill_(7.0)
    # the bench's timed step: the same forward, the expert returning its outputs
    disp.forward(d_x, d_idx, d_w, lambda i, recv, ridx, rw: ys[i], out=out)
    torch.cuda.synchronize()
    ep.check_workspaces()
    got = {"out": bits(out), "first": first, "send_counts": host(disp.counts.send_counts),
           "dest": host(disp.counts.dest), "chunks": []}
    for i, (a, b) in enumerate(disp.bounds):
        N = int(got["send_counts"][i].sum())
        lay = disp.layouts[i]
        q, sc = disp.recv[i]
        got["chunks"].append(dict(
            N=N, token_row=host(lay.token_row), sti=host(lay.send_token_idx)[:N],
            srk=host(lay.send_rank)[:N], sidx=host(lay.send_idx)[:N],
            sw=host(lay.send_w)[:N], q=host(q[:N]), sc=host(sc[:N])))
    del disp, ys
    torch.cuda.empty_cache()
    return s, idx, w, x, got


def test_fp8_chunked_counts_full_size(fp8_chunked):
    s, idx, w, x, got = fp8_chunked
    dest, _, sc, _ = O.compute_send_counts(idx, s.P, s.E_local, s.chunks)
    assert np.array_equal(got["send_counts"], sc)
    assert np.array_equal(got["dest"], dest)
    # the timed forward (expert outputs reused) equals the first one
    assert np.array_equal(got["out"], got["first"])


@pytest.mark.parametrize("chunk", [0, 1, 2, 3])
def test_fp8_chunked_full_size(fp8_chunked, chunk):
    s, idx, w, x, got = fp8_chunked
    a, b = O.chunk_bounds(s.T, s.chunks)[chunk]
    g = got["chunks"][chunk]
    sti, srk, sidx, sw, trow = O.build_send_layout(idx[a:b], w[a:b], s.P, s.E_local)
    N = len(sti)
    print(f"  chunk {chunk}: tokens [{a},{b}) N={N}", flush=True)
    assert g["N"] == N
    assert np.array_equal(g["token_row"], trow)
    assert np.array_equal(g["sti"], sti)
    assert np.array_equal(g["srk"], srk)
    assert np.array_equal(g["sidx"], sidx)
    assert np.array_equal(g["sw"].view(np.uint32), sw.view(np.uint32))
    # every send row's codes and scales
    oq, osc = O.dispatch_permute_fp8(x[a:b], sti)
    assert np.array_equal(g["q"], oq)
    assert np.array_equal(g["sc"].view(np.uint32), osc.view(np.uint32))
    # every token's combine of the identity expert behind fp8
    ref = O.combine(O.dequantize_rows_fp8(oq, osc), trow, w[a:b])
    del oq, osc
    assert np.array_equal(got["out"][a:b], ref)


# ---------------------------------------------------------------------------
# fewer tokens than chunks (leading chunks empty)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1, 3, 5, 7])
@pytest.mark.parametrize("fp8", [False, True])
def test_chunked_pipeline_fewer_tokens_than_chunks(T, fp8):
    s = spec("fp8_t32768", T=T, H=512, seed=T)
    idx, w = make_routing(s)
    x = make_hidden(s)
    C = 4
    print(f"case: chunked pipeline T={T} chunks={C} fp8={fp8}", flush=True)
    d_idx, d_w, d_x = to_dev(idx), to_dev(w), to_dev(x)
    c = ep.ep_compute_send_counts(d_idx, s.P, s.E_local, C)
    dest, iir, sc, tpe = O.compute_send_counts(idx, s.P, s.E_local, C)
    assert np.array_equal(host(c.send_counts), sc)
    assert np.array_equal(host(c.tokens_per_expert), tpe)
    assert np.array_equal(host(c.dest), dest)
    assert np.array_equal(host(c.is_in_rank), iir)

    def expert(rx, ri, rw):
        return _dequantize(rx[0], rx[1], s.H) if fp8 else rx

    for exact in (True, False):
        out = ep.dispatch_chunked_forward(d_x, d_idx, d_w, expert, num_local_experts=s.E_local,
                                          num_ranks=s.P, chunks=C, fp8=fp8, exact_counts=exact)
        torch.cuda.synchronize()
        ref = np.zeros_like(x)
        for a, b in O.chunk_bounds(T, C):
            if b == a:
                continue
            sti, _, _, _, trow = O.build_send_layout(idx[a:b], w[a:b], s.P, s.E_local)
            y = (O.dequantize_rows_fp8(*O.dispatch_permute_fp8(x[a:b], sti)) if fp8
                 else O.dispatch_permute(x[a:b], sti))
            ref[a:b] = O.combine(y, trow, w[a:b])
        assert np.array_equal(bits(out), ref), exact


@pytest.mark.parametrize("streams", [1, 2, 3])
def test_chunked_pipeline_matches_the_oracle_per_chunk_bf16(streams):
    """dispatch_chunked_forward (bf16, exact counts, 1 to 3 streams) equals
    the oracle chunk by chunk."""
    s = spec("fp8_t32768", T=4096, H=1024)
    idx, w = make_routing(s)
    x = make_hidden(s)
    print(f"case: chunked pipeline bf16 T={s.T} H={s.H} streams={streams}", flush=True)
    d_idx, d_w, d_x = to_dev(idx), to_dev(w), to_dev(x)
    out = ep.dispatch_chunked_forward(d_x, d_idx, d_w, lambda rx, ri, rw: rx,
                                      num_local_experts=s.E_local, num_ranks=s.P, chunks=4,
                                      streams=streams)
    torch.cuda.synchronize()
    ref = np.empty_like(x)
    for a, b in O.chunk_bounds(s.T, 4):
        sti, _, _, _, trow = O.build_send_layout(idx[a:b], w[a:b], s.P, s.E_local)
        ref[a:b] = O.combine(O.dispatch_permute(x[a:b], sti), trow, w[a:b])
    assert np.array_equal(bits(out), ref)
