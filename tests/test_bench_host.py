"""Host-side checks of bench.py, no GPU: it refuses more than one GPU before
touching one, and its algorithmic byte counts (the numerator of every GB/s
figure and of the roofline) equal the sizes of the arrays each call must read
and write, counted here from the oracle's outputs on small workloads."""

import os
import subprocess
import sys

import numpy as np
import pytest

import bench as B
import oracle as O
from epgen import make_hidden, make_routing, spec

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert proc.returncode == 2
    assert "one GPU" in proc.stderr and proc.stdout == ""


def _nbytes(*arrays):
    return sum(np.asarray(a).nbytes for a in arrays)


@pytest.mark.parametrize("name,T,H", [("tiny", 256, 512), ("skewed_t16384", 700, 1024),
                                      ("uniform_t4096", 300, 256)])
def test_send_path_bytes_are_the_arrays(name, T, H):
    s = spec(name, T=T, H=H)
    idx, w = make_routing(s)
    x = make_hidden(s)
    K, P, El, E = s.K, s.P, s.E_local, s.E
    dest, iir, sc, tpe = O.compute_send_counts(idx, P, El)
    sti, srk, sidx, sw, trow = O.build_send_layout(idx, w, P, El)
    N = len(sti)
    U = len(np.unique(sti))
    assert U == int((idx >= 0).any(axis=1).sum())

    # counts: ids in; dest, membership, counts and expert counts out
    assert B.bytes_counts(T, K, P, E, 1) == _nbytes(idx, dest, iir, sc, tpe)
    # layout: ids, weights, dest and the counts in; the send rows' metadata
    # and token_row out
    assert B.bytes_layout(T, K, P, N) == _nbytes(idx, w, dest, sc[0], sti, srk, sidx, sw, trow)
    # both in one launch: ids and weights read once, dest and counts written
    assert B.bytes_dispatch_layout(T, K, P, E, N) == \
        _nbytes(idx, w, dest, iir, sc, tpe, sti, srk, sidx, sw, trow)

    # permute: each routed token's row read once, every send row written
    send_x = O.dispatch_permute(x, sti)
    assert B.bytes_permute(H, U, N) == _nbytes(x[np.unique(sti)], send_x)
    q, scales = O.dispatch_permute_fp8(x, sti)
    assert B.bytes_permute_fp8(H, U, N) == _nbytes(x[np.unique(sti)], q, scales)

    # combine: every distinct row named by token_row read once, token_row
    # and the weights, the output rows
    rows = np.unique(trow[trow >= 0])
    assert len(rows) == N
    out = O.combine(send_x, trow, w)
    assert B.bytes_combine(H, T, K, N) == _nbytes(send_x[rows], trow, w, out)


@pytest.mark.parametrize("fmt", [None, "f32", "ue8m0"])
def test_batched_bytes_are_the_arrays(fmt):
    s = spec("batched_t8192", T=300, H=1024, max_num_tokens=40)
    idx, _ = make_routing(s)
    x = make_hidden(s)
    T, K, El, H, M = s.T, s.K, s.E_local, s.H, s.max_num_tokens
    local = ((idx >= 0) & (idx < El)).any(axis=1)
    U_local = int(local.sum())
    if fmt is None:
        b_x, tpe, trow = O.batched_prepare(x, idx, 0, El, M)
        want = _nbytes(x[local], idx, b_x, tpe, trow)
        assert B.bytes_batched(H, T, K, El, M, U_local) == want
    else:
        b_q, b_s, tpe, trow = O.batched_prepare_fp8(x, idx, 0, El, M, fmt)
        units = H // 512 if fmt == "ue8m0" else H // 128
        storage = O.scale_storage(b_s, fmt == "ue8m0")
        assert storage.nbytes == 4 * units * El * M
        want = _nbytes(x[local], idx, b_q, storage, tpe, trow)
        assert B.bytes_batched_fp8(H, T, K, El, M, U_local, units) == want


def test_regroup_bytes_are_the_arrays():
    s = spec("expert_major_t16384", T=400, H=512, align=16)
    idx, w = make_routing(s)
    x = make_hidden(s)
    K, P, El, H = s.K, s.P, s.E_local, s.H
    sti, srk, sidx, sw, _ = O.build_send_layout(idx, w, P, El)
    recv_x = O.dispatch_permute(x, sti)
    N = len(sti)
    perm_x, src, pw, tpe, off, row_map = O.regroup_by_expert(
        recv_x, sidx, sw, El, align=s.align, row_group=srk, num_groups=P)
    M = len(src)
    Bn = P * El
    # ids (int32), weights and row groups of the received rows in; row_map,
    # the source and weight of every regrouped row, counts and offsets out;
    # each received row read once, every regrouped row written
    want = _nbytes(sidx, sw, srk, row_map, src, pw, tpe, off, recv_x, perm_x)
    assert B.bytes_regroup(H, N, K, M, int((src >= 0).sum()), Bn) == want


def test_chunked_one_launch_layout_bytes_are_the_arrays():
    s = spec("fp8_t32768", T=777, H=512)
    idx, w = make_routing(s)
    T, K, P, El, C = s.T, s.K, s.P, s.E_local, s.chunks
    dest, iir, sc, _ = O.compute_send_counts(idx, P, El, C)
    rows, N = [], 0
    for a, b in O.chunk_bounds(T, C):
        sti, srk, sidx, sw, trow = O.build_send_layout(idx[a:b], w[a:b], P, El)
        rows += [sti, srk, sidx, sw]
        N += len(sti)
    # ids and weights in; dest, membership, the [C, P] counts, every chunk's
    # send rows' metadata and token_row out
    want = _nbytes(idx, w, dest, iir, sc, *rows, np.empty((T, K), np.int32))
    assert B.bytes_dispatch_layout_chunked(T, K, P, C, N) == want


@pytest.mark.parametrize("C,S", [(1, 1), (4, 1), (4, 2), (5, 2), (3, 3), (7, 4)])
def test_chunk_streams_start_on_the_callers_stream(C, S):
    """The chunked dispatcher's stream schedule: the first chunk runs on the
    caller's stream (index 0) and neighbouring chunks alternate."""
    from types import SimpleNamespace
    import combine_ep_send_amd as ep
    idx = [ep.ChunkedDispatcher.chunk_stream_index(SimpleNamespace(C=C), i, S) for i in range(C)]
    assert idx[0] == 0
    assert all(0 <= v < S for v in idx)
    assert all(idx[i + 1] == (idx[i] + 1) % S for i in range(C - 1))
