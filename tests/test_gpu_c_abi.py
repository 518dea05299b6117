"""The C ABI on its own: tests/c/epdc_c_check.cpp drives counts + layout, the
bf16 and fp8 permutes and the weighted combine with nothing but the HIP runtime (no
PyTorch in that process), and its outputs match the CPU oracle bit for bit.
It also checks the ABI version, that an invalid call is refused, and that
the send path captured into a HIP graph replays to the eager results.
tests/c/epdc_c_paths.cpp does the same for the other calls: the two-call
layout, the chunked layout, both expert-batched layouts and the regroup."""

import os
import subprocess

import numpy as np
import pytest
import torch

import oracle as O
from epgen import make_hidden, make_routing, spec

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

CHECK = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "epdc_c_check")


def _write_case(path, idx, w, x, P, El):
    T, K = idx.shape
    with open(path, "wb") as f:
        f.write(np.int64([T, K, P, El, x.shape[1]]).tobytes())
        f.write(np.ascontiguousarray(idx, np.int64).tobytes())
        f.write(np.ascontiguousarray(w, np.float32).tobytes())
        f.write(np.ascontiguousarray(x, np.uint16).tobytes())


def _read_out(path, T, K, P, H):
    buf = open(path, "rb").read()
    off = 0

    def take(dtype, n):
        nonlocal off
        a = np.frombuffer(buf, dtype, n, off)
        off += a.nbytes
        return a

    N = int(take(np.int64, 1)[0])
    sc = take(np.int32, P)
    trow = take(np.int32, T * K).reshape(T, K)
    sti = take(np.int32, N)
    sx = take(np.uint16, N * H).reshape(N, H)
    out = take(np.uint16, T * H).reshape(T, H)
    q = take(np.uint8, N * H).reshape(N, H)
    qs = take(np.float32, N * (H // 128)).reshape(N, H // 128)
    assert off == len(buf)
    return sc, trow, sti, sx, out, q, qs


@pytest.mark.parametrize("name,T,H", [("tiny", 256, 512), ("skewed_t16384", 3000, 2048),
                                      ("uniform_t4096", 1537, 4096)])
def test_c_program_matches_oracle(tmp_path, name, T, H):
    if not os.path.exists(CHECK):
        pytest.fail(f"{CHECK} is not built (run __graft_entry__.build())")
    s = spec(name, T=T, H=H)
    idx, w = make_routing(s)
    x = make_hidden(s)
    case, out = tmp_path / "case.bin", tmp_path / "out.bin"
    _write_case(case, idx, w, x, s.P, s.E_local)
    print(f"case: C ABI {name} T={T} H={H} K={s.K} P={s.P}", flush=True)
    proc = subprocess.run([CHECK, str(case), str(out)], capture_output=True, text=True,
                          timeout=60, close_fds=True)
    assert proc.returncode == 0, (proc.returncode, proc.stderr)
    sc, trow, sti, sx, got, q, qs = _read_out(out, s.T, s.K, s.P, s.H)

    _, _, osc, _ = O.compute_send_counts(idx, s.P, s.E_local)
    osti, _, _, _, otrow = O.build_send_layout(idx, w, s.P, s.E_local)
    assert np.array_equal(sc, osc[0])
    assert np.array_equal(sti, osti)
    assert np.array_equal(trow, otrow)
    assert np.array_equal(sx, O.dispatch_permute(x, osti))
    assert np.array_equal(got, O.combine(O.dispatch_permute(x, osti), otrow, w))
    oq, oqs = O.dispatch_permute_fp8(x, osti)
    assert np.array_equal(q, oq)
    assert np.array_equal(qs.view(np.uint32), oqs.view(np.uint32))


PATHS = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "epdc_c_paths")


class _Reader:
    def __init__(self, path):
        self.buf = open(path, "rb").read()
        self.off = 0

    def take(self, dtype, n):
        a = np.frombuffer(self.buf, dtype, n, self.off)
        self.off += a.nbytes
        return a

    def done(self):
        return self.off == len(self.buf)


@pytest.mark.parametrize("name,T,H,C,align", [("skewed_t16384", 1500, 1024, 4, 16),
                                              ("uniform_t4096", 1001, 512, 3, 1)])
def test_c_program_other_paths_match_oracle(tmp_path, name, T, H, C, align):
    """tests/c/epdc_c_paths.cpp, with only the HIP runtime: the two-call send
    layout, every chunk's layout in one launch, both expert-batched layouts
    (bf16; fp8 with UE8M0 scales stored column-major) and the regroup of all
    destination segments by local expert, each against the CPU oracle."""
    if not os.path.exists(PATHS):
        pytest.fail(f"{PATHS} is not built (run __graft_entry__.build())")
    s = spec(name, T=T, H=H)
    idx, w = make_routing(s)
    x = make_hidden(s)
    K, P, El = s.K, s.P, s.E_local
    first, Eb, M = 2 * El, 2 * El, T           # two ranks' experts, batched
    case, out = tmp_path / "case.bin", tmp_path / "out.bin"
    with open(case, "wb") as f:
        f.write(np.int64([T, K, P, El, H, C, first, Eb, M, align]).tobytes())
        f.write(np.ascontiguousarray(idx, np.int64).tobytes())
        f.write(np.ascontiguousarray(w, np.float32).tobytes())
        f.write(np.ascontiguousarray(x, np.uint16).tobytes())
    print(f"case: C ABI other paths {name} T={T} H={H} K={K} P={P} C={C} align={align}",
          flush=True)
    proc = subprocess.run([PATHS, str(case), str(out)], capture_output=True, text=True,
                          timeout=60, close_fds=True)
    assert proc.returncode == 0, (proc.returncode, proc.stderr)
    r = _Reader(out)

    # two-call layout
    _, _, osc, otpe = O.compute_send_counts(idx, P, El)
    osti, osrk, osidx, osw, otrow = O.build_send_layout(idx, w, P, El)
    assert np.array_equal(r.take(np.int32, P), osc[0])
    assert np.array_equal(r.take(np.int32, P * El), otpe[0])
    N = int(r.take(np.int64, 1)[0])
    assert N == len(osti)
    assert np.array_equal(r.take(np.int32, N), osti)
    assert np.array_equal(r.take(np.int32, N), osrk)
    assert np.array_equal(r.take(np.int32, N * K).reshape(N, K), osidx)
    assert np.array_equal(r.take(np.uint32, N * K).reshape(N, K), osw.view(np.uint32))
    assert np.array_equal(r.take(np.int32, T * K).reshape(T, K), otrow)

    # every chunk's layout in one launch
    cap = int(r.take(np.int64, 1)[0])
    _, _, csc, _ = O.compute_send_counts(idx, P, El, C)
    assert np.array_equal(r.take(np.int32, C * P).reshape(C, P), csc)
    csti = r.take(np.int32, C * cap).reshape(C, cap)
    csrk = r.take(np.int32, C * cap).reshape(C, cap)
    csidx = r.take(np.int32, C * cap * K).reshape(C, cap, K)
    csw = r.take(np.uint32, C * cap * K).reshape(C, cap, K)
    ctrow = r.take(np.int32, T * K).reshape(T, K)
    for c, (a, b) in enumerate(O.chunk_bounds(T, C)):
        sti, srk, sidx, sw, trow = O.build_send_layout(idx[a:b], w[a:b], P, El)
        n = len(sti)
        assert np.array_equal(csti[c, :n], sti) and np.all(csti[c, n:] == -1)
        assert np.array_equal(csrk[c, :n], srk) and np.all(csrk[c, n:] == -1)
        assert np.array_equal(csidx[c, :n], sidx) and np.all(csidx[c, n:] == -1)
        assert np.array_equal(csw[c, :n], sw.view(np.uint32))
        assert np.all(csw[c, n:] == 0xFFFFFFFF)
        assert np.array_equal(ctrow[a:b], trow)

    # expert-batched layouts
    bx, btpe, btrow = O.batched_prepare(x, idx, first, Eb, M)
    assert np.array_equal(r.take(np.int32, Eb), btpe)
    assert np.array_equal(r.take(np.int32, T * K).reshape(T, K), btrow)
    assert np.array_equal(r.take(np.uint16, Eb * M * H).reshape(Eb, M, H), bx)
    bq, bs, qtpe, qtrow = O.batched_prepare_fp8(x, idx, first, Eb, M, "ue8m0")
    assert np.array_equal(r.take(np.int32, Eb), qtpe)
    assert np.array_equal(r.take(np.int32, T * K).reshape(T, K), qtrow)
    assert np.array_equal(r.take(np.uint8, Eb * M * H).reshape(Eb, M, H), bq)
    assert np.array_equal(r.take(np.int32, Eb * M * (H // 512)),
                          O.scale_storage(bs, True).astype(np.int32))

    # regroup of every destination segment by local expert
    ox, osrc, ow, ocnt, ooff, omap = O.regroup_by_expert(
        O.dispatch_permute(x, osti), osidx, osw, El, align, row_group=osrk, num_groups=P)
    R = int(r.take(np.int64, 1)[0])
    assert R == int(ooff[-1])
    assert np.array_equal(r.take(np.int32, P * El), ocnt)
    assert np.array_equal(r.take(np.int32, P * El + 1), ooff)
    assert np.array_equal(r.take(np.int32, R), osrc)
    assert np.array_equal(r.take(np.uint32, R), ow.view(np.uint32))
    assert np.array_equal(r.take(np.uint16, R * H).reshape(R, H), ox)
    assert np.array_equal(r.take(np.int32, N * K).reshape(N, K), omap)
    assert r.done()
