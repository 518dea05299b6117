"""The C ABI on its own: tests/c/epdc_c_check.cpp drives counts + layout, the
bf16 and fp8 permutes and the weighted combine with nothing but the HIP runtime (no
PyTorch in that process), and its outputs match the CPU oracle bit for bit.
It also checks the ABI version, that an invalid call is refused, and that
the send path captured into a HIP graph replays to the eager results."""

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
