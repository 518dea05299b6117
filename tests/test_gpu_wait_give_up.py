"""A bounded wait that gives up is reported to the caller.

The one-launch layout's grid barrier waits for every workgroup's arrival; a
wait that outlasts its spin limit gives up, sets EP_WS_WAIT_GAVE_UP in the
workspace header and the call carries on.  Here the condition is forced from
the host, with no kernel changed: the count the next call starts from
(header word 2) is set 2^30 past the arrival count (word 0), so the target
the barrier waits for is never reached and every workgroup's wait runs to
its limit.  Every kernel still finishes; ep_workspace_status reports the
give-up once, and the binding raises WaitGaveUpError."""

import time

import numpy as np
import pytest
import torch

import oracle as O
from epgen import make_routing, spec
from tests.gpu_helpers import gpu_available, host, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

import combine_ep_send_amd as ep  # noqa: E402


def _poison_barrier(ws):
    hdr = ws[:16].view(torch.int32)
    arrivals = int(hdr[0].item())
    v = (arrivals + (1 << 30)) & 0xFFFFFFFF
    hdr[2] = v - (1 << 32) if v >= (1 << 31) else v
    torch.cuda.synchronize()


def test_fused_barrier_give_up_is_reported():
    s = spec("skewed_t16384", T=4096)
    T, K, P, El = s.T, s.K, s.P, s.E_local
    idx, w = make_routing(s)
    d_idx, d_w = to_dev(idx), to_dev(w)
    cap = T * min(K, P)
    ws = torch.zeros(ep.ep_dispatch_layout_workspace_bytes(T, P, El), dtype=torch.uint8,
                     device="cuda")
    c, lay = ep.ep_dispatch_layout(d_idx, d_w, P, El, cap, workspace=ws)
    assert ep.ep_workspace_status(ws) == 0

    _poison_barrier(ws)
    print(f"case: poisoned grid barrier, ep_dispatch_layout T={T} K={K} P={P}", flush=True)
    t0 = time.perf_counter()
    ep.ep_dispatch_layout(d_idx, d_w, P, El, cap, counts=c, out=lay, workspace=ws)
    torch.cuda.synchronize()                 # returns: every workgroup left its wait
    print(f"  the launch gave up and finished after {time.perf_counter() - t0:.3f} s",
          flush=True)
    with pytest.raises(ep.WaitGaveUpError):
        ep.check_workspaces(ws)
    assert ep.ep_workspace_status(ws) == 0   # the query cleared the word

    # a re-zeroed workspace serves again, and the outputs are the oracle's
    ws.zero_()
    c, lay = ep.ep_dispatch_layout(d_idx, d_w, P, El, cap, counts=c, out=lay, workspace=ws)
    torch.cuda.synchronize()
    assert ep.ep_workspace_status(ws) == 0
    sti, srk, sidx, sw, trow = O.build_send_layout(idx, w, P, El)
    N = len(sti)
    assert np.array_equal(host(lay.token_row), trow)
    assert np.array_equal(host(lay.send_token_idx)[:N], sti)
    assert np.array_equal(host(lay.send_idx)[:N], sidx)


def test_status_of_cached_workspaces_is_clean_after_normal_calls():
    s = spec("skewed_t16384", T=2048)
    idx, w = make_routing(s)
    d_idx, d_w = to_dev(idx), to_dev(w)
    cap = s.T * min(s.K, s.P)
    ep.ep_dispatch_layout(d_idx, d_w, s.P, s.E_local, cap)
    c = ep.ep_compute_send_counts(d_idx, s.P, s.E_local, 1)
    ep.ep_build_send_layout(d_idx, d_w, c.dest, c.send_counts[0], s.P, s.E_local, cap)
    ep.check_workspaces()                    # raises if any cached workspace has a flag
