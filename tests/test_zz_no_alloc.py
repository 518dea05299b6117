"""ep_dispatch_layout_noalloc, through the C ABI, against ep_dispatch_layout
with a workspace: the same outputs bit for bit, on calls in a row whose
inputs shrink and grow again (the library's scratch keeps its control words
from one call to the next)."""

import numpy as np
import pytest
import torch

from epgen import make_routing, spec
from tests.gpu_helpers import gpu_available, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

import combine_ep_send_amd as ep  # noqa: E402


def _outputs(T, K, P, E, cap):
    dev = "cuda"
    counts = ep.Counts(
        dest=torch.full((T, K), -7, dtype=torch.int32, device=dev),
        is_in_rank=torch.full((T, P), 7, dtype=torch.uint8, device=dev),
        send_counts=torch.full((1, P), -7, dtype=torch.int32, device=dev),
        tokens_per_expert=torch.full((1, E), -7, dtype=torch.int32, device=dev),
        diag=torch.full((1,), -7, dtype=torch.int32, device=dev))
    lay = ep.SendLayout(
        send_token_idx=torch.full((cap,), -7, dtype=torch.int32, device=dev),
        send_rank=torch.full((cap,), -7, dtype=torch.int32, device=dev),
        send_idx=torch.full((cap, K), -7, dtype=torch.int32, device=dev),
        send_w=torch.full((cap, K), -7.0, dtype=torch.float32, device=dev),
        token_row=torch.full((T, K), -7, dtype=torch.int32, device=dev))
    return counts, lay


def _same(a, b):
    for name in a._fields:
        x, y = getattr(a, name), getattr(b, name)
        if x is None:
            assert y is None, name
            continue
        assert torch.equal(x.view(torch.uint8) if x.dtype == torch.float32 else x,
                           y.view(torch.uint8) if y.dtype == torch.float32 else y), name


@pytest.mark.parametrize("shapes", [
    (("skewed_t16384", {}), ("uniform_t4096", {"T": 1000, "seed": 1}),
     ("skewed_t16384", {"seed": 2})),
])
def test_noalloc_layout_equals_the_workspace_call(shapes):
    for name, over in shapes:
        s = spec(name, **over)
        T, K, P, El, E = s.T, s.K, s.P, s.E_local, s.E
        print(f"case: noalloc layout {name} T={T} K={K} P={P} E={E} seed={s.seed}", flush=True)
        idx, w = make_routing(s)
        d_idx, d_w = to_dev(idx), to_dev(w)
        cap = T * min(K, P)
        ref_c, ref_l = _outputs(T, K, P, E, cap)
        ep.ep_dispatch_layout(d_idx, d_w, P, El, cap, counts=ref_c, out=ref_l)
        got_c, got_l = _outputs(T, K, P, E, cap)
        ep.ep_dispatch_layout_noalloc(d_idx, d_w, P, El, cap, counts=got_c, out=got_l)
        torch.cuda.synchronize()
        _same(ref_c, got_c)
        _same(ref_l, got_l)
        N = int(ref_c.send_counts.sum().item())
        assert N == int(((d_idx >= 0).view(T, K, 1) &
                         ((d_idx // El).view(T, K, 1) == torch.arange(P, device="cuda")))
                        .any(dim=1).sum().item())
        assert np.all(got_l.send_rank[:N].cpu().numpy() >= 0)
    assert ep.library_scratch_status() == 0
    ep.check_workspaces()
