"""Grids past the launch limit.  A launch spans at most 2^32-1 work-items per
grid dimension, so a row kernel over more workgroups than that splits into
several launches, each told its first item.  Narrow rows make such token
counts cheap: 34 million tokens of 8 channels need 34 million 128-thread
workgroups in the bf16 permute and the sparse combine (two launches each),
68 million need more than one launch of the 64-thread fp8 permute and dense
combine.  The full outputs are checked by properties that hold at any size
(with one slot per token the permute is a scatter by a permutation and the
unweighted combine its gather), and sampled tokens on both sides of each
split point against the CPU oracle."""

import numpy as np
import pytest
import torch

import oracle as O
from tests.gpu_helpers import host

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

import combine_ep_send_amd as ep  # noqa: E402

LIMIT = 2 ** 32 - 1                      # work-items per grid dimension


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _samples(T, split, n=96, seed=0):
    """Sorted token ids: both ends, both sides of the split and random ones."""
    r = np.random.default_rng(seed)
    edge = [0, 1, split - 2, split - 1, split, split + 1, T - 2, T - 1]
    return np.unique(np.concatenate([edge, r.integers(0, T, n)])).astype(np.int64)


def _inputs(T, H, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randn((T, H), dtype=torch.bfloat16, device="cuda", generator=g)
    perm = torch.randperm(T, device="cuda", generator=g).to(torch.int32)
    return x, perm


def test_bf16_permute_and_sparse_combine_split_launches():
    T, H = 34_000_000, 8
    split = LIMIT // 128                  # 128-thread workgroups, one per token
    assert T > split
    print(f"case: bf16 permute + sparse combine, T={T} H={H}", flush=True)
    x, perm = _inputs(T, H, 11)
    token_row = perm.view(T, 1)
    send_x = ep.ep_dispatch_permute(x, token_row, T)
    # row perm[t] holds token t, every row written once
    assert torch.equal(send_x[perm.long()], x)
    # the unweighted combine gathers each token's row back (R = T: sparse form)
    out = ep.ep_combine(send_x, token_row, None)
    assert torch.equal(out, x)
    ones = torch.ones((T, 1), dtype=torch.float32, device="cuda")
    assert torch.equal(ep.ep_combine(send_x, token_row, ones), x)
    toks = _samples(T, split)
    xs = _bits(x[torch.from_numpy(toks).cuda()])
    rows = torch.from_numpy(host(perm)[toks].astype(np.int64)).cuda()
    assert np.array_equal(_bits(send_x[rows]), O.dispatch_permute(xs, np.arange(len(toks))))
    loc = np.arange(len(toks), dtype=np.int32).reshape(-1, 1)
    assert np.array_equal(_bits(out[torch.from_numpy(toks).cuda()]), O.combine_partials(xs, loc))


def test_fp8_permute_split_launches():
    T, H = 68_000_000, 128
    split = LIMIT // 64                   # one-wave workgroups, one per token
    assert T > split
    print(f"case: fp8 permute, T={T} H={H}", flush=True)
    x, perm = _inputs(T, H, 12)
    token_row = perm.view(T, 1)
    # sentinels no written row can hold: 0xFF is an e4m3 NaN (codes saturate
    # to +-448) and a scale is never NaN
    q = torch.full((T, H), 0xFF, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
    sc = torch.full((T, 1), float("nan"), dtype=torch.float32, device="cuda")
    ep.ep_dispatch_permute(x, token_row, T, fp8=True, out=q, out_scale=sc)
    assert not bool((q.view(torch.uint8) == 0xFF).any())
    assert not bool(torch.isnan(sc).any())
    toks = _samples(T, split)
    xs = _bits(x[torch.from_numpy(toks).cuda()])
    oq, osc = O.dispatch_permute_fp8(xs, np.arange(len(toks)))
    rows = torch.from_numpy(host(perm)[toks].astype(np.int64)).cuda()
    assert np.array_equal(q[rows].view(torch.uint8).cpu().numpy(), oq)
    assert np.array_equal(sc[rows].cpu().numpy().view(np.uint32), osc.view(np.uint32))


def test_dense_combine_split_launches():
    T, H = 68_000_000, 8
    split = LIMIT // 64                   # 8 channels: one 64-thread workgroup per token
    assert T > split
    print(f"case: dense combine, T={T} H={H}", flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(13)
    y = torch.randn((2 * T, H), dtype=torch.bfloat16, device="cuda", generator=g)  # R = 2T: dense form
    token_row = torch.randint(0, 2 * T, (T, 2), device="cuda", generator=g, dtype=torch.int64)
    token_row = token_row.to(torch.int32)
    token_row[::7, 1] = -1                # some tokens with one slot
    w = torch.rand((T, 2), device="cuda", generator=g) + 0.25   # no zero weights, so no -0.0 products
    out = ep.ep_combine(y, token_row, w)
    toks = _samples(T, split)
    tr = host(token_row)[toks]
    used = np.unique(tr[tr >= 0])
    ys = _bits(y[torch.from_numpy(used.astype(np.int64)).cuda()])
    loc = np.where(tr >= 0, np.searchsorted(used, tr), -1).astype(np.int32)
    ws = host(w)[toks]
    assert np.array_equal(_bits(out[torch.from_numpy(toks).cuda()]), O.combine(ys, loc, ws))
    # the whole output against the same sums in torch (fp32 products, then adds)
    yf = y.float()
    r0, r1 = token_row[:, 0].long(), token_row[:, 1].long()
    acc = w[:, :1] * yf[r0]
    acc = acc + torch.where((r1 >= 0)[:, None], w[:, 1:] * yf[r1.clamp(min=0)], 0.0)
    assert torch.equal(out, acc.to(torch.bfloat16))
