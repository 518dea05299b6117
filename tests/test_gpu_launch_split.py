"""Grids past the launch limit.  A launch spans at most 2^32-1 work-items per
grid dimension, so a row kernel over more workgroups than that splits into
several launches, each told its first item.  Narrow rows make such token
counts cheap: 34 million tokens of 8 channels need 34 million 128-thread
workgroups in the bf16 permute (two launches), 68 million need more than
one launch of the 64-thread fp8 permute, dense combine and sparse combine,
and the expert-batched fills run just under and just past the limit.  The full outputs are checked by properties that hold at any size
(with one slot per token the permute is a scatter by a permutation and the
unweighted combine its gather; the batched routing has closed-form counts
and slots), and sampled tokens on both sides of each split point against
the CPU oracle."""

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
    """Sorted ids in [0, T): both ends, both sides of the split and random
    ones."""
    r = np.random.default_rng(seed)
    edge = [0, 1, split - 2, split - 1, split, split + 1, T - 2, T - 1]
    ids = np.unique(np.concatenate([edge, r.integers(0, T, n)])).astype(np.int64)
    ids = ids[(ids >= 0) & (ids < T)]
    assert len(ids) and ids[0] >= 0 and ids[-1] < T
    return ids


def _inputs(T, H, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randn((T, H), dtype=torch.bfloat16, device="cuda", generator=g)
    perm = torch.randperm(T, device="cuda", generator=g).to(torch.int32)
    return x, perm


def test_bf16_permute_split_launches_and_combine():
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


def test_sparse_combine_split_launches():
    T, H = 68_000_000, 8
    split = LIMIT // 64                   # 8 channels: one 64-thread workgroup per token
    assert T > split
    print(f"case: sparse combine, T={T} H={H}", flush=True)
    y, perm = _inputs(T, H, 14)
    token_row = perm.view(T, 1)           # R = T rows: the sparse form
    out = ep.ep_combine(y, token_row, None)
    # torch's one-call gather y[perm] is not exact at this size (it differed
    # in 2^26 rows here), so the reference is gathered 8M rows at a time
    for a in range(0, T, 8_000_000):
        b = min(T, a + 8_000_000)
        assert torch.equal(out[a:b], y[perm[a:b].long()]), (a, b)
    toks = _samples(T, split)
    rows = host(perm)[toks]
    ys = _bits(y[torch.from_numpy(rows.astype(np.int64)).cuda()])
    loc = np.arange(len(toks), dtype=np.int32).reshape(-1, 1)
    assert np.array_equal(_bits(out[torch.from_numpy(toks).cuda()]), O.combine_partials(ys, loc))


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


def _batched_expect(T, El, M):
    """Routing of the batched launch cases: token t names expert t % (El+1),
    so expert e < El takes tokens e, e+El+1, ... in order and the last id is
    not local; counts, slot and token_row follow in closed form."""
    t = torch.arange(T, device="cuda", dtype=torch.int64)
    idx = (t % (El + 1)).view(T, 1)
    cnt = [(T - e + El) // (El + 1) for e in range(El)]
    e_of = idx[:, 0]
    trow = torch.where(e_of < El, e_of * M + t // (El + 1), -1).to(torch.int32).view(T, 1)
    return idx, cnt, trow


@pytest.mark.parametrize("T", [33_500_000, 34_000_000])
def test_batched_bf16_one_launch_and_split(T):
    """The expert-batched fill over one-piece rows: 33.5M tokens fit one
    launch of the sparse permute, just under the limit; 34M need two."""
    H, El = 8, 2
    M = T
    print(f"case: batched bf16, T={T} H={H} E_local={El} max={M}", flush=True)
    x, _ = _inputs(T, H, 14)
    idx, cnt, trow = _batched_expect(T, El, M)
    b_x = torch.empty((El, M, H), dtype=torch.bfloat16, device="cuda")
    b_x.view(torch.int16).fill_(-1)
    b, tpe, tr = ep.ep_batched_prepare(x, idx, 0, El, M, out=b_x)
    assert host(tpe).tolist() == cnt
    assert torch.equal(tr, trow)
    for e in range(El):
        assert torch.equal(b[e, :cnt[e]], x[e::El + 1])
        assert int(torch.count_nonzero(b[e, cnt[e]:].view(torch.int16))) == 0


@pytest.mark.parametrize("T", [66_000_000, 68_000_000])
def test_batched_fp8_one_launch_and_split(T):
    """As above for the fp8 layout (one-wave fill items): 66M tokens in one
    launch, 68M in two; sampled rows against the oracle, every data row
    written, every padding code and scale zero."""
    H, El = 128, 2
    M = T
    print(f"case: batched fp8, T={T} H={H} E_local={El} max={M}", flush=True)
    x, _ = _inputs(T, H, 15)
    idx, cnt, trow = _batched_expect(T, El, M)
    q = torch.full((El, M, H), 0xFF, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
    sc = ep.batched_scale_like(El, M, H, "f32", False, "cuda")
    sc.fill_(float("nan"))
    bq, bs, tpe, tr = ep.ep_batched_prepare_fp8(x, idx, 0, El, M, scale_fmt="f32", out=q,
                                                out_scale=sc)
    assert host(tpe).tolist() == cnt
    assert torch.equal(tr, trow)
    for e in range(El):
        assert not bool((bq[e, :cnt[e]].view(torch.uint8) == 0xFF).any())
        assert not bool(torch.isnan(bs[e, :cnt[e]]).any())
        assert int(torch.count_nonzero(bq[e, cnt[e]:].view(torch.uint8))) == 0
        assert int(torch.count_nonzero(bs[e, cnt[e]:])) == 0
    split_tok = min(T, LIMIT // 64)       # first token of a second fp8 permute launch
    for e in range(El):
        slots = _samples(cnt[e], (split_tok - e) // (El + 1), n=48, seed=e)
        assert slots[-1] < cnt[e] and slots[-1] * (El + 1) + e < T   # in bounds of x and b_q
        toks = torch.from_numpy(slots * (El + 1) + e).cuda()
        oq, osc = O.quantize_rows_fp8(_bits(x[toks]), "f32")
        sl = torch.from_numpy(slots).cuda()
        assert np.array_equal(bq[e][sl].view(torch.uint8).cpu().numpy(), oq)
        assert np.array_equal(bs[e][sl].cpu().numpy().view(np.uint32), osc.view(np.uint32))
