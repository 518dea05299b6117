"""GPU parity of ep_regroup_by_expert (the receive side: rows regrouped by
local expert with alignment padding) against the CPU oracle, bit for bit,
and of its inverse through ep_combine."""

import numpy as np
import pytest
import torch

import oracle as O
from epgen import make_hidden, make_routing, spec
from tests.gpu_helpers import bits, gpu_available, host, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

import combine_ep_send_amd as ep  # noqa: E402


def _received(name, T, H, p=None, seed=0):
    """What destination p receives (its send segment), or with p=None the
    whole send buffer as one receiver with global expert ids."""
    s = spec(name, T=T, H=H, seed=seed)
    idx, w = make_routing(s)
    x = make_hidden(s)
    sti, srk, sidx, sw, trow = O.build_send_layout(idx, w, s.P, s.E_local)
    if p is None:
        gid = np.where(sidx >= 0, sidx + srk[:, None] * s.E_local, -1).astype(np.int32)
        return x[sti], gid, sw, s.E
    seg = srk == p
    return x[sti[seg]], sidx[seg].astype(np.int32), sw[seg], s.E_local


def _check(rx, ridx, rw, El, align, cap=None, workspace=None):
    R, K = ridx.shape
    H = rx.shape[1]
    ox, osrc, ow, ocnt, ooff, omap = O.regroup_by_expert(rx, ridx, rw, El, align)
    M = int(ooff[-1])
    if cap is None:
        cap = R * min(K, El) + El * (align - 1)
    out = ep.Regrouped(
        perm_x=torch.full((cap + 2, H), 0x1234, dtype=torch.int16, device="cuda")
        .view(torch.bfloat16),
        perm_src=torch.full((cap + 2,), -7, dtype=torch.int32, device="cuda"),
        perm_w=torch.full((cap + 2,), -7.0, dtype=torch.float32, device="cuda"),
        tokens_per_expert=torch.full((El,), -7, dtype=torch.int32, device="cuda"),
        expert_offsets=torch.full((El + 1,), -7, dtype=torch.int32, device="cuda"),
        row_map=torch.full((R, K), -7, dtype=torch.int32, device="cuda"))
    ep.ep_regroup_by_expert(to_dev(rx), to_dev(ridx), to_dev(rw), El, align, cap, out=out,
                            workspace=workspace)
    assert np.array_equal(host(out.tokens_per_expert), ocnt)
    assert np.array_equal(host(out.expert_offsets), ooff)
    n = min(M, cap)
    assert np.array_equal(host(out.row_map), np.where(omap < cap, omap, -1))
    assert np.array_equal(host(out.perm_src)[:n], osrc[:n])
    assert np.array_equal(host(out.perm_w)[:n].view(np.uint32), ow[:n].view(np.uint32))
    gx = bits(out.perm_x)
    assert np.array_equal(gx[:n], ox[:n])
    assert np.all(host(out.perm_src)[n:] == -7) and np.all(gx[n:] == 0x1234)   # untouched
    return out, (ox, osrc, ow, ocnt, ooff, omap)


@pytest.mark.parametrize("name,T,H,p,align", [
    ("skewed_t16384", 2000, 256, 0, 1),
    ("skewed_t16384", 2000, 256, 7, 16),
    ("uniform_t4096", 1500, 512, 3, 4),
    ("uniform_t4096", 1500, 512, 5, 128),
    ("tiny", 256, 512, 1, 8),
    ("fp8_t32768", 3000, 7168, 11, 32),
])
def test_regroup_segment_matches_oracle(name, T, H, p, align):
    print(f"case: {name} T={T} H={H} p={p} align={align}", flush=True)
    rx, ridx, rw, El = _received(name, T, H, p)
    out, ref = _check(rx, ridx, rw, El, align)
    # the inverse: an identity expert restored through row_map, weighted and not
    ox, osrc, ow, ocnt, ooff, omap = ref
    M = int(ooff[-1])
    back = bits(ep.restore_by_expert(out.perm_x[:M], out, to_dev(rw)))
    assert np.array_equal(back, O.combine(ox, omap, rw))
    back = bits(ep.restore_by_expert(out.perm_x[:M], out, None))
    assert np.array_equal(back, O.combine_partials(ox, omap))


def test_regroup_whole_send_buffer_by_global_expert():
    rx, gid, rw, E = _received("skewed_t16384", 4096, 128, None)
    _check(rx, gid, rw, E, 16)


def test_regroup_capacity_overflow_and_empty():
    rx, ridx, rw, El = _received("uniform_t4096", 1000, 64, 2)
    M = int(O.regroup_by_expert(rx, ridx, rw, El, 8)[4][-1])
    _check(rx, ridx, rw, El, 8, cap=M // 2)
    _check(rx, ridx, rw, El, 8, cap=M)
    # no rows at all: counts and offsets are zeros
    z = ep.ep_regroup_by_expert(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"),
                                torch.empty((0, 4), dtype=torch.int32, device="cuda"),
                                None, 8, 4)
    assert host(z.tokens_per_expert).tolist() == [0] * 8
    assert host(z.expert_offsets).tolist() == [0] * 9


def test_regroup_workspace_reused():
    ws = torch.zeros(ep.ep_regroup_workspace_bytes(20000, 256), dtype=torch.uint8, device="cuda")
    for i, (name, T, p, align) in enumerate([("skewed_t16384", 3000, 4, 8),
                                             ("uniform_t4096", 700, 1, 1),
                                             ("skewed_t16384", 5000, 0, 32)]):
        rx, ridx, rw, El = _received(name, T, 64, p, seed=i)
        _check(rx, ridx, rw, El, align, workspace=ws)
    hdr = ws[:16].view(torch.int32).cpu().numpy()
    assert hdr[3] == 0 and hdr[0] > 0 and hdr[0] == hdr[2]   # no time-out; count handed on


@pytest.mark.parametrize("name,T,H,align", [("skewed_t16384", 3000, 256, 16),
                                            ("uniform_t4096", 2000, 512, 128)])
def test_regroup_all_destination_segments_at_once(name, T, H, align):
    """row_group = send_rank: every destination's received rows regrouped in
    one call, against the oracle's regroup with the same groups."""
    s = spec(name, T=T, H=H)
    idx, w = make_routing(s)
    x = make_hidden(s)
    sti, srk, sidx, sw, trow = O.build_send_layout(idx, w, s.P, s.E_local)
    rx, ridx = x[sti], sidx.astype(np.int32)
    ox, osrc, ow, ocnt, ooff, omap = O.regroup_by_expert(rx, ridx, sw, s.E_local, align,
                                                         row_group=srk, num_groups=s.P)
    out = ep.ep_regroup_by_expert(to_dev(rx), to_dev(ridx), to_dev(sw), s.E_local, align,
                                  row_group=to_dev(srk.astype(np.int32)), num_groups=s.P)
    M = int(ooff[-1])
    assert np.array_equal(host(out.tokens_per_expert), ocnt)
    assert np.array_equal(host(out.expert_offsets), ooff)
    assert np.array_equal(host(out.row_map), omap)
    assert np.array_equal(host(out.perm_src)[:M], osrc)
    assert np.array_equal(host(out.perm_w)[:M].view(np.uint32), ow.view(np.uint32))
    assert np.array_equal(bits(out.perm_x)[:M], ox)


def test_regroup_expert_major_workload_full_size():
    """The expert-major workload as the bench times it (T=16384, every
    destination segment of the send buffer regrouped in one call, align
    128), compared element by element with the oracle.  The one call is the
    regroups of the P segments one after the other (bins are (segment,
    expert), segment-major), so the oracle regroups each segment on its own
    and the GPU's result is checked piece by piece: rows, sources (offset by
    the segment's first row), weights, counts, offsets and row_map."""
    s = spec("expert_major_t16384")
    print(f"case: full-size expert_major_t16384 T={s.T} H={s.H} P={s.P} align={s.align}",
          flush=True)
    idx, w = make_routing(s)
    x = make_hidden(s)
    P, El, A, T, K, H = s.P, s.E_local, s.align, s.T, s.K, s.H
    c, lay = ep.ep_dispatch_layout(to_dev(idx), to_dev(w), P, El, T * min(K, P))
    N = int(host(c.send_counts).sum())
    send_x = ep.ep_dispatch_permute(to_dev(x), lay.token_row, T * min(K, P))
    B = P * El
    out = ep.ep_regroup_by_expert(send_x[:N], lay.send_idx[:N], lay.send_w[:N], El, A,
                                  T * K + B * (A - 1), row_group=lay.send_rank[:N],
                                  num_groups=P)
    torch.cuda.synchronize()
    ep.check_workspaces()
    del send_x
    sti, srk, sidx, sw, trow = O.build_send_layout(idx, w, P, El)
    assert len(sti) == N
    assert np.array_equal(host(lay.send_idx)[:N], sidx)
    cnt, off = host(out.tokens_per_expert), host(out.expert_offsets)
    src, pw, rmap = host(out.perm_src), host(out.perm_w), host(out.row_map)
    M = int(off[-1])
    px = bits(out.perm_x[:M])
    del out
    seg = np.concatenate([[0], np.cumsum(np.bincount(srk, minlength=P))])
    for p in range(P):
        r0, r1 = int(seg[p]), int(seg[p + 1])
        ox = O.dispatch_permute(x, sti[r0:r1])
        opx, osrc, ow, ocnt, ooff, ormap = O.regroup_by_expert(ox, sidx[r0:r1], sw[r0:r1], El, A)
        base = int(off[p * El])
        m = int(ooff[-1])
        assert np.array_equal(cnt[p * El:(p + 1) * El], ocnt), p
        assert np.array_equal(off[p * El:(p + 1) * El + 1] - base, ooff), p
        assert np.array_equal(src[base:base + m], np.where(osrc >= 0, osrc + r0, -1)), p
        assert np.array_equal(pw[base:base + m].view(np.uint32), ow.view(np.uint32)), p
        assert np.array_equal(rmap[r0:r1], np.where(ormap >= 0, ormap + base, -1)), p
        assert np.array_equal(px[base:base + m], opx), p
    print(f"  N={N} rows regrouped into M={M} rows, every one compared", flush=True)
