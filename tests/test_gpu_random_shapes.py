"""GPU parity against the CPU oracle on seeded random shapes: the whole send
path (counts + layout in one launch, the permute in bf16 and fp8, the
weighted and unweighted combine), the expert-batched layouts (bf16 and fp8),
and the regroup by expert, each over shapes drawn from a fixed seed (T, K,
E, P, H, routing, unrouted fraction, alignment), bit for bit."""

import numpy as np
import pytest
import torch

import oracle as O
from epgen import make_hidden, make_routing, spec
from tests.gpu_helpers import bits, host, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

import combine_ep_send_amd as ep  # noqa: E402


def _shape(seed):
    """A random but valid configuration: P divides E, K <= E, H a multiple of
    128 (512 when UE8M0 scales are drawn)."""
    r = np.random.default_rng(1000 + seed)
    P = int(r.choice([1, 2, 3, 4, 8, 16, 32, 64]))
    El = int(r.choice([1, 2, 3, 4, 8]))
    E = P * El
    K = int(r.integers(1, min(E, 16) + 1))
    T = int(r.choice([1, 7, 63, 64, 65, 255, 256, 257, 1000, 3000, 5000, 9000]))
    H = int(r.choice([512, 1024, 1536, 2048, 3584]))
    routing = "zipf" if r.random() < 0.5 else "uniform"
    unrouted = float(r.choice([0.0, 0.0, 0.05, 0.3]))
    s = spec("tiny").replace(name="rand", T=T, H=H, E=E, K=K, P=P, routing=routing,
                             unrouted_frac=unrouted, seed=seed)
    return s, r


SEEDS = list(range(12))


@pytest.mark.parametrize("seed", SEEDS)
def test_send_path_random_shape(seed):
    s, r = _shape(seed)
    print(f"case: seed={seed} T={s.T} K={s.K} E={s.E} P={s.P} H={s.H} {s.routing} "
          f"unrouted={s.unrouted_frac}", flush=True)
    idx, w = make_routing(s)
    x = make_hidden(s)
    T, K, P, El, H = s.T, s.K, s.P, s.E_local, s.H
    cap = T * min(K, P)
    d_idx, d_w, d_x = to_dev(idx), to_dev(w), to_dev(x)
    c, lay = ep.ep_dispatch_layout(d_idx, d_w, P, El, cap)
    dest, iir, sc, tpe = O.compute_send_counts(idx, P, El, 1)
    assert np.array_equal(host(c.dest), dest)
    assert np.array_equal(host(c.is_in_rank), iir)
    assert np.array_equal(host(c.send_counts), sc)
    assert np.array_equal(host(c.tokens_per_expert), tpe)
    sti, srk, sidx, sw, trow = O.build_send_layout(idx, w, P, El)
    N = len(sti)
    assert np.array_equal(host(lay.send_token_idx)[:N], sti)
    assert np.array_equal(host(lay.send_rank)[:N], srk)
    assert np.array_equal(host(lay.send_idx)[:N], sidx)
    assert np.array_equal(host(lay.send_w)[:N].view(np.uint32), sw.view(np.uint32))
    assert np.array_equal(host(lay.token_row), trow)
    send_x = ep.ep_dispatch_permute(d_x, lay.token_row, cap)
    y = bits(send_x)[:N]
    assert np.array_equal(y, O.dispatch_permute(x, sti))
    q, scl = ep.ep_dispatch_permute(d_x, lay.token_row, cap, fp8=True)
    oq, osc = O.dispatch_permute_fp8(x, sti)
    assert np.array_equal(host(q)[:N], oq)
    assert np.array_equal(host(scl)[:N].view(np.uint32), osc.view(np.uint32))
    # combine of the permuted rows, weighted and as partial sums
    assert np.array_equal(bits(ep.ep_combine(send_x, lay.token_row, d_w)),
                          O.combine(y, trow, w))
    assert np.array_equal(bits(ep.ep_combine(send_x, lay.token_row, None)),
                          O.combine_partials(y, trow))


@pytest.mark.parametrize("seed", SEEDS)
def test_batched_and_regroup_random_shape(seed):
    s, r = _shape(seed)
    idx, w = make_routing(s)
    x = make_hidden(s)
    T, K, P, El, H = s.T, s.K, s.P, s.E_local, s.H
    rank = int(r.integers(0, P))
    first = rank * El
    M = int(r.choice([1, 16, max(1, T // 4), T + 3]))
    print(f"case: seed={seed} T={T} K={K} E={s.E} P={P} H={H} rank={rank} max={M}", flush=True)
    d_idx, d_x = to_dev(idx), to_dev(x)
    # bf16 batched layout; the oracle raises past max, so compare against a large max
    b_x, tpe, trow = ep.ep_batched_prepare(d_x, d_idx, first, El, M)
    Mb = max(M, T)
    ob, otpe, otrow = O.batched_prepare(x, idx, first, El, Mb)
    assert np.array_equal(host(tpe), otpe)
    e_of, slot = otrow // Mb, otrow % Mb
    assert np.array_equal(host(trow), np.where((otrow >= 0) & (slot < M), e_of * M + slot, -1))
    assert np.array_equal(bits(b_x), ob[:, :M])
    # fp8 batched layout, a random scale format and storage order
    fmt = str(r.choice(["f32", "pow2"] + (["ue8m0"] if H % 512 == 0 else [])))
    col = bool(r.random() < 0.5)
    bq, bs, _, _ = ep.ep_batched_prepare_fp8(d_x, d_idx, first, El, M, scale_fmt=fmt,
                                             scale_col_major=col)
    oq, osc, _, _ = O.batched_prepare_fp8(x, idx, first, El, Mb, fmt)
    assert np.array_equal(host(bq), oq[:, :M])
    flat = torch.as_strided(bs, (bs.numel(),), (1,)).cpu().numpy().view(np.uint32)
    assert np.array_equal(flat, O.scale_storage(osc[:, :M], col).view(np.uint32))
    # regroup of the whole send buffer by destination segment, random alignment
    sti, srk, sidx, sw, _ = O.build_send_layout(idx, w, P, El)
    if len(sti) == 0:
        return
    A = int(r.choice([1, 2, 8, 128]))
    rx = x[sti]
    ox, osrc, ow, ocnt, ooff, omap = O.regroup_by_expert(rx, sidx.astype(np.int32), sw, El, A,
                                                         row_group=srk, num_groups=P)
    out = ep.ep_regroup_by_expert(to_dev(rx), to_dev(sidx.astype(np.int32)), to_dev(sw), El, A,
                                  row_group=to_dev(srk.astype(np.int32)), num_groups=P)
    Mr = int(ooff[-1])
    assert np.array_equal(host(out.tokens_per_expert), ocnt)
    assert np.array_equal(host(out.expert_offsets), ooff)
    assert np.array_equal(host(out.row_map), omap)
    assert np.array_equal(host(out.perm_src)[:Mr], osrc)
    assert np.array_equal(host(out.perm_w)[:Mr].view(np.uint32), ow.view(np.uint32))
    assert np.array_equal(bits(out.perm_x)[:Mr], ox)
