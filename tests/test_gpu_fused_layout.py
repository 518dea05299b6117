"""GPU parity of ep_dispatch_layout (counts + send layout in one launch)
against the CPU oracle, bit for bit, on the same seeded inputs as the
two-call path; plus the cases the one-launch design adds: several tiles per
workgroup, capacity overflow, bad ids, and a workspace reused across calls of
different sizes (its barrier generation must rearm)."""

import numpy as np
import pytest
import torch

import oracle as O
from epgen import make_routing, spec
from tests.gpu_helpers import gpu_available, host, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

import combine_ep_send_amd as ep  # noqa: E402


def _case(T, E, K, P, routing="uniform", unrouted=0.0, seed=0):
    s = spec("tiny").replace(name="case", T=T, E=E, K=K, P=P, routing=routing,
                             unrouted_frac=unrouted, seed=seed)
    return make_routing(s)


def _fused(idx, w, P, El, cap, workspace=None):
    """Run the fused call with sentinel-filled outputs (so untouched rows can
    be checked) and return host copies of everything."""
    T, K = idx.shape
    E = P * El
    dev = "cuda"
    counts = ep.Counts(
        dest=torch.full((T, K), -9, dtype=torch.int32, device=dev),
        is_in_rank=torch.full((T, P), 9, dtype=torch.uint8, device=dev),
        send_counts=torch.full((1, P), -9, dtype=torch.int32, device=dev),
        tokens_per_expert=torch.full((1, E), -9, dtype=torch.int32, device=dev),
        diag=torch.full((1,), -9, dtype=torch.int32, device=dev))
    lay = ep.SendLayout(
        send_token_idx=torch.full((cap + 3,), -7, dtype=torch.int32, device=dev),
        send_rank=torch.full((cap + 3,), -7, dtype=torch.int32, device=dev),
        send_idx=torch.full((cap + 3, K), -7, dtype=torch.int32, device=dev),
        send_w=torch.full((cap + 3, K), -7.0, dtype=torch.float32, device=dev),
        token_row=torch.full((T, K), -7, dtype=torch.int32, device=dev))
    ep.ep_dispatch_layout(to_dev(idx), to_dev(w), P, El, cap, counts=counts, out=lay,
                          workspace=workspace)
    c = {k: host(v) for k, v in counts._asdict().items()}
    l_ = {k: host(v) for k, v in lay._asdict().items()}
    return c, l_


def check_fused(idx, w, P, El, cap=None, workspace=None):
    T, K = idx.shape
    if cap is None:
        cap = T * min(K, P)
    c, lay = _fused(idx, w, P, El, cap, workspace)
    dest, iir, sc, tpe = O.compute_send_counts(idx, P, El, 1)
    assert np.array_equal(c["dest"], dest)
    assert np.array_equal(c["is_in_rank"], iir)
    assert np.array_equal(c["send_counts"], sc)
    assert np.array_equal(c["tokens_per_expert"], tpe)
    assert c["diag"][0] == 0
    sti, srk, sidx, sw, trow = O.build_send_layout(idx, w, P, El)
    N = len(sti)
    n = min(N, cap)
    assert np.array_equal(lay["send_token_idx"][:n], sti[:n])
    assert np.array_equal(lay["send_rank"][:n], srk[:n])
    assert np.array_equal(lay["send_idx"][:n], sidx[:n])
    assert np.array_equal(lay["send_w"][:n].view(np.uint32), sw[:n].view(np.uint32))
    assert np.array_equal(lay["token_row"], np.where(trow < cap, trow, -1))
    assert np.all(lay["send_token_idx"][n:] == -7)          # rows past N / cap untouched
    assert np.all(lay["send_idx"][n:] == -7)
    return N


@pytest.mark.parametrize("T,E,K,P,routing,unrouted", [
    (256, 8, 2, 2, "uniform", 0.0),           # the tiny workload's routing
    (1000, 64, 6, 8, "uniform", 0.0),         # K = 6, ragged last tile
    (1537, 256, 8, 32, "zipf", 0.05),         # skewed, unrouted slots
    (16384, 256, 8, 32, "zipf", 0.05),        # the skewed 16k workload's shape
    (300, 16, 16, 4, "uniform", 0.1),         # K = 16
    (513, 4, 1, 4, "uniform", 0.0),           # K = 1
    (400, 96, 3, 1, "uniform", 0.0),          # one destination
    (700, 30, 5, 6, "uniform", 0.0),          # P not a multiple of 4
    (1, 8, 2, 2, "uniform", 0.0),             # a single token
    (76800, 16, 2, 4, "uniform", 0.0),        # 300 tiles: two tiles per workgroup
    (20000, 256, 8, 64, "zipf", 0.05),        # 79 groups x 64 bins: the two-pass scan
    (8192, 256, 8, 256, "uniform", 0.0),      # 32 groups x 256 bins: 8 bins per group
    (3000, 1024, 4, 512, "uniform", 0.0),     # 12 groups x 512 bins: single pass, many loads
])
def test_fused_layout_matches_oracle(T, E, K, P, routing, unrouted):
    print(f"case: T={T} E={E} K={K} P={P} {routing}", flush=True)
    idx, w = _case(T, E, K, P, routing, unrouted)
    check_fused(idx, w, P, E // P)


@pytest.mark.parametrize("K,P,words", [(6, 8, 1), (6, 16, 2), (8, 32, 1), (8, 32, 2), (2, 2, 1),
                                         (4, 16, 3)])
def test_fused_layout_unaligned_rows(K, P, words):
    """Arrays that start a few words past 16-byte alignment (views into
    larger buffers) take the narrower whole-row accesses, or one word per
    slot, and give the same results."""
    T, El = 777, 4
    idx, w = _case(T, P * El, K, P, seed=5)
    cap = T * min(K, P)
    print(f"case: unaligned K={K} P={P} offset={words} words", flush=True)

    def at(shape, dtype, fill, k):
        n = int(np.prod(shape))
        return torch.full((n + k,), fill, dtype=dtype, device="cuda")[k:].view(shape)

    d_idx = at((T, K), torch.int64, 0, 1)                # 8 bytes off
    d_idx.copy_(to_dev(idx))
    d_w = at((T, K), torch.float32, 0.0, words)
    d_w.copy_(to_dev(w))
    counts = ep.Counts(dest=at((T, K), torch.int32, -9, words),
                       is_in_rank=at((T, P), torch.uint8, 9, 4 * words),
                       send_counts=at((1, P), torch.int32, -9, words),
                       tokens_per_expert=at((1, P * El), torch.int32, -9, words),
                       diag=at((1,), torch.int32, -9, words))
    lay = ep.SendLayout(send_token_idx=at((cap,), torch.int32, -7, words),
                        send_rank=at((cap,), torch.int32, -7, words),
                        send_idx=at((cap, K), torch.int32, -7, words),
                        send_w=at((cap, K), torch.float32, -7.0, words),
                        token_row=at((T, K), torch.int32, -7, words))
    ep.ep_dispatch_layout(d_idx, d_w, P, El, cap, counts=counts, out=lay)
    dest, iir, sc, tpe = O.compute_send_counts(idx, P, El, 1)
    assert np.array_equal(host(counts.dest), dest)
    assert np.array_equal(host(counts.is_in_rank), iir)
    assert np.array_equal(host(counts.send_counts), sc)
    assert np.array_equal(host(counts.tokens_per_expert), tpe)
    sti, srk, sidx, sw, trow = O.build_send_layout(idx, w, P, El)
    N = len(sti)
    assert np.array_equal(host(lay.send_token_idx)[:N], sti)
    assert np.array_equal(host(lay.send_rank)[:N], srk)
    assert np.array_equal(host(lay.send_idx)[:N], sidx)
    assert np.array_equal(host(lay.send_w)[:N].view(np.uint32), sw.view(np.uint32))
    assert np.array_equal(host(lay.token_row), trow)
    assert np.all(host(lay.send_idx)[N:] == -7)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_fused_layout_other_seeds(seed):
    idx, w = _case(4000, 256, 8, 32, "zipf", 0.05, seed=seed)
    check_fused(idx, w, 32, 8)


def test_fused_equals_two_calls_at_full_size():
    """The 16k skewed workload: fused and two-call paths agree bit for bit."""
    s = spec("skewed_t16384")
    idx, w = make_routing(s)
    d_idx, d_w = to_dev(idx), to_dev(w)
    cap = s.T * 8
    c2 = ep.ep_compute_send_counts(d_idx, s.P, s.E_local, 1)
    l2 = ep.ep_build_send_layout(d_idx, d_w, c2.dest, c2.send_counts[0], s.P, s.E_local, cap)
    c1, l1 = ep.ep_dispatch_layout(d_idx, d_w, s.P, s.E_local, cap)
    N = int(host(c2.send_counts).sum())
    for a, b in zip(c1, c2):
        assert torch.equal(a, b)
    for name in ("send_token_idx", "send_rank", "send_idx", "send_w"):
        assert torch.equal(getattr(l1, name)[:N], getattr(l2, name)[:N]), name
    assert torch.equal(l1.token_row, l2.token_row)


def test_fused_capacity_overflow():
    idx, w = _case(500, 64, 6, 8)
    N = int(O.compute_send_counts(idx, 8, 8)[1].sum())
    check_fused(idx, w, 8, 8, cap=N // 2)
    check_fused(idx, w, 8, 8, cap=N)            # exact capacity
    check_fused(idx, w, 8, 8, cap=0)            # nothing fits


def test_fused_bad_ids_and_empty():
    idx, w = _case(400, 32, 4, 4)
    bad = idx.copy()
    bad[5, 1] = 32
    bad[9, 0] = -5
    bad[77, 3] = 1 << 40
    c, lay = _fused(bad, w, 4, 8, 400 * 4)
    assert c["diag"][0] == 3
    clean = bad.copy()
    clean[(clean < -1) | (clean >= 32)] = -1
    dest, iir, sc, tpe = O.compute_send_counts(clean, 4, 8)
    assert np.array_equal(c["dest"], dest)
    assert np.array_equal(c["send_counts"], sc)
    assert np.array_equal(c["tokens_per_expert"], tpe)
    sti, _, _, _, trow = O.build_send_layout(clean, w, 4, 8)
    assert np.array_equal(lay["token_row"], trow)
    assert np.array_equal(lay["send_token_idx"][:len(sti)], sti)
    # every slot unrouted
    none = np.full((130, 4), -1, dtype=np.int64)
    check_fused(none, np.zeros((130, 4), np.float32), 4, 8)
    # T = 0: counts are still written (zeros)
    c, lay = _fused(np.zeros((0, 4), np.int64), np.zeros((0, 4), np.float32), 4, 8, 0)
    assert c["send_counts"].tolist() == [[0] * 4]
    assert c["tokens_per_expert"].tolist() == [[0] * 32]
    assert c["diag"][0] == 0


def _arrivals(T, P):
    """Barrier arrivals of one fused call: one per workgroup and barrier, and
    two barriers when the groups x bins table is scanned bin by bin (more
    than 8 entries per thread of a workgroup, at most 8 bins per group).
    Tiles are 64 tokens up to T = 4096, 128 up to 8192, 256 above (one token
    per thread)."""
    waves = 1 if T <= 4096 else (2 if T <= 8192 else 4)
    tiles = max(1, -(-T // (64 * waves)))
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    per = -(-tiles // min(cus, 256))
    groups = -(-tiles // per)
    barriers = 2 if groups * P > 8 * 64 * waves and -(-P // groups) <= 8 else 1
    return barriers * groups, barriers


def test_fused_workspace_reused_across_calls_and_sizes():
    sizes = [(5000, 64), (37, 8), (20000, 64), (70000, 4), (1, 2), (2999, 64), (256, 32),
             (20000, 128)]
    nbytes = max(ep.ep_dispatch_layout_workspace_bytes(T, P, 2) for T, P in sizes)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for i, (T, P) in enumerate(sizes):
        idx, w = _case(T, P * 2, 4 if P >= 4 else 2, P, seed=20 + i)
        check_fused(idx, w, P, 2, workspace=ws)
    hdr = ws[:16].view(torch.int32).cpu().numpy()
    assert hdr[3] == 0                        # no barrier time-out
    assert sum(_arrivals(T, P)[1] for T, P in sizes) > len(sizes)   # some took two barriers
    want = sum(_arrivals(T, P)[0] for T, P in sizes)
    assert hdr[0] == want and hdr[2] == want  # every arrival counted, handed to the next call
