"""Pins for the oracle's routing metadata: counts, send layout, permute,
batched layout and chunking.  Every expectation here comes from something
other than the oracle itself: pure-Python brute force, library sorts and
bincounts, closed forms and a hand-worked example."""

import itertools

import numpy as np
import pytest

import oracle as O
from epgen import CONFIGS, balanced_routing, make_hidden, make_routing, spec


# --------------------------------------------------------------------------
# brute force (pure Python, built from sets and a sort of (p, t) pairs)
# --------------------------------------------------------------------------

def brute_layout(idx, w, P, El):
    T, K = len(idx), len(idx[0])
    pairs = []
    for t in range(T):
        owners = {int(i) // El for i in idx[t] if i >= 0}
        pairs.extend((p, t) for p in owners)
    pairs.sort()
    sti, srk, sidx, sw = [], [], [], []
    row_of = {}
    for n, (p, t) in enumerate(pairs):
        row_of[(t, p)] = n
        sti.append(t)
        srk.append(p)
        sidx.append([int(i) - p * El if i >= 0 and int(i) // El == p else -1 for i in idx[t]])
        sw.append([float(w[t][k]) if idx[t][k] >= 0 and int(idx[t][k]) // El == p else 0.0
                   for k in range(K)])
    trow = [[row_of[(t, int(i) // El)] if i >= 0 else -1 for i in idx[t]] for t in range(T)]
    counts = [sum(1 for (p, _) in pairs if p == q) for q in range(P)]
    tpe = [sum(1 for t in range(T) for i in idx[t] if i == e) for e in range(P * El)]
    return sti, srk, sidx, sw, trow, counts, tpe


def tiny_cases():
    """Every ordered K-subset pattern for small E, plus unrouted slots."""
    cases = []
    for E, K, P in [(4, 2, 2), (4, 1, 4), (6, 3, 3), (8, 2, 2), (8, 3, 4), (4, 4, 1)]:
        El = E // P
        subsets = list(itertools.permutations(range(E), K))
        rng = np.random.default_rng(E * 100 + K * 10 + P)
        order = rng.permutation(len(subsets))
        for start in range(0, min(len(subsets), 48), 8):
            rows = [list(subsets[j]) for j in order[start:start + 8]]
            idx = np.array(rows, dtype=np.int64)
            drop = rng.random(idx.shape) < 0.2
            idx[drop] = -1
            w = rng.random(idx.shape).astype(np.float32)
            w[drop] = 0.0
            cases.append((idx, w, P, El))
    return cases


@pytest.mark.parametrize("case", tiny_cases())
def test_layout_matches_brute_force(case):
    idx, w, P, El = case
    sti, srk, sidx, sw, trow, counts, tpe = brute_layout(idx.tolist(), w.tolist(), P, El)
    dest, iir, sc, tpe_o = O.compute_send_counts(idx, P, El)
    assert sc[0].tolist() == counts
    assert tpe_o[0].tolist() == tpe
    assert int(iir.sum()) == len(sti)
    a, b, c, d, e = O.build_send_layout(idx, w, P, El)
    assert a.tolist() == sti
    assert b.tolist() == srk
    assert c.tolist() == sidx
    assert np.array_equal(d, np.array(sw, dtype=np.float32).reshape(d.shape))
    assert e.tolist() == trow


def test_dest_definition_small():
    idx = np.array([[5, -1, 0], [3, 4, 1]], dtype=np.int64)
    dest, iir, sc, tpe = O.compute_send_counts(idx, 3, 2)
    assert dest.tolist() == [[2, -1, 0], [1, 2, 0]]
    assert iir.tolist() == [[1, 0, 1], [1, 1, 1]]
    assert sc.tolist() == [[2, 1, 2]]


# --------------------------------------------------------------------------
# library routines: np.lexsort, np.bincount, stable argsort
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "uniform_t4096"])
def test_layout_equals_lexsort(name):
    s = spec(name)
    idx, w = make_routing(s)
    P, El = s.P, s.E_local
    dest, iir, sc, tpe = O.compute_send_counts(idx, P, El)
    t_all, p_all = np.nonzero(iir)
    order = np.lexsort((t_all, p_all))               # primary key p, then t
    sti, srk, sidx, sw, trow = O.build_send_layout(idx, w, P, El)
    assert np.array_equal(sti, t_all[order])
    assert np.array_equal(srk, p_all[order])
    assert np.array_equal(sc[0], np.bincount(p_all, minlength=P))
    routed = idx[idx >= 0]
    assert np.array_equal(tpe[0], np.bincount(routed, minlength=P * El))


def test_layout_invariants_skewed():
    s = spec("skewed_t16384", T=4096)
    idx, w = make_routing(s)
    P, El = s.P, s.E_local
    dest, iir, sc, tpe = O.compute_send_counts(idx, P, El)
    sti, srk, sidx, sw, trow = O.build_send_layout(idx, w, P, El)
    N = len(sti)
    assert N == int(iir.sum()) == int(sc.sum())
    # send_rank non-decreasing; tokens strictly ascending inside a segment
    assert np.all(np.diff(srk) >= 0)
    same = srk[1:] == srk[:-1]
    assert np.all(np.diff(sti)[same] > 0)
    # segment starts are the exclusive prefix of send_counts
    starts = np.concatenate([[0], np.cumsum(sc[0])[:-1]])
    for p in range(P):
        if sc[0, p]:
            assert srk[starts[p]] == p
    # every send row carries >= 1 local id, and local ids agree slot by slot
    assert np.all((sidx >= 0).any(axis=1))
    t = sti.astype(np.int64)
    glob = np.where(sidx >= 0, sidx + srk[:, None] * El, -1)
    assert np.array_equal(glob[sidx >= 0], idx[t][sidx >= 0])
    assert np.all(sidx < El)
    assert np.array_equal(sw[sidx >= 0], w[t][sidx >= 0])
    assert np.all(sw[sidx < 0] == 0)
    # token_row is the inverse: slot k of token t lands on a row of t owned by dest
    for tt in range(0, s.T, 97):
        for k in range(s.K):
            r = trow[tt, k]
            if idx[tt, k] < 0:
                assert r == -1
            else:
                assert sti[r] == tt and srk[r] == dest[tt, k]
                assert sidx[r, k] == idx[tt, k] - dest[tt, k] * El
    # bijection: every (t, p) member appears exactly once
    key = sti.astype(np.int64) * P + srk
    assert len(np.unique(key)) == N
    # tokens_per_expert sums to the routed slots; send_counts bounded by experts
    assert tpe.sum() == int((idx >= 0).sum())
    assert np.all(sc[0] <= tpe[0].reshape(P, El).sum(axis=1))


# --------------------------------------------------------------------------
# closed forms: forced-balanced routing (NeMo static benchmark routing)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T,K,E,P", [(64, 2, 8, 2), (256, 8, 256, 32), (96, 3, 12, 4),
                                     (128, 4, 16, 2)])
def test_balanced_routing_closed_form(T, K, E, P):
    idx, w = balanced_routing(T, K, E)
    El = E // P
    dest, iir, sc, tpe = O.compute_send_counts(idx, P, El)
    assert (T * K) % E == 0
    assert np.all(tpe[0] == T * K // E)
    if El % K == 0 and T % (E // K) == 0:
        # each token's K consecutive ids sit inside one destination, and the
        # first ids t*K mod E cycle through every destination equally often
        assert np.all(sc[0] == T // P)
        assert int(iir.sum()) == T


# --------------------------------------------------------------------------
# chunking
# --------------------------------------------------------------------------

def test_chunk_bounds_cases(golden):
    assert O.chunk_bounds(5, 2) == [tuple(b) for b in golden["expected"]["chunks_2"]["bounds"]]
    assert O.chunk_bounds(3, 4) == [tuple(b) for b in golden["expected"]["chunk_bounds_3_4"]]
    assert O.chunk_bounds(32768, 4) == [(0, 8192), (8192, 16384), (16384, 24576), (24576, 32768)]
    assert O.chunk_bounds(0, 3) == [(0, 0), (0, 0), (0, 0)]
    for T in range(0, 40):
        for C in range(1, 7):
            b = O.chunk_bounds(T, C)
            assert len(b) == C and b[0][0] == 0 and b[-1][1] == T
            assert all(b[i][1] == b[i + 1][0] for i in range(C - 1))
            sizes = [e - s for s, e in b]
            assert all(sz == T // C for sz in sizes[:-1])


def test_chunked_counts_sum_to_whole():
    s = spec("fp8_t32768", T=2000)
    idx, _ = make_routing(s)
    _, _, sc4, tpe4 = O.compute_send_counts(idx, s.P, s.E_local, 4)
    _, _, sc1, tpe1 = O.compute_send_counts(idx, s.P, s.E_local, 1)
    assert np.array_equal(sc4.sum(axis=0), sc1[0])
    assert np.array_equal(tpe4.sum(axis=0), tpe1[0])
    for c, (a, b) in enumerate(O.chunk_bounds(2000, 4)):
        _, _, scc, _ = O.compute_send_counts(idx[a:b], s.P, s.E_local, 1)
        assert np.array_equal(scc[0], sc4[c])


# --------------------------------------------------------------------------
# hand-worked example
# --------------------------------------------------------------------------

def test_hand_worked_metadata(golden):
    g, ex = golden, golden["expected"]
    idx = np.array(g["topk_idx"], dtype=np.int64)
    w = np.array(g["topk_weights"], dtype=np.float32)
    dest, iir, sc, tpe = O.compute_send_counts(idx, g["P"], g["E_local"])
    assert dest.tolist() == ex["dest"]
    assert iir.tolist() == ex["is_in_rank"]
    assert sc[0].tolist() == ex["send_counts"]
    assert tpe[0].tolist() == ex["tokens_per_expert"]
    _, _, sc2, tpe2 = O.compute_send_counts(idx, g["P"], g["E_local"], 2)
    assert sc2.tolist() == ex["chunks_2"]["send_counts"]
    assert tpe2.tolist() == ex["chunks_2"]["tokens_per_expert"]
    sti, srk, sidx, sw, trow = O.build_send_layout(idx, w, g["P"], g["E_local"])
    assert len(sti) == ex["num_send"]
    assert sti.tolist() == ex["send_token_idx"]
    assert srk.tolist() == ex["send_rank"]
    assert sidx.tolist() == ex["send_idx"]
    assert sw.tolist() == ex["send_w"]
    assert trow.tolist() == ex["token_row"]


def test_hand_worked_permute_and_batched(golden):
    g, ex = golden, golden["expected"]
    import torch
    x = (torch.tensor(g["x"], dtype=torch.float32).to(torch.bfloat16)
         .view(torch.int16).numpy().view(np.uint16))
    idx = np.array(g["topk_idx"], dtype=np.int64)
    sx = O.dispatch_permute(x, np.array(ex["send_token_idx"]))
    assert np.array_equal(sx, x[ex["send_token_idx"]])
    b = ex["batched"]
    bx, tpe, trow = O.batched_prepare(x, idx, b["first_expert"], b["E_local"],
                                      b["max_num_tokens"])
    assert tpe.tolist() == b["tokens_per_expert"]
    assert trow.tolist() == b["token_row"]
    for e in range(b["E_local"]):
        for s, t in enumerate(b["slot_token"][e]):
            if t < 0:
                assert not bx[e, s].any()
            else:
                assert np.array_equal(bx[e, s], x[t])


# --------------------------------------------------------------------------
# batched layout vs library routines
# --------------------------------------------------------------------------

@pytest.mark.parametrize("first,El", [(0, 32), (96, 32), (250, 6)])
def test_batched_equals_stable_argsort(first, El):
    s = spec("batched_t8192", T=512, H=16)
    idx, w = make_routing(s)
    rng = np.random.default_rng(7)
    x = rng.integers(0, 1 << 16, size=(s.T, s.H), dtype=np.uint16)
    M = 64
    bx, tpe, trow = O.batched_prepare(x, idx, first, El, M)
    local = (idx >= first) & (idx < first + El)
    t_all, k_all = np.nonzero(local)
    e_all = idx[t_all, k_all] - first
    assert np.array_equal(tpe, np.bincount(e_all, minlength=El))
    order = np.argsort(e_all * s.T + t_all, kind="stable")
    slots = np.concatenate([np.arange(c) for c in tpe])
    assert np.array_equal(trow[t_all[order], k_all[order]], e_all[order] * M + slots)
    assert np.all(trow[~local] == -1)
    for e in range(El):
        assert not bx[e, tpe[e]:].any()           # zero padding
        toks = t_all[order][e_all[order] == e]
        assert np.array_equal(bx[e, :tpe[e]], x[toks])


def test_batched_overflow_raises():
    idx = np.array([[0], [0], [0]], dtype=np.int64)
    x = np.zeros((3, 8), dtype=np.uint16)
    with pytest.raises(ValueError):
        O.batched_prepare(x, idx, 0, 1, 2)


def test_validation_rejects_bad_ids():
    with pytest.raises(ValueError):
        O.compute_send_counts(np.array([[8, 0]]), 2, 4)
    with pytest.raises(ValueError):
        O.compute_send_counts(np.array([[-2, 0]]), 2, 4)
    with pytest.raises(ValueError):
        O.compute_send_counts(np.array([[1, 1]]), 2, 4)


@pytest.mark.parametrize("name", list(CONFIGS))
def test_config_routing_invariants(name):
    s = spec(name, T=min(CONFIGS[name].T, 2048))
    idx, w = make_routing(s)
    O.validate_routing(idx, s.E)
    P = s.P
    dest, iir, sc, tpe = O.compute_send_counts(idx, P, s.E_local, s.chunks)
    assert int(sc.sum()) == int(iir.sum())
    assert int(tpe.sum()) == int((idx >= 0).sum())


# --------------------------------------------------------------------------
# receive-side regroup by local expert
# --------------------------------------------------------------------------

def _recv_segment(name="skewed_t16384", T=600, p=5, seed=0):
    """The rows one destination receives: its send segment with K-wide local
    ids (-1 elsewhere) and weights, as the send layout builds them."""
    s = spec(name, T=T, H=16, seed=seed)
    idx, w = make_routing(s)
    rng = np.random.default_rng(seed)
    x = rng.integers(0, 1 << 16, size=(s.T, s.H), dtype=np.uint16)
    sti, srk, sidx, sw, trow = O.build_send_layout(idx, w, s.P, s.E_local)
    seg = srk == p
    return x[sti[seg]], sidx[seg], sw[seg], s.E_local


@pytest.mark.parametrize("align", [1, 4, 16, 128])
def test_regroup_equals_stable_sort_and_bincount(align):
    rx, ridx, rw, El = _recv_segment()
    px, src, pw, cnt, off, rmap = O.regroup_by_expert(rx, ridx, rw, El, align)
    r_all, k_all = np.nonzero(ridx >= 0)
    e_all = ridx[r_all, k_all]
    assert np.array_equal(cnt, np.bincount(e_all, minlength=El))
    padded = -(-cnt // align) * align
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(padded)]))
    order = np.lexsort((r_all, e_all))                   # expert, then row
    rank = np.concatenate([np.arange(c) for c in cnt]) if len(cnt) else np.zeros(0)
    want = off[e_all[order]] + rank
    assert np.array_equal(rmap[r_all[order], k_all[order]], want)
    assert np.all(rmap[ridx < 0] == -1)
    assert np.array_equal(src[want], r_all[order])
    assert np.array_equal(px[want], rx[r_all[order]])
    assert np.array_equal(pw[want].view(np.uint32), rw[r_all[order], k_all[order]].view(np.uint32))
    pad = np.ones(len(src), dtype=bool)
    pad[want] = False
    assert np.all(src[pad] == -1) and not px[pad].any() and not pw[pad].any()
    assert len(src) == off[-1] and np.all(off % align == 0)


def test_regroup_brute_force_tiny():
    # 5 received rows, K=3, 3 local experts, alignment 2, worked by hand:
    # e0 <- rows 0, 3 ; e1 <- rows 1, 3, 4 ; e2 <- row 2
    ridx = np.array([[0, -1, -1], [-1, 1, -1], [2, -1, -1], [1, 0, -1], [-1, -1, 1]])
    rw = np.arange(15, dtype=np.float32).reshape(5, 3) / 16
    rx = np.arange(10, dtype=np.uint16).reshape(5, 2) + 1
    px, src, pw, cnt, off, rmap = O.regroup_by_expert(rx, ridx, rw, 3, 2)
    assert cnt.tolist() == [2, 3, 1]
    assert off.tolist() == [0, 2, 6, 8]
    assert src.tolist() == [0, 3, 1, 3, 4, -1, 2, -1]
    assert pw.tolist() == [0 / 16, 10 / 16, 4 / 16, 9 / 16, 14 / 16, 0, 6 / 16, 0]
    assert rmap.tolist() == [[0, -1, -1], [-1, 2, -1], [6, -1, -1], [3, 1, -1], [-1, -1, 4]]
    assert px.tolist() == [[1, 2], [7, 8], [3, 4], [7, 8], [9, 10], [0, 0], [5, 6], [0, 0]]


def test_regroup_restore_is_weighted_sum():
    # an identity expert over the regrouped rows, restored by the weighted
    # combine through row_map, gives each received row times its local weights
    s = spec("uniform_t4096", T=400, H=32)
    idx, w = make_routing(s)
    x = make_hidden(s)
    sti, srk, sidx, sw, trow = O.build_send_layout(idx, w, s.P, s.E_local)
    seg = srk == 3
    px, src, pw, cnt, off, rmap = O.regroup_by_expert(x[sti[seg]], sidx[seg], sw[seg],
                                                      s.E_local, 8)
    back = O.combine(px, rmap, sw[seg])
    lw = sw[seg].astype(np.float64).sum(axis=1)[:, None]
    exact = lw * O.bf16_to_f32(x[sti[seg]]).astype(np.float64)
    got = O.bf16_to_f32(back).astype(np.float64)
    ulp = np.maximum(np.abs(exact), 2.0 ** -126) * 2.0 ** -7
    assert np.all(np.abs(got - exact) <= ulp)


def test_regroup_rejects_bad_ids_and_alignment():
    with pytest.raises(ValueError):
        O.regroup_by_expert(np.zeros((1, 8), np.uint16), np.array([[3]]), np.ones((1, 1)), 3)
    with pytest.raises(ValueError):
        O.regroup_by_expert(np.zeros((1, 8), np.uint16), np.array([[1, 1]]), np.ones((1, 2)), 3)
    with pytest.raises(ValueError):
        O.regroup_by_expert(np.zeros((1, 8), np.uint16), np.array([[1]]), np.ones((1, 1)), 3, 0)


def test_regroup_groups_are_segments_end_to_end():
    # every destination's segment regrouped at once (row_group = send_rank)
    # equals the per-segment regroups laid end to end
    s = spec("uniform_t4096", T=300, H=8)
    idx, w = make_routing(s)
    rng = np.random.default_rng(2)
    x = rng.integers(0, 1 << 16, size=(s.T, s.H), dtype=np.uint16)
    sti, srk, sidx, sw, trow = O.build_send_layout(idx, w, s.P, s.E_local)
    A = 4
    px, src, pw, cnt, off, rmap = O.regroup_by_expert(x[sti], sidx, sw, s.E_local, A,
                                                      row_group=srk, num_groups=s.P)
    base = 0
    for p in range(s.P):
        seg = np.flatnonzero(srk == p)
        qx, qs, qw, qc, qo, qm = O.regroup_by_expert(x[sti[seg]], sidx[seg], sw[seg],
                                                     s.E_local, A)
        assert np.array_equal(cnt[p * s.E_local:(p + 1) * s.E_local], qc)
        assert np.array_equal(off[p * s.E_local:(p + 1) * s.E_local + 1], qo + base)
        M = int(qo[-1])
        assert np.array_equal(px[base:base + M], qx)
        assert np.array_equal(src[base:base + M], np.where(qs >= 0, seg[qs], -1))
        assert np.array_equal(rmap[seg], np.where(qm >= 0, qm + base, -1))
        base += M
    assert base == len(src)
