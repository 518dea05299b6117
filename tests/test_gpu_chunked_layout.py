"""ep_dispatch_layout_chunked against the oracle: the counts of every chunk
and every chunk's send layout in one launch (axolotl "torch_dispatch":
chunk_bounds, dispatch_chunked_forward, compute_send_counts,
build_send_layout).  Chunk c's rows sit from row c * capacity on and must
equal the oracle's layout of that chunk's tokens, bit for bit; rows past a
chunk's count are left untouched."""

import numpy as np
import pytest
import torch

import oracle as O
from epgen import make_routing, spec
from tests.gpu_helpers import gpu_available, host, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

import combine_ep_send_amd as ep  # noqa: E402

SENTINEL = -7


def _run(s, C, cap=None, bad_ids=False):
    idx, w = make_routing(s)
    if bad_ids:
        idx = idx.copy()
        idx[::97, 0] = s.E + 3                 # ids past E: counted in diag, treated as unrouted
    T, K, P, El = s.T, s.K, s.P, s.E_local
    worst = max((b - a) * min(K, P) for a, b in O.chunk_bounds(T, C))
    cap = worst if cap is None else cap
    print(f"case: chunked layout {s.name} T={T} K={K} P={P} C={C} cap={cap} bad={bad_ids}",
          flush=True)
    rows = C * cap
    dev = "cuda"
    out = ep.SendLayout(
        send_token_idx=torch.full((rows,), SENTINEL, dtype=torch.int32, device=dev),
        send_rank=torch.full((rows,), SENTINEL, dtype=torch.int32, device=dev),
        send_idx=torch.full((rows, K), SENTINEL, dtype=torch.int32, device=dev),
        send_w=torch.full((rows, K), float(SENTINEL), dtype=torch.float32, device=dev),
        token_row=torch.full((T, K), SENTINEL, dtype=torch.int32, device=dev))
    c, lay = ep.ep_dispatch_layout_chunked(to_dev(idx), to_dev(w), P, El, C, cap, out=out)
    torch.cuda.synchronize()
    ep.check_workspaces()
    return idx, w, cap, c, lay


def _check(s, C, idx, w, cap, c, lay, bad=0):
    T, K, P, El = s.T, s.K, s.P, s.E_local
    clean = np.where(idx < s.E, idx, -1)       # the oracle's precondition: ids in [-1, E)
    dest, iir, sc, _ = O.compute_send_counts(clean, P, El, C)
    assert np.array_equal(host(c.dest), dest)
    assert np.array_equal(host(c.is_in_rank), iir)
    assert np.array_equal(host(c.send_counts), sc)
    assert int(host(c.diag)[0]) == bad
    g_sti, g_srk = host(lay.send_token_idx), host(lay.send_rank)
    g_sidx, g_sw, g_trow = host(lay.send_idx), host(lay.send_w), host(lay.token_row)
    for i, (a, b) in enumerate(O.chunk_bounds(T, C)):
        sti, srk, sidx, sw, trow = O.build_send_layout(clean[a:b], w[a:b], P, El)
        n = min(len(sti), cap)
        r0 = i * cap
        assert np.array_equal(g_sti[r0:r0 + n], sti[:n]), i
        assert np.array_equal(g_srk[r0:r0 + n], srk[:n]), i
        assert np.array_equal(g_sidx[r0:r0 + n], sidx[:n]), i
        assert np.array_equal(g_sw[r0:r0 + n].view(np.uint32), sw[:n].view(np.uint32)), i
        assert np.array_equal(g_trow[a:b], np.where(trow < cap, trow, -1)), i
        # rows past the chunk's count are left as they were
        assert np.all(g_sti[r0 + n:r0 + cap] == SENTINEL), i
        assert np.all(g_sidx[r0 + n:r0 + cap] == SENTINEL), i


# The launch reads back, per workgroup, only the rows of the groups its
# chunks span (chunk-local single pass) unless a chunk spans so many groups
# that the two-pass scan over every bin is cheaper.
@pytest.mark.parametrize("name,over,C", [
    ("fp8_t32768", {}, 4),                       # the chunked workload (chunk-local)
    ("fp8_t32768", {"T": 1000}, 3),              # ragged chunks; tiles straddle chunk ends
    ("skewed_t16384", {"T": 5}, 8),              # fewer tokens than chunks (7 empty ones)
    ("skewed_t16384", {"T": 3000, "seed": 2}, 2),
    ("uniform_t4096", {}, 16),                   # 8 destinations x 16 chunks
    ("uniform_t4096", {"K": 2, "T": 2500}, 5),
    ("uniform_t4096", {"K": 6, "T": 700, "seed": 3}, 7),
    ("fp8_t32768", {"T": 65536, "seed": 1}, 4),  # 256 workgroups: the two-pass scan
])
def test_chunked_layout_equals_the_oracle_per_chunk(name, over, C):
    s = spec(name, **over)
    idx, w, cap, c, lay = _run(s, C)
    _check(s, C, idx, w, cap, c, lay)


def test_chunked_layout_capacity_overflow_and_bad_ids():
    s = spec("skewed_t16384", T=4000, seed=5)
    C = 4
    idx, w, cap, c, lay = _run(s, C, cap=3000, bad_ids=True)
    bad = int(((idx >= s.E) | (idx < -1)).sum())
    _check(s, C, idx, w, cap, c, lay, bad=bad)


def test_chunked_pipeline_uses_the_one_launch_layout():
    """ChunkedDispatcher without exact counts takes its layouts from the one
    launch; its chunks' layouts are the oracle's."""
    s = spec("fp8_t32768", T=6000, H=256)
    idx, w = make_routing(s)
    d = ep.ChunkedDispatcher(s.T, s.K, s.H, num_local_experts=s.E_local, num_ranks=s.P,
                             chunks=4, exact_counts=False)
    from epgen import make_hidden
    x = make_hidden(s)
    d.forward(to_dev(x), to_dev(idx), to_dev(w), lambda i, rx, ri, rw: rx)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(d.bounds):
        sti, srk, sidx, sw, trow = O.build_send_layout(idx[a:b], w[a:b], s.P, s.E_local)
        lay = d.layouts[i]
        assert np.array_equal(host(lay.token_row), trow)
        assert np.array_equal(host(lay.send_token_idx)[:len(sti)], sti)
        assert np.array_equal(host(lay.send_idx)[:len(sti)], sidx)


def _random_case(seed):
    r = np.random.default_rng(1000 + seed)
    P = int(r.choice([1, 2, 3, 5, 8, 16, 32]))
    C = int(r.integers(1, max(2, min(16, 512 // P)) + 1))
    El = int(r.choice([1, 2, 3, 4, 8]))
    K = int(r.integers(1, min(16, P * El) + 1))
    T = int(r.choice([1, 2, 63, 64, 65, 257, 1000, 4097, 9000]))
    routing = str(r.choice(["uniform", "zipf"]))
    unrouted = float(r.choice([0.0, 0.05, 0.3]))
    s = spec("skewed_t16384").replace(name=f"random{seed}", T=T, E=P * El, K=K, P=P,
                                       routing=routing, unrouted_frac=unrouted, seed=seed)
    worst = max((b - a) * min(K, P) for a, b in O.chunk_bounds(T, C))
    cap = worst if r.random() < 0.7 else max(0, worst // 3)
    return s, C, cap


@pytest.mark.parametrize("seed", range(12))
def test_chunked_layout_random_shapes(seed):
    s, C, cap = _random_case(seed)
    idx, w, cap, c, lay = _run(s, C, cap=cap)
    _check(s, C, idx, w, cap, c, lay)


@pytest.mark.parametrize("streams", [1, 2])
def test_chunked_pipeline_on_a_callers_side_stream(streams):
    """A forward called with another stream current runs stream 0's work on
    that stream; its result, read after that stream alone is synchronized,
    is the oracle's, and a second forward on the default stream agrees."""
    s = spec("fp8_t32768", T=3000, H=512, seed=4)
    idx, w = make_routing(s)
    from epgen import make_hidden
    x = make_hidden(s)
    print(f"case: chunked pipeline on a side stream T={s.T} streams={streams}", flush=True)
    d_idx, d_w, d_x = to_dev(idx), to_dev(w), to_dev(x)
    d = ep.ChunkedDispatcher(s.T, s.K, s.H, num_local_experts=s.E_local, num_ranks=s.P,
                             chunks=3, streams=streams, exact_counts=False)
    caller = torch.cuda.Stream()
    caller.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(caller):
        out = torch.empty((s.T, s.H), dtype=torch.bfloat16, device="cuda")
        d.forward(d_x, d_idx, d_w, lambda i, rx, ri, rw: rx, out=out)
    caller.synchronize()
    got = host(out)
    ref = np.empty_like(x)
    for a, b in O.chunk_bounds(s.T, 3):
        sti, _, _, _, trow = O.build_send_layout(idx[a:b], w[a:b], s.P, s.E_local)
        ref[a:b] = O.combine(O.dispatch_permute(x[a:b], sti), trow, w[a:b])
    assert np.array_equal(got, ref)
    out2 = d.forward(d_x, d_idx, d_w, lambda i, rx, ri, rw: rx)
    torch.cuda.synchronize()
    assert np.array_equal(host(out2), ref)


class _Recorder:
    """A forward's timer hook that records the order in which launches are
    issued (and records nothing on the GPU)."""

    def __init__(self, log):
        self.log = log

    def start(self, name, stream):
        self.log.append(name)
        return None

    def stop(self, token):
        pass


@pytest.mark.parametrize("T,C,streams", [(3000, 4, 1), (3000, 4, 2), (3, 5, 2)])
def test_chunked_pipeline_issue_order(T, C, streams):
    """Chunk i+1's permute is issued before chunk i's local kernel, and chunk
    i's combine after it (axolotl dispatch_chunked_forward); chunks with no
    token issue nothing.  The result is the oracle's."""
    s = spec("fp8_t32768", T=T, H=512, seed=6)
    idx, w = make_routing(s)
    from epgen import make_hidden
    x = make_hidden(s)
    print(f"case: chunked pipeline issue order T={T} C={C} streams={streams}", flush=True)
    d = ep.ChunkedDispatcher(s.T, s.K, s.H, num_local_experts=s.E_local, num_ranks=s.P,
                             chunks=C, streams=streams, exact_counts=False)
    log = []

    def local(i, rx, ri, rw):
        log.append(f"local{i}")
        return rx

    out = d.forward(to_dev(x), to_dev(idx), to_dev(w), local, timer=_Recorder(log))
    torch.cuda.synchronize()
    live = [i for i, (a, b) in enumerate(O.chunk_bounds(T, C)) if b > a]
    want = ["dispatch_layout", "permute"]
    for n, i in enumerate(live):
        if n + 1 < len(live):
            want.append("permute")
        want += [f"local{i}", "combine"]
    assert log == want
    ref = np.empty_like(x)
    for a, b in O.chunk_bounds(T, C):
        sti, _, _, _, trow = O.build_send_layout(idx[a:b], w[a:b], s.P, s.E_local)
        ref[a:b] = O.combine(O.dispatch_permute(x[a:b], sti), trow, w[a:b])
    assert np.array_equal(host(out), ref)
