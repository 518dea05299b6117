"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on
seeded inputs, at sizes the oracle finishes quickly but that span several
scan tiles and a ragged tail, plus edge cases.  Integer, index and byte
outputs must match bit for bit; combine must be within 1 bf16 ulp of the
oracle's fixed-order fp32 result (and is expected to match exactly)."""

import numpy as np
import pytest
import torch

import oracle as O
from epgen import balanced_routing, make_hidden, make_routing, spec
from tests.gpu_helpers import (bf16_ulp_diff, bits, gpu_available, host, oracle_combine_subset,
                               to_dev)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

import combine_ep_send_amd as ep  # noqa: E402


def _print_case(**kw):
    print("case:", " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def send_case(T, H, E, K, P, routing="uniform", unrouted=0.0, seed=0):
    s = spec("tiny").replace(name="case", T=T, H=H, E=E, K=K, P=P, routing=routing,
                             unrouted_frac=unrouted, seed=seed)
    idx, w = make_routing(s)
    x = make_hidden(s)
    return s, idx, w, x


def check_send_path(idx, w, x, P, El, cap=None, fp8=False):
    """Run counts -> layout -> permute -> combine on the GPU and compare every
    output with the oracle."""
    T, K = idx.shape
    E = P * El
    d_idx, d_w, d_x = to_dev(idx), to_dev(w), to_dev(x)
    c = ep.ep_compute_send_counts(d_idx, P, El, 1)
    dest, iir, sc, tpe = O.compute_send_counts(idx, P, El, 1)
    assert np.array_equal(host(c.dest), dest)
    assert np.array_equal(host(c.is_in_rank), iir)
    assert np.array_equal(host(c.send_counts), sc)
    assert np.array_equal(host(c.tokens_per_expert), tpe)
    assert host(c.diag)[0] == 0

    sti, srk, sidx, sw, trow = O.build_send_layout(idx, w, P, El)
    N = len(sti)
    if cap is None:
        cap = T * min(K, P)
    # pre-fill the outputs with sentinels so untouched rows can be checked
    lay = ep.SendLayout(
        send_token_idx=torch.full((cap + 3,), -7, dtype=torch.int32, device="cuda"),
        send_rank=torch.full((cap + 3,), -7, dtype=torch.int32, device="cuda"),
        send_idx=torch.full((cap + 3, K), -7, dtype=torch.int32, device="cuda"),
        send_w=torch.full((cap + 3, K), -7.0, dtype=torch.float32, device="cuda"),
        token_row=torch.full((T, K), -7, dtype=torch.int32, device="cuda"))
    ep.ep_build_send_layout(d_idx, d_w, c.dest, c.send_counts[0], P, El, cap, out=lay)
    g_sti, g_srk = host(lay.send_token_idx), host(lay.send_rank)
    g_sidx, g_sw, g_trow = host(lay.send_idx), host(lay.send_w), host(lay.token_row)
    assert np.array_equal(g_sti[:N], sti)
    assert np.array_equal(g_srk[:N], srk)
    assert np.array_equal(g_sidx[:N], sidx)
    assert np.array_equal(g_sw[:N].view(np.uint32), sw.view(np.uint32))
    assert np.array_equal(g_trow, trow)
    assert np.all(g_sti[N:] == -7) and np.all(g_sidx[N:] == -7)     # rows >= N untouched

    if fp8:
        q = torch.full((cap, x.shape[1]), 0x55, dtype=torch.uint8, device="cuda")
        q = q.view(torch.float8_e4m3fn)
        s = torch.full((cap, x.shape[1] // 128), -1.0, dtype=torch.float32, device="cuda")
        ep.ep_dispatch_permute(d_x, lay.token_row, cap, fp8=True, out=q, out_scale=s)
        oq, osc = O.dispatch_permute_fp8(x, sti)
        gq, gs = host(q), host(s)
        assert np.array_equal(gq[:N], oq)
        assert np.array_equal(gs[:N].view(np.uint32), osc.view(np.uint32))
        assert np.all(gq[N:] == 0x55)
        y_orc = O.dequantize_rows_fp8(oq, osc)
    else:
        sx = torch.full((cap, x.shape[1]), 0x1234, dtype=torch.int16, device="cuda")
        sx = sx.view(torch.bfloat16)
        ep.ep_dispatch_permute(d_x, lay.token_row, cap, out=sx)
        gsx = bits(sx)
        assert np.array_equal(gsx[:N], O.dispatch_permute(x, sti))
        assert np.all(gsx[N:] == 0x1234)
        y_orc = O.dispatch_permute(x, sti)

    # combine: GPU reads its own expert-output rows; the oracle its own
    y_dev = to_dev(y_orc) if fp8 else sx[:N]
    out = ep.ep_combine(y_dev, lay.token_row, d_w)
    ref = O.combine(y_orc, trow, w)
    got = bits(out)
    assert bf16_ulp_diff(got, ref).max(initial=0) <= 1
    assert np.array_equal(got, ref), "combine differs from the fixed-order fp32 oracle"
    return N


# ---------------------------------------------------------------------------

def test_hand_worked_example(golden):
    g, ex = golden, golden["expected"]
    idx = np.array(g["topk_idx"], dtype=np.int64)
    w = np.array(g["topk_weights"], dtype=np.float32)
    x = (torch.tensor(g["x"], dtype=torch.float32).to(torch.bfloat16)
         .view(torch.int16).numpy().view(np.uint16))
    c = ep.ep_compute_send_counts(to_dev(idx), g["P"], g["E_local"], 2)
    assert host(c.dest).tolist() == ex["dest"]
    assert host(c.is_in_rank).tolist() == ex["is_in_rank"]
    assert host(c.send_counts).tolist() == ex["chunks_2"]["send_counts"]
    assert host(c.tokens_per_expert).tolist() == ex["chunks_2"]["tokens_per_expert"]
    recv_x, recv_idx, recv_w, h = ep.dispatch(to_dev(x), to_dev(idx), to_dev(w),
                                              num_local_experts=g["E_local"], num_ranks=g["P"])
    assert h.num_send == ex["num_send"]
    assert host(h.send_token_idx).tolist() == ex["send_token_idx"]
    assert host(h.send_rank).tolist() == ex["send_rank"]
    assert host(recv_idx).tolist() == ex["send_idx"]
    assert host(recv_w).tolist() == ex["send_w"]
    assert host(h.token_row).tolist() == ex["token_row"]
    assert np.array_equal(bits(recv_x), x[ex["send_token_idx"]])
    out = ep.combine(recv_x, h)
    assert out.float().cpu().tolist() == ex["combine_identity"]
    b = ex["batched"]
    bx, tpe, trow = ep.ep_batched_prepare(to_dev(x), to_dev(idx), b["first_expert"],
                                          b["E_local"], b["max_num_tokens"])
    assert host(tpe).tolist() == b["tokens_per_expert"]
    assert host(trow).tolist() == b["token_row"]
    gbx = bits(bx)
    for e in range(b["E_local"]):
        for s, t in enumerate(b["slot_token"][e]):
            assert np.array_equal(gbx[e, s], x[t] if t >= 0 else np.zeros(8, np.uint16))


@pytest.mark.parametrize("T,H,E,K,P,routing,unrouted", [
    (256, 512, 8, 2, 2, "uniform", 0.0),          # the tiny workload
    (1000, 256, 64, 6, 8, "uniform", 0.0),        # several tiles + ragged tail
    (1537, 1024, 256, 8, 32, "zipf", 0.05),       # skewed, unrouted slots
    (700, 7168, 256, 8, 32, "uniform", 0.0),      # full hidden size
    (300, 64, 16, 16, 4, "uniform", 0.1),         # K = 16
    (513, 8, 4, 1, 4, "uniform", 0.0),            # K = 1, H = 8
    (400, 128, 96, 3, 1, "uniform", 0.0),         # one destination
    (300, 16384, 64, 4, 8, "uniform", 0.0),       # H beyond one workgroup's row (2 combine chunks)
    (200, 9216, 64, 6, 8, "zipf", 0.05),          # ragged combine chunks (2 x 576 pieces)
])
def test_send_path_matches_oracle(T, H, E, K, P, routing, unrouted):
    _print_case(T=T, H=H, E=E, K=K, P=P, routing=routing)
    s, idx, w, x = send_case(T, H, E, K, P, routing, unrouted)
    check_send_path(idx, w, x, P, E // P)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_send_path_other_seeds(seed):
    _print_case(seed=seed)
    s, idx, w, x = send_case(2000, 512, 64, 6, 8, seed=seed)
    check_send_path(idx, w, x, 8, 8)


@pytest.mark.parametrize("T,H,K,P", [(600, 1024, 8, 32), (257, 128, 4, 8), (64, 7168, 8, 32),
                                     (100, 16384, 8, 32)])
def test_fp8_path_matches_oracle(T, H, K, P):
    _print_case(T=T, H=H, K=K, P=P, fp8=True)
    s, idx, w, x = send_case(T, H, 256, K, P)
    # plant exact zeros, negative zeros and a tiny group to cover the edge rules
    x[0, :128] = 0
    x[1, 128:256] = 0x8000
    x[2, :] = np.where(np.arange(H) % 2 == 0, 0x0001, 0x8001).astype(np.uint16)
    idx[0] = np.arange(K)
    check_send_path(idx, w, x, P, 256 // P, fp8=True)


def test_exact_capacity_and_tight_buffers():
    s, idx, w, x = send_case(777, 256, 64, 6, 8)
    N = int(O.compute_send_counts(idx, 8, 8)[1].sum())
    check_send_path(idx, w, x, 8, 8, cap=N)


def test_capacity_overflow_drops_rows_without_writing_past():
    _print_case(case="overflow")
    s, idx, w, x = send_case(500, 64, 64, 6, 8)
    sti, srk, sidx, sw, trow = O.build_send_layout(idx, w, 8, 8)
    N = len(sti)
    cap = N // 2
    d_idx, d_w, d_x = to_dev(idx), to_dev(w), to_dev(x)
    c = ep.ep_compute_send_counts(d_idx, 8, 8)
    big = cap + 64
    lay = ep.SendLayout(*(torch.full(sh, -7, dtype=dt, device="cuda") for sh, dt in
                          (((big,), torch.int32), ((big,), torch.int32), ((big, 6), torch.int32),
                           ((big, 6), torch.float32), ((500, 6), torch.int32))))
    ep.ep_build_send_layout(d_idx, d_w, c.dest, c.send_counts[0], 8, 8, cap, out=lay)
    assert np.array_equal(host(lay.send_token_idx)[:cap], sti[:cap])
    assert np.all(host(lay.send_token_idx)[cap:] == -7)
    g_trow = host(lay.token_row)
    assert np.array_equal(g_trow, np.where(trow < cap, trow, -1))
    sx = torch.zeros((big, 64), dtype=torch.bfloat16, device="cuda")
    ep.ep_dispatch_permute(d_x, lay.token_row, cap, out=sx)
    assert not bits(sx)[cap:].any()
    assert host(c.send_counts).sum() == N                  # true counts still reported


def test_unrouted_and_empty_inputs():
    _print_case(case="unrouted/empty")
    s, idx, w, x = send_case(300, 64, 32, 4, 4)
    idx[::3] = -1
    w[::3] = 0
    check_send_path(idx, w, x, 4, 8)
    # all slots unrouted: nothing is sent, combine gives zeros
    idx_all = np.full((130, 4), -1, dtype=np.int64)
    w0 = np.zeros((130, 4), np.float32)
    x0 = make_hidden(spec("tiny", T=130, H=64))
    check_send_path(idx_all, w0, x0, 4, 8)
    # T = 0
    e_idx = torch.empty((0, 4), dtype=torch.int64, device="cuda")
    c = ep.ep_compute_send_counts(e_idx, 4, 8, 3)
    assert host(c.send_counts).tolist() == [[0] * 4] * 3
    lay = ep.ep_build_send_layout(e_idx, torch.empty((0, 4), device="cuda"), c.dest,
                                  c.send_counts[0], 4, 8, 0)
    out = ep.ep_combine(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"),
                        lay.token_row, torch.empty((0, 4), device="cuda"))
    assert out.shape == (0, 64)


def test_one_hot_destination():
    _print_case(case="one hot destination")
    T, K, E, P = 1200, 4, 64, 8
    rng = np.random.default_rng(5)
    idx = np.stack([rng.permutation(8)[:K] + 16 for _ in range(T)]).astype(np.int64)
    w = np.full((T, K), 0.25, np.float32)
    x = make_hidden(spec("tiny", T=T, H=256))
    n = check_send_path(idx, w, x, P, E // P)
    assert n == T


def test_balanced_routing_round_trip_is_exact():
    T, K, E, P = 2048, 8, 256, 32
    idx, w = balanced_routing(T, K, E)
    x = make_hidden(spec("tiny", T=T, H=512))
    check_send_path(idx, w, x, P, E // P)
    recv_x, _, _, h = ep.dispatch(to_dev(x), to_dev(idx), to_dev(w), num_local_experts=E // P,
                                  num_ranks=P)
    out = ep.combine(recv_x, h)
    # weights 1/8: every product and partial sum is exact, so the values
    # round-trip; a -0.0 input comes back +0.0 (the sum starts at +0.0)
    assert np.array_equal(O.bf16_to_f32(bits(out)), O.bf16_to_f32(x))


def test_bad_ids_are_counted_and_unrouted():
    _print_case(case="bad ids")
    s, idx, w, x = send_case(400, 64, 32, 4, 4)
    bad = idx.copy()
    bad[5, 1] = 32
    bad[9, 0] = -5
    bad[77, 3] = 1 << 40
    c = ep.ep_compute_send_counts(to_dev(bad), 4, 8)
    assert host(c.diag)[0] == 3
    clean = bad.copy()
    clean[(clean < -1) | (clean >= 32)] = -1
    dest, iir, sc, tpe = O.compute_send_counts(clean, 4, 8)
    assert np.array_equal(host(c.dest), dest)
    assert np.array_equal(host(c.send_counts), sc)


@pytest.mark.parametrize("chunks", [1, 3, 4, 7])
def test_chunked_counts(chunks):
    s, idx, w, x = send_case(1001, 64, 256, 8, 32)
    c = ep.ep_compute_send_counts(to_dev(idx), 32, 8, chunks)
    _, _, sc, tpe = O.compute_send_counts(idx, 32, 8, chunks)
    assert np.array_equal(host(c.send_counts), sc)
    assert np.array_equal(host(c.tokens_per_expert), tpe)


def test_workspace_reused_across_calls_and_sizes():
    """The scan workspace rearms itself: many calls of different sizes on one
    workspace, without clearing it, each match the oracle."""
    ws = torch.zeros(ep.ep_layout_workspace_bytes(5000, 64), dtype=torch.uint8, device="cuda")
    for i, (T, P) in enumerate([(5000, 64), (37, 8), (4096, 32), (1, 2), (2999, 64), (256, 32)]):
        s, idx, w, x = send_case(T, 16, P * 2, 4, P, seed=10 + i)
        d_idx, d_w = to_dev(idx), to_dev(w)
        c = ep.ep_compute_send_counts(d_idx, P, 2)
        lay = ep.ep_build_send_layout(d_idx, d_w, c.dest, c.send_counts[0], P, 2, T * 4,
                                      workspace=ws)
        sti, srk, sidx, sw, trow = O.build_send_layout(idx, w, P, 2)
        assert np.array_equal(host(lay.token_row), trow)
        assert np.array_equal(host(lay.send_token_idx)[:len(sti)], sti)
    hdr = ws[:16].view(torch.int32).cpu().numpy()
    assert hdr[0] == 0 and hdr[1] == 0 and hdr[3] == 0     # ticket, done rearmed; no error
    assert hdr[2] == 6                                       # one epoch per call


# ---------------------------------------------------------------------------
# expert-batched layout
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,H,E,K,first,El,M", [
    (1000, 256, 256, 8, 0, 32, 1000),
    (777, 512, 64, 6, 40, 8, 200),
    (300, 64, 16, 4, 0, 16, 300),
    (5, 8, 6, 3, 2, 2, 4),
])
def test_batched_matches_oracle(T, H, E, K, first, El, M):
    _print_case(T=T, H=H, E=E, K=K, first=first, El=El, M=M)
    s = spec("batched_t8192").replace(T=T, H=H, E=E, K=K, P=E // El)
    idx, w = make_routing(s)
    x = make_hidden(s)
    d_x, d_idx, d_w = to_dev(x), to_dev(idx), to_dev(w)
    bx = torch.full((El, M, H), 7.0, dtype=torch.bfloat16, device="cuda")
    ep.ep_batched_prepare(d_x, d_idx, first, El, M, out=bx)
    obx, otpe, otrow = O.batched_prepare(x, idx, first, El, M)
    _, gtpe, gtrow = ep.ep_batched_prepare(d_x, d_idx, first, El, M, out=bx)
    assert np.array_equal(bits(bx), obx)
    assert np.array_equal(host(gtpe), otpe)
    assert np.array_equal(host(gtrow), otrow)
    out = ep.ep_combine(bx, gtrow, d_w)
    ref = O.combine(obx.reshape(-1, H), otrow, w)
    assert np.array_equal(bits(out), ref)


def test_batched_overflow_drops_slots():
    _print_case(case="batched overflow")
    T, K = 300, 4
    idx = np.zeros((T, K), dtype=np.int64)
    idx[:, 1:] = -1                                  # every token names expert 0
    x = make_hidden(spec("tiny", T=T, H=64))
    bx, tpe, trow = ep.ep_batched_prepare(to_dev(x), to_dev(idx), 0, 2, 100)
    assert host(tpe).tolist() == [300, 0]
    g = host(trow)
    assert np.array_equal(g[:100, 0], np.arange(100)) and np.all(g[100:, 0] == -1)
    assert np.array_equal(bits(bx)[0], x[:100]) and not bits(bx)[1].any()
