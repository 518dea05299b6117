"""GPU parity of the combine's other modes against the CPU oracle, bit for
bit: the unweighted per-destination partial sums (the local expert kernel
has already weighted its slots) and the optional biases, on send layouts of
several shapes including the full 7168-wide hidden size."""

import numpy as np
import pytest
import torch

import oracle as O
from epgen import make_hidden, make_routing, spec
from tests.gpu_helpers import bits, gpu_available, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

import combine_ep_send_amd as ep  # noqa: E402


def _layout(T, H, E, K, P, routing="uniform", unrouted=0.0, seed=0):
    s = spec("tiny").replace(name="case", T=T, H=H, E=E, K=K, P=P, routing=routing,
                             unrouted_frac=unrouted, seed=seed)
    idx, w = make_routing(s)
    return idx, w, O.build_send_layout(idx, w, P, E // P)


def _rand_bf16(rng, shape):
    return (torch.from_numpy(rng.standard_normal(shape).astype(np.float32))
            .to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


@pytest.mark.parametrize("T,H,E,K,P,routing,unrouted", [
    (256, 512, 8, 2, 2, "uniform", 0.0),
    (1537, 1024, 256, 8, 32, "zipf", 0.05),
    (1000, 7168, 256, 8, 32, "uniform", 0.0),
    (300, 64, 16, 16, 4, "uniform", 0.1),
    (700, 256, 30, 5, 6, "uniform", 0.0),
    (300, 16384, 16, 4, 8, "uniform", 0.0),    # few rows per token (the sparse form), 3 chunks
    (400, 9216, 64, 8, 8, "zipf", 0.05),       # many rows per token, 2 ragged chunks
])
def test_partial_sums_and_biases(T, H, E, K, P, routing, unrouted):
    print(f"case: T={T} H={H} E={E} K={K} P={P}", flush=True)
    idx, w, (sti, srk, sidx, sw, trow) = _layout(T, H, E, K, P, routing, unrouted)
    rng = np.random.default_rng(T)
    y = _rand_bf16(rng, (len(sti), H))          # one partial output per send row
    b0, b1 = _rand_bf16(rng, (T, H)), _rand_bf16(rng, (T, H))
    d_y, d_trow, d_w = to_dev(y), to_dev(trow), to_dev(w)
    d_b0, d_b1 = to_dev(b0), to_dev(b1)
    got = bits(ep.ep_combine(d_y, d_trow, None))
    assert np.array_equal(got, O.combine_partials(y, trow))
    got = bits(ep.ep_combine(d_y, d_trow, None, bias=(d_b0, d_b1)))
    assert np.array_equal(got, O.combine_partials(y, trow, biases=(b0, b1)))
    got = bits(ep.ep_combine(d_y, d_trow, d_w, bias=d_b0))
    assert np.array_equal(got, O.combine(y, trow, w, biases=(b0,)))
    got = bits(ep.ep_combine(d_y, d_trow, d_w, bias=(d_b0, d_b1)))
    assert np.array_equal(got, O.combine(y, trow, w, biases=(b0, b1)))


def test_local_kernel_weights_then_partial_sums():
    """The torch_dispatch flow: the expert side weights and sums its slots of
    each send row (here an identity expert, in fp32), and the unweighted
    combine adds the partials; the result is the token within 2 bf16 ulp."""
    T, H, E, K, P = 2048, 256, 64, 6, 8
    idx, w, (sti, srk, sidx, sw, trow) = _layout(T, H, E, K, P)
    x = make_hidden(spec("tiny", T=T, H=H))
    xf = O.bf16_to_f32(x)
    part = (sw.sum(axis=1, dtype=np.float32)[:, None] * xf[sti]).astype(np.float32)
    y = O.f32_to_bf16(part)
    recv_x, recv_idx, recv_w, h = ep.dispatch(to_dev(x), to_dev(idx), to_dev(w),
                                              num_local_experts=E // P, num_ranks=P,
                                              num_send=T * min(K, P))
    got = bits(ep.combine(to_dev(y), h, weighted=False))
    ref = O.combine_partials(y, trow)
    assert np.array_equal(got, ref)
    of = O.bf16_to_f32(ref).astype(np.float64)
    exact = w.astype(np.float64).sum(axis=1)[:, None] * xf
    ulp = np.maximum(np.abs(exact), 2.0 ** -126) * 2.0 ** -7
    assert np.all(np.abs(of - exact) <= 2 * ulp)


def test_duplicate_rows_added_once_and_bias_only_tokens():
    rng = np.random.default_rng(9)
    H = 128
    y = _rand_bf16(rng, (6, H))
    trow = np.array([[3, 3, 5], [3, -1, 3], [-1, -1, -1], [0, 1, 2]], dtype=np.int32)
    b0 = _rand_bf16(rng, (4, H))
    got = bits(ep.ep_combine(to_dev(y), to_dev(trow), None, bias=to_dev(b0)))
    ref = O.combine_partials(y, trow, biases=(b0,))
    assert np.array_equal(got, ref)
    assert np.array_equal(got[2], b0[2])        # no rows: the bias itself


@pytest.mark.parametrize("T,H,E,K,P", [(1200, 7168, 256, 8, 32), (500, 1024, 64, 6, 8),
                                       (300, 4096, 16, 16, 4)])
def test_combine_launch_shapes_agree(T, H, E, K, P):
    """The same send rows combined as a buffer of exactly the send rows
    (R <= K*T: all of a token's rows loaded at once) and inside a larger
    padded buffer (R > K*T: rows walked one after another): both equal the
    oracle bit for bit, weighted and unweighted."""
    idx, w, (sti, _, _, _, trow) = _layout(T, H, E, K, P, "zipf", 0.05, seed=4)
    rng = np.random.default_rng(9)
    N = len(sti)
    y = _rand_bf16(rng, (N, H))
    want_w = O.combine(y, trow, w)
    want_u = O.combine_partials(y, trow)
    pad = K * T + 5 - N                       # rows past the send rows, never named
    assert pad > 0
    y_big = np.concatenate([y, _rand_bf16(rng, (pad, H))])
    print(f"case: launch shapes T={T} H={H} K={K} P={P} N={N} R={len(y_big)}", flush=True)
    d_trow, d_w = to_dev(trow), to_dev(w)
    for rows in (y, y_big):
        d_y = to_dev(rows)
        assert np.array_equal(bits(ep.ep_combine(d_y, d_trow, d_w)), want_w)
        assert np.array_equal(bits(ep.ep_combine(d_y, d_trow, None)), want_u)
