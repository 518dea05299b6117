"""GPU parity of ep_batched_prepare_fp8 (the expert-batched layout with e4m3
rows and float, power-of-two or packed UE8M0 scales, stored row- or
column-major) against the CPU oracle, bit for bit: codes, scale words,
counts, token_row and the zero padding."""

import numpy as np
import pytest
import torch

import oracle as O
from epgen import make_hidden, make_routing, spec
from tests.gpu_helpers import host, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

import combine_ep_send_amd as ep  # noqa: E402

FORMATS = ["f32", "pow2", "ue8m0"]


def _inputs(T, H, E, K, P, routing="uniform", unrouted=0.0, seed=0, extremes=True):
    s = spec("batched_t8192").replace(name="case", T=T, H=H, E=E, K=K, P=P, routing=routing,
                                      unrouted_frac=unrouted, seed=seed)
    idx, _ = make_routing(s)
    x = make_hidden(s)
    if extremes and T > 8:
        # rows whose scales are float32 subnormals (UE8M0 clamps them to
        # 2^-127), huge rows, and rows with all-zero groups
        f = O.bf16_to_f32(x)
        for t, mul in ((1, 2.0 ** -128), (3, 2.0 ** -120), (5, 2.0 ** 100)):
            x[t] = torch.from_numpy(f[t] * np.float32(mul)).to(torch.bfloat16) \
                .view(torch.int16).numpy().view(np.uint16)
        x[7, : H // 2] = 0
    return idx, x


def _scale_words(b_scale, fmt):
    """Host copy of the GPU scale tensor in logical [E_local, max, units]
    order, as uint32 words."""
    a = b_scale.cpu().numpy()            # a strided view keeps logical order
    return np.ascontiguousarray(a).view(np.uint32)


def _check(idx, x, first, El, M, fmt, col_major, sentinel=True):
    T, H = x.shape
    d_idx, d_x = to_dev(idx), to_dev(x)
    out = torch.empty((El, M, H), dtype=torch.uint8, device="cuda")
    if sentinel:
        out.fill_(0x5A)
    out = out.view(torch.float8_e4m3fn)
    sc = ep.batched_scale_like(El, M, H, fmt, col_major, "cuda")
    if sentinel:
        sc.view(torch.int32).fill_(0x3F3F3F3F) if sc.dtype == torch.float32 else sc.fill_(-77)
    q, s_, tpe, trow = ep.ep_batched_prepare_fp8(d_x, d_idx, first, El, M, scale_fmt=fmt,
                                                 scale_col_major=col_major, out=out,
                                                 out_scale=sc)
    # the strides of the scale tensor are the memory layout the caller asked for
    units = H // (512 if fmt == "ue8m0" else 128)
    if s_.numel():
        assert s_.stride() == ((M * units, 1, M) if col_major else (M * units, units, 1))
    M_big = max(M, T)
    oq, osc, otpe, otrow = O.batched_prepare_fp8(x, idx, first, El, M_big, fmt)
    assert np.array_equal(host(tpe), otpe)
    e_of, slot_of = otrow // M_big, otrow % M_big
    want_trow = np.where((otrow >= 0) & (slot_of < M), e_of * M + slot_of, -1)
    assert np.array_equal(host(trow), want_trow)
    gq = host(q)
    gs = _scale_words(s_, fmt)
    want_q = oq[:, :M]
    want_s = np.ascontiguousarray(osc[:, :M]).view(np.uint32)
    assert np.array_equal(gq, want_q)
    assert np.array_equal(gs, want_s)
    # the flat memory order is the oracle's storage order
    flat = torch.as_strided(s_, (s_.numel(),), (1,)).cpu().numpy().view(np.uint32)
    assert np.array_equal(flat, O.scale_storage(osc[:, :M], col_major).view(np.uint32))
    return otpe


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("col_major", [False, True])
@pytest.mark.parametrize("T,H,E,K,P,first_rank,M", [
    (300, 512, 16, 4, 4, 1, 300),        # small, several tiles
    (2000, 1536, 64, 6, 8, 3, 256),       # K = 6, ragged chunk of a row
    (700, 7168, 256, 8, 8, 0, 256),       # the batched workload's row and expert shape
])
def test_batched_fp8_matches_oracle(fmt, col_major, T, H, E, K, P, first_rank, M):
    print(f"case: fmt={fmt} col_major={col_major} T={T} H={H} E={E} K={K}", flush=True)
    idx, x = _inputs(T, H, E, K, P)
    El = E // P
    tpe = _check(idx, x, first_rank * El, El, M, fmt, col_major)
    assert tpe.max() <= M


@pytest.mark.parametrize("fmt", FORMATS)
def test_batched_fp8_overflow_drops_slots(fmt):
    idx, x = _inputs(1500, 512, 16, 4, 2)
    tpe = _check(idx, x, 8, 8, 100, fmt, fmt == "ue8m0")
    assert tpe.max() > 100                 # true counts reported past max


def test_batched_fp8_edge_cases():
    # no tokens: counts are zeros and every slot is padding
    for fmt in FORMATS:
        _check(np.zeros((0, 4), np.int64), np.zeros((0, 512), np.uint16), 0, 4, 16, fmt, True)
    # no local tokens at all, and a single token
    idx, x = _inputs(64, 512, 16, 2, 4, extremes=False)
    _check(np.full_like(idx, -1), x, 0, 4, 8, "ue8m0", False)
    _check(idx[:1], x[:1], 0, 16, 1, "pow2", True)
    # max_num_tokens = 0: nothing to write
    _check(idx, x, 0, 4, 0, "f32", True)


def test_batched_fp8_rejects_bad_arguments():
    idx, x = _inputs(32, 640, 10, 2, 2, extremes=False)
    d_idx, d_x = to_dev(idx), to_dev(x)
    with pytest.raises(ValueError):          # UE8M0 packs 512 channels per word
        ep.ep_batched_prepare_fp8(d_x, d_idx, 0, 5, 32, scale_fmt="ue8m0")
    with pytest.raises(ValueError):
        ep.ep_batched_prepare_fp8(d_x, d_idx, 0, 5, 32, scale_fmt="e5m2")
    wrong = ep.batched_scale_like(5, 32, 640, "f32", False, "cuda")
    with pytest.raises(ValueError):          # row-major tensor for a column-major call
        ep.ep_batched_prepare_fp8(d_x, d_idx, 0, 5, 32, scale_col_major=True, out_scale=wrong)


def test_batched_fp8_workload_full_size():
    """The batched fp8 workload as the bench times it (T=8192, E_local=32,
    max 8192, H=7168, UE8M0 scales stored column-major), compared with the
    oracle element by element: counts, token_row, every code of the
    [E_local, max, H] buffer (padding included) and every scale word in
    memory order."""
    s = spec("batched_fp8_t8192")
    print(f"case: full-size batched_fp8_t8192 T={s.T} H={s.H} E_local={s.E_local} "
          f"max={s.max_num_tokens} {s.scale_fmt} col_major={s.scale_col_major}", flush=True)
    idx, _ = make_routing(s)
    x = make_hidden(s)
    T, H, El, M, first = s.T, s.H, s.E_local, s.max_num_tokens, s.first_expert
    q, sc, tpe, trow = ep.ep_batched_prepare_fp8(to_dev(x), to_dev(idx), first, El, M,
                                                 scale_fmt=s.scale_fmt,
                                                 scale_col_major=s.scale_col_major)
    torch.cuda.synchronize()
    ep.check_workspaces()
    oq, osc, otpe, otrow = O.batched_prepare_fp8(x, idx, first, El, M, s.scale_fmt)
    assert np.array_equal(host(tpe), otpe)
    assert np.array_equal(host(trow), otrow)
    for e in range(El):
        assert np.array_equal(q[e].view(torch.uint8).cpu().numpy(), oq[e]), e
    # the scale tensor's memory, in order, against the oracle's storage order
    flat = torch.as_strided(sc, (sc.numel(),), (1,)).cpu().numpy().view(np.uint32)
    assert np.array_equal(flat, O.scale_storage(osc, s.scale_col_major).view(np.uint32))
