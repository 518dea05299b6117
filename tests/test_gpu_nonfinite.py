"""GPU parity on non-finite inputs, which the pages leave open (the readings
are pinned on the CPU in test_oracle_nonfinite.py): the combine's sums that
overflow, meet infinities of both signs or NaNs (quiet and signalling, both
signs, in the rows and in the weights), in the dense and the sparse form,
weighted and unweighted; the fp8 permute and the expert-batched fp8 layout
on rows holding NaNs, infinities and groups of NaNs only, in every scale
format.  Everything bit for bit against the oracle, except that any two
NaNs of the combine match (their sign and payload are left open)."""

import numpy as np
import pytest
import torch

import oracle as O
from tests.gpu_helpers import bits, host, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

import combine_ep_send_amd as ep  # noqa: E402

SPECIALS = np.uint16([0x7FC0, 0xFFC0, 0x7F81, 0xFF81, 0x7FFF,      # NaNs
                      0x7F80, 0xFF80,                              # infinities
                      0x7F7F, 0xFF7F, 0x7F70])                      # near the largest bf16


def _same_bf16(got, want):
    """Bit for bit, except that any two NaNs match (a NaN's sign and payload
    after arithmetic are not specified)."""
    nan_g = (got & 0x7FFF) > 0x7F80
    nan_w = (want & 0x7FFF) > 0x7F80
    return np.array_equal(nan_g, nan_w) and np.array_equal(got[~nan_g], want[~nan_w])


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _rows_with_specials(R, H, seed, frac=0.02):
    r = np.random.default_rng(seed)
    y = _bf16(r.standard_normal((R, H)))
    flat = y.reshape(-1)
    pos = r.choice(flat.size, int(frac * flat.size), replace=False)
    flat[pos] = SPECIALS[r.integers(0, len(SPECIALS), len(pos))]
    return y


def _routing(T, K, R, seed, dense):
    r = np.random.default_rng(seed)
    if dense:
        row = r.integers(0, R, (T, K)).astype(np.int32)
    else:                                   # about one row per token
        row = np.full((T, K), -1, np.int32)
        row[:, 0] = r.permutation(R)[:T]
        extra = r.random(T) < 0.2
        row[extra, 1] = r.integers(0, R, int(extra.sum()))
    row[r.random((T, K)) < 0.1] = -1
    return row


# products and sums that overflow to infinity or meet inf - inf are the point
# of this test: numpy's warnings about them say nothing here
@pytest.mark.filterwarnings("ignore:overflow encountered:RuntimeWarning")
@pytest.mark.filterwarnings("ignore:invalid value encountered:RuntimeWarning")
@pytest.mark.parametrize("dense", [True, False])
def test_combine_nonfinite(dense):
    T, K, H = 300, 4, 1024
    R = 3 * T if dense else T               # dense form reads >= 2 rows per token
    y = _rows_with_specials(R, H, 5)
    row = _routing(T, K, R, 6, dense)
    r = np.random.default_rng(7)
    w = r.random((T, K)).astype(np.float32) + np.float32(0.5)
    w.reshape(-1)[r.choice(T * K, 40, replace=False)] = \
        np.float32([np.nan, np.inf, -np.inf, 0.0])[r.integers(0, 4, 40)]
    big = np.where(r.random((T, K)) < 0.05, np.float32(3e38), np.float32(1.0))
    w = (w * big).astype(np.float32)        # products that overflow
    print(f"case: combine non-finite dense={dense} T={T} K={K} H={H} R={R}", flush=True)
    d_y, d_row, d_w = to_dev(y), to_dev(row), to_dev(w)
    got = bits(ep.ep_combine(d_y, d_row, d_w))
    assert _same_bf16(got, O.combine(y, row, w))
    got = bits(ep.ep_combine(d_y, d_row, None))
    assert _same_bf16(got, O.combine_partials(y, row))
    assert ((got & 0x7FFF) > 0x7F80).any() and (got == 0x7F80).any() and (got == 0xFF80).any()


def _fp8_rows(T, H, seed):
    x = _rows_with_specials(T, H, seed, frac=0.01)
    x[3, 128:256] = 0x7FC0                  # a group of NaNs only
    x[4, :64] = 0xFF81                      # NaNs and zeros
    x[4, 64:128] = 0
    x[5, 300] = 0x7F80                      # an infinity with finite neighbours
    x[6, 700] = 0xFF80
    return x


def test_fp8_permute_nonfinite():
    T, H, K, P, El = 200, 1024, 4, 4, 2
    x = _fp8_rows(T, H, 8)
    r = np.random.default_rng(9)
    idx = np.stack([r.permutation(P * El)[:K] for _ in range(T)]).astype(np.int64)
    w = np.full((T, K), 0.25, np.float32)
    print(f"case: fp8 permute non-finite T={T} H={H}", flush=True)
    cap = T * min(K, P)
    _, lay = ep.ep_dispatch_layout(to_dev(idx), to_dev(w), P, El, cap)
    q, sc = ep.ep_dispatch_permute(to_dev(x), lay.token_row, cap, fp8=True)
    sti = O.build_send_layout(idx, w, P, El)[0]
    oq, osc = O.dispatch_permute_fp8(x, sti)
    N = len(sti)
    assert np.array_equal(host(q)[:N], oq)
    assert np.array_equal(host(sc)[:N].view(np.uint32), osc.view(np.uint32))
    assert (oq == 0x7F).any() and np.isinf(osc).any()


@pytest.mark.parametrize("fmt", ["f32", "pow2", "ue8m0"])
def test_batched_fp8_nonfinite(fmt):
    T, H, K, El, M = 150, 1024, 3, 4, 160
    x = _fp8_rows(T, H, 10)
    r = np.random.default_rng(11)
    idx = np.stack([r.permutation(16)[:K] for _ in range(T)]).astype(np.int64)
    print(f"case: batched fp8 non-finite fmt={fmt} T={T} H={H}", flush=True)
    bq, bs, tpe, _ = ep.ep_batched_prepare_fp8(to_dev(x), to_dev(idx), 0, El, M, scale_fmt=fmt,
                                               scale_col_major=fmt == "ue8m0")
    oq, osc, otpe, _ = O.batched_prepare_fp8(x, idx, 0, El, M, fmt)
    assert np.array_equal(host(tpe), otpe)
    assert np.array_equal(host(bq), oq)
    flat = torch.as_strided(bs, (bs.numel(),), (1,)).cpu().numpy().view(np.uint32)
    assert np.array_equal(flat, O.scale_storage(osc, fmt == "ue8m0").view(np.uint32))
