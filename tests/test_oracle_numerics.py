"""Pins for the oracle's number formats (bf16, OCP e4m3), the fp8
quantize-on-dispatch rule and the weighted combine.  Expectations come from
library conversions (torch bf16 / float8_e4m3fn), the format definitions,
exact float64 arithmetic, closed forms and the hand-worked example."""

import numpy as np
import pytest
import torch

import oracle as O
from epgen import balanced_routing, make_routing, make_hidden, spec


def torch_bf16_bits(f32):
    return (torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32))
            .to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def bf16_ulp(v):
    """Spacing of bf16 values at |v| (float64)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126)
    return 2.0 ** (e - 7)


# --------------------------------------------------------------------------
# bf16
# --------------------------------------------------------------------------

def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(50000) * 1e-38).astype(np.float32),
        (rng.standard_normal(50000) * 1e30).astype(np.float32),
        rng.integers(0, 1 << 32, 200000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    vals = vals[np.isfinite(vals) & (np.abs(vals) < 3.38e38)]
    # exact halfway cases, both parities of the kept LSB
    base = rng.integers(0, 0x7F00, 20000, dtype=np.uint32) << 16
    halves = (base | np.uint32(0x8000)).view(np.float32)
    vals = np.concatenate([vals, halves, -halves, np.float32([0.0, -0.0])])
    assert np.array_equal(O.f32_to_bf16(vals), torch_bf16_bits(vals))


def test_bf16_roundtrip_exact():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = O.bf16_to_f32(bits)
    finite = np.isfinite(f)
    assert np.array_equal(O.f32_to_bf16(f[finite]), bits[finite])
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(f[finite], t[finite])


# --------------------------------------------------------------------------
# e4m3 (OCP, float8_e4m3fn)
# --------------------------------------------------------------------------

def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    mine = O.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert O.e4m3_decode(0x7E) == 448.0 and np.isnan(O.e4m3_decode(0x7F))


def test_e4m3_encode_reencodes_every_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = O.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(O.e4m3_encode(vals), codes)


def test_e4m3_encode_matches_torch():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.uniform(-448, 448, 300000),
        rng.standard_normal(200000) * 2.0 ** rng.integers(-12, 8, 200000),
    ]).astype(np.float32)
    # all midpoints between neighbouring codes (ties) and their neighbours
    pos = O.e4m3_decode(np.arange(0x7F)).astype(np.float64)
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    vals = np.concatenate([vals, mids, -mids, up, -up, dn, -dn])
    vals = vals[np.abs(vals) <= 448]
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(vals), ref)


def test_e4m3_saturates_and_keeps_sign():
    v = np.float32([448.0, 449.0, 464.0, 1e6, 3.0e38, -500.0, -0.0, -1e-9, 1e-9])
    assert O.e4m3_encode(v).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x80, 0x00]


def test_e4m3_hand_cases(golden):
    for val, code in golden["fp8"]["encode_cases"]:
        assert int(O.e4m3_encode(np.float32([val]))[0]) == code, val


# --------------------------------------------------------------------------
# fp8 quantize-on-dispatch
# --------------------------------------------------------------------------

def test_quantize_hand_row(golden):
    r = golden["fp8"]["row_amax448"]
    x = np.zeros((1, 256), dtype=np.float32)
    x[0, :4] = r["x_first4"]
    x[0, 128] = 2.0                                  # second group: amax 2
    bits = torch_bf16_bits(x)
    q, s = O.quantize_rows_fp8(bits)
    assert s[0, 0] == np.float32(r["scale"])
    assert q[0, :4].tolist() == r["codes_first4"]
    assert not q[0, 4:128].any()
    assert s[0, 1] == np.float32(2.0) / np.float32(448.0)
    assert q[0, 128] == 0x7E


def test_quantize_properties():
    s = spec("fp8_t32768", T=64, H=1024)
    x = make_hidden(s)
    x[3, 128:256] = 0                               # an all-zero group
    x[5, 0:128] = 0x8000                            # an all -0.0 group
    q, sc = O.quantize_rows_fp8(x)
    xf = O.bf16_to_f32(x).reshape(64, 8, 128).astype(np.float64)
    amax = np.abs(xf).max(axis=2)
    assert np.array_equal(sc, (amax.astype(np.float32) / np.float32(448)).astype(np.float32))
    assert sc[3, 1] == 0 and not q[3, 128:256].any()
    assert sc[5, 0] == 0 and not q[5, 0:128].any()
    deq = O.e4m3_decode(q).reshape(64, 8, 128) * sc[:, :, None].astype(np.float64)
    nz = sc > 0
    # the max-|x| element of each nonzero group encodes to +-448
    qg = q.reshape(64, 8, 128)
    am = np.abs(xf).argmax(axis=2)
    top = np.take_along_axis(qg, am[:, :, None], axis=2)[:, :, 0]
    assert np.all((top[nz] & 0x7F) == 0x7E)
    # relative error <= 2^-4 in the normal range, <= 2^-10 * scale below it
    err = np.abs(deq - xf)
    normal = np.abs(xf) / sc[:, :, None].astype(np.float64).clip(1e-300) >= 2.0 ** -6
    bound = np.where(normal, 2.0 ** -4 * np.abs(xf), 2.0 ** -10 * sc[:, :, None])
    assert np.all(err[nz] <= bound[nz] * (1 + 1e-6))


# --------------------------------------------------------------------------
# combine
# --------------------------------------------------------------------------

def test_combine_identity_round_trip_within_1ulp():
    s = spec("skewed_t16384", T=512, H=256)
    idx, w = make_routing(s)
    x = make_hidden(s)
    sti, srk, sidx, sw, trow = O.build_send_layout(idx, w, s.P, s.E_local)
    sx = O.dispatch_permute(x, sti)
    out = O.combine(sx, trow, w)
    xf = O.bf16_to_f32(x).astype(np.float64)
    of = O.bf16_to_f32(out).astype(np.float64)
    routed = (idx >= 0).any(axis=1)
    wsum = w.astype(np.float64).sum(axis=1)
    # exact value is wsum * x; rounding in fp32 then bf16 stays within 1 ulp
    exact = wsum[:, None] * xf
    assert np.all(np.abs(of - exact)[routed] <= bf16_ulp(exact)[routed])
    assert not out[~routed].any()


def test_combine_within_1ulp_of_exact_sum():
    rng = np.random.default_rng(3)
    T, K, H, R = 300, 8, 64, 900
    y = torch_bf16_bits(rng.standard_normal((R, H)).astype(np.float32))
    row = rng.integers(-1, R, size=(T, K)).astype(np.int32)
    w = rng.random((T, K)).astype(np.float32)
    out = O.combine(y, row, w)
    yf = O.bf16_to_f32(y).astype(np.float64)
    exact = np.zeros((T, H))
    for k in range(K):
        m = row[:, k] >= 0
        exact[m] += w[m, k].astype(np.float64)[:, None] * yf[row[m, k]]
    of = O.bf16_to_f32(out).astype(np.float64)
    # fp32 accumulation error is ~K * 2^-24 relative to sum |terms|; allow 1 bf16
    # ulp of the exact value plus that slack (cancellation can shrink |exact|)
    mag = np.zeros((T, H))
    for k in range(K):
        m = row[:, k] >= 0
        mag[m] += np.abs(w[m, k].astype(np.float64)[:, None] * yf[row[m, k]])
    assert np.all(np.abs(of - exact) <= bf16_ulp(exact) + K * 2.0 ** -23 * mag)


def test_combine_k1_weight1_is_copy_and_unrouted_is_zero():
    rng = np.random.default_rng(4)
    y = rng.integers(0, 0x7F00, size=(10, 32), dtype=np.uint16)   # finite positives
    row = np.array([[3], [-1], [0], [9]], dtype=np.int32)
    w = np.ones((4, 1), dtype=np.float32)
    out = O.combine(y, row, w)
    assert np.array_equal(out[0], y[3]) and np.array_equal(out[2], y[0])
    assert np.array_equal(out[3], y[9])
    assert not out[1].any()


def test_combine_balanced_power_of_two_weights_exact():
    # uniform weights 1/K with K a power of two: every product and partial sum
    # of a bf16 value is exact in fp32, so the identity round trip is bit-exact
    T, K, E, P = 256, 8, 64, 8
    idx, w = balanced_routing(T, K, E)
    x = make_hidden(spec("tiny", T=T, H=64))
    sti, srk, sidx, sw, trow = O.build_send_layout(idx, w, P, E // P)
    out = O.combine(O.dispatch_permute(x, sti), trow, w)
    # equal as values: a -0.0 input returns +0.0 because the sum starts at +0.0
    assert np.array_equal(O.bf16_to_f32(out), O.bf16_to_f32(x))
    assert np.all(out[x == 0x8000] == 0)


def test_combine_order_is_k_ascending():
    # products 1+2^-8, 2^-24, 2^-24 (fp32).  k ascending: 1+2^-8 absorbs each
    # 2^-24 (a tie that keeps the even mantissa), and bf16(1+2^-8) is a tie that
    # rounds to 1.0.  Any other order first forms 2^-23, giving 1+2^-8+2^-23,
    # which rounds up to bf16 1.0078125.
    y = torch_bf16_bits(np.float32([[1.0]]))
    row = np.zeros((1, 3), dtype=np.int32)
    w = np.float32([[1.0 + 2.0 ** -8, 2.0 ** -24, 2.0 ** -24]])
    assert O.bf16_to_f32(O.combine(y, row, w))[0, 0] == 1.0
    assert O.bf16_to_f32(O.combine(y, row, w[:, ::-1].copy()))[0, 0] == 1.0078125


def test_combine_rounds_product_before_sum():
    # slot 0 adds 1 * (1 + 2^-8).  Slot 1 multiplies y = 2^-24 (1 + 2^-4) by
    # w = 1 - a + a^2 - ... + a^6 with a = 2^-4 (24 significant bits, so w is
    # an fp32 value); the exact product is 2^-24 (1 + a^7) = 2^-24 + 2^-52.
    # Rounded to fp32 first, that product is 2^-24, and 1 + 2^-8 + 2^-24 is an
    # fp32 tie that keeps 1 + 2^-8, itself a bf16 tie that gives 1.0.  A fused
    # multiply-add (or a wider accumulator) keeps the 2^-52, lands above the
    # tie at 1 + 2^-8 + 2^-23 and rounds to bf16 1.0078125.
    a = 2.0 ** -4
    w1 = sum((-a) ** i for i in range(7))
    assert float(np.float32(w1)) == w1
    prod = (2.0 ** -24 * (1 + a)) * w1
    assert prod == 2.0 ** -24 + 2.0 ** -52                 # exact in float64
    y = torch_bf16_bits(np.float32([[1.0], [2.0 ** -24 * (1 + a)]]))
    row = np.array([[0, 1]], dtype=np.int32)
    w = np.float32([[1 + 2.0 ** -8, w1]])
    assert O.bf16_to_f32(O.combine(y, row, w))[0, 0] == 1.0


def test_combine_hand_worked(golden):
    g, ex = golden, golden["expected"]
    x = torch_bf16_bits(np.array(g["x"], dtype=np.float32))
    w = np.array(g["topk_weights"], dtype=np.float32)
    trow = np.array(ex["token_row"], dtype=np.int32)
    sx = x[ex["send_token_idx"]]
    out = O.combine(sx, trow, w)
    assert np.array_equal(O.bf16_to_f32(out), np.array(ex["combine_identity"], np.float32))
    yc = torch_bf16_bits(np.repeat(np.arange(1, 10, dtype=np.float32)[:, None], 8, axis=1))
    outc = O.bf16_to_f32(O.combine(yc, trow, w))
    assert np.array_equal(outc, np.repeat(np.float32(ex["combine_rowconst"])[:, None], 8, axis=1))
    b = ex["batched"]
    idx = np.array(g["topk_idx"], dtype=np.int64)
    bx, tpe, btr = O.batched_prepare(x, idx, b["first_expert"], b["E_local"], b["max_num_tokens"])
    outb = O.bf16_to_f32(O.combine(bx.reshape(-1, 8), btr, w))
    want = np.float32(b["combine_identity_scale"])[:, None] * O.bf16_to_f32(x)
    assert np.array_equal(outb, want)


# --------------------------------------------------------------------------
# unweighted per-destination partial sums, and combine biases
# --------------------------------------------------------------------------

def test_combine_partials_counts_each_destination_once():
    # slots 0 and 1 share destination row 3, slot 2 is row 5: the partial of
    # row 3 is added once, not twice (each destination sends one partial)
    y = torch_bf16_bits(np.float32([[0.0], [0.0], [0.0], [1.5], [0.0], [0.25]]))
    row = np.array([[3, 3, 5], [3, -1, 3], [-1, -1, -1]], dtype=np.int32)
    out = O.bf16_to_f32(O.combine_partials(y, row))
    assert out[:, 0].tolist() == [1.75, 1.5, 0.0]


def test_combine_partials_within_1ulp_of_exact_sum():
    rng = np.random.default_rng(6)
    T, K, H, R = 200, 8, 32, 64
    y = torch_bf16_bits(rng.standard_normal((R, H)).astype(np.float32))
    row = rng.integers(-1, R, size=(T, K)).astype(np.int32)
    out = O.bf16_to_f32(O.combine_partials(y, row)).astype(np.float64)
    yf = O.bf16_to_f32(y).astype(np.float64)
    exact = np.zeros((T, H))
    mag = np.zeros((T, H))
    for t in range(T):
        for r in set(int(v) for v in row[t] if v >= 0):      # a set: distinct rows
            exact[t] += yf[r]
            mag[t] += np.abs(yf[r])
    assert np.all(np.abs(out - exact) <= bf16_ulp(exact) + K * 2.0 ** -23 * mag)


def test_combine_partials_single_destination_is_copy():
    s = spec("tiny", T=300, H=64, P=1, E=8, K=2)
    idx, w = make_routing(s)
    x = make_hidden(s)
    sti, srk, sidx, sw, trow = O.build_send_layout(idx, w, 1, 8)
    out = O.combine_partials(O.dispatch_permute(x, sti), trow)
    # one destination: every routed token's only row is its own hidden row
    # (values compare equal; -0.0 comes back +0.0 since the sum starts at +0.0)
    assert np.array_equal(O.bf16_to_f32(out), O.bf16_to_f32(x))


def test_combine_biases_are_added():
    # small integers: every sum is exact, so the result is the plain sum
    y = torch_bf16_bits(np.float32([[1.0, 2.0], [4.0, 8.0]]))
    row = np.array([[0, 1], [-1, -1]], dtype=np.int32)
    w = np.float32([[1.0, 2.0], [0.0, 0.0]])
    b0 = torch_bf16_bits(np.float32([[16.0, -32.0], [3.0, 5.0]]))
    b1 = torch_bf16_bits(np.float32([[64.0, 1.0], [-7.0, 0.5]]))
    got = O.bf16_to_f32(O.combine(y, row, w, biases=(b0,)))
    assert got.tolist() == [[1 + 8 + 16, 2 + 16 - 32], [3, 5]]
    got = O.bf16_to_f32(O.combine(y, row, w, biases=(b0, b1)))
    assert got.tolist() == [[1 + 8 + 16 + 64, 2 + 16 - 32 + 1], [-4, 5.5]]
    got = O.bf16_to_f32(O.combine_partials(y, row, biases=(b0, b1)))
    assert got.tolist() == [[1 + 4 + 16 + 64, 2 + 8 - 32 + 1], [-4, 5.5]]
    # a token with no slot returns the bias bit for bit
    assert np.array_equal(O.combine(y, row, w, biases=(b0,))[1], b0[1])
