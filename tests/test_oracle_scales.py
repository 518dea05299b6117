"""Pins of the oracle's power-of-two and UE8M0 fp8 scales and of the
expert-batched fp8 layout, against definitions the oracle does not reuse:
the minimality of a power of two, torch's float8_e8m0fnu and float8_e4m3fn
conversions, a little-endian memory view for the packing, a hand-worked
example (tests/golden/fp8_scale_formats.*), and the gather of the
per-token quantized rows for the batched buffer."""

import json
import math
import os

import numpy as np
import torch

import oracle as O
from epgen import make_hidden, make_routing, spec

HERE = os.path.dirname(os.path.abspath(__file__))
with open(os.path.join(HERE, "golden", "fp8_scale_formats.json")) as f:
    SCALE_GOLDEN = json.load(f)


def _bf16_bits(values):
    return torch.from_numpy(np.asarray(values, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _torch_e4m3(values_f32):
    t = torch.from_numpy(np.ascontiguousarray(values_f32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_pow2_is_the_smallest_power_at_or_above():
    rng = np.random.default_rng(5)
    ex = rng.uniform(-149, 121, 4000)
    s = np.float32(np.exp2(ex))
    s = np.concatenate([s, np.float32(np.exp2(np.arange(-149, 121))),    # exact powers
                        np.float32([0.75, 1.0, 3.0, 1.0 + 2 ** -23, 2.0 ** -126 * 0.75])])
    p = O.round_scale_pow2(s).astype(np.float64)
    s64 = s.astype(np.float64)
    pos = s64 > 0
    assert np.all(np.frexp(p[pos])[0] == 0.5)                # a power of two
    assert np.all(p[pos] >= s64[pos])                         # at or above s
    assert np.all(p[pos] / 2 < s64[pos])                      # and the smallest such
    for v in (0.75, 3.0, 5.5, 1000.0, 1e-30):                 # the textbook form
        assert O.round_scale_pow2(np.float32([v]))[0] == np.float32(2.0 ** math.ceil(math.log2(v)))
    assert O.round_scale_pow2(np.float32([0.0]))[0] == 0.0


def test_ue8m0_bytes_match_torch_e8m0_on_powers_of_two():
    e = np.arange(-127, 128)
    p = np.float32(np.ldexp(1.0, e))
    b = O.ue8m0_encode(p)
    ref = torch.from_numpy(p).to(torch.float8_e8m0fnu).view(torch.uint8).numpy()
    assert np.array_equal(b, ref)
    codes = np.arange(255, dtype=np.uint8)
    ref_vals = torch.from_numpy(codes).view(torch.float8_e8m0fnu).float().numpy()
    assert np.array_equal(O.ue8m0_decode(codes), ref_vals)


def test_ue8m0_small_scales_clamp_to_the_lowest_code():
    p = np.float32([2.0 ** -128, 2.0 ** -141, 2.0 ** -149, 0.0])
    assert O.ue8m0_encode(p).tolist() == [0, 0, 0, 0]
    assert O.ue8m0_decode(np.uint8([0]))[0] == np.float32(2.0 ** -127)


def test_packing_is_a_little_endian_int_view():
    rng = np.random.default_rng(6)
    b = rng.integers(0, 255, size=(7, 3, 16), dtype=np.uint8)
    packed = O.pack_ue8m0(b)
    assert packed.shape == (7, 3, 4) and packed.dtype == np.int32
    assert np.array_equal(packed, np.ascontiguousarray(b).view("<i4"))
    assert np.array_equal(O.unpack_ue8m0(packed), b)


def _golden_rows():
    H = SCALE_GOLDEN["H"]
    rows = SCALE_GOLDEN["rows"]
    x = np.zeros((len(rows), H), dtype=np.float32)
    for i, r in enumerate(rows):
        for c, v in r["x"].items():
            x[i, int(c)] = v
    return _bf16_bits(x), rows


def test_scale_formats_hand_worked():
    bits, rows = _golden_rows()
    assert np.array_equal(O.bf16_to_f32(bits)[0, [0, 1, 2]], np.float32([3, -1, 41 / 4096]))
    q2, s2 = O.quantize_rows_fp8(bits, "pow2")
    q8, s8 = O.quantize_rows_fp8(bits, "ue8m0")
    for i, r in enumerate(rows):
        assert s2[i].tolist() == [np.float32(v) for v in r["pow2_scales"]]
        assert O.unpack_ue8m0(s8[i:i + 1])[0].tolist() == r["ue8m0_bytes"]
        assert s8[i].tolist() == r["ue8m0_packed"]
        for c, code in r["pow2_codes"].items():
            assert q2[i, int(c)] == code, (i, c)
        for c, code in r["ue8m0_codes"].items():
            assert q8[i, int(c)] == code, (i, c)
        rest = np.ones(bits.shape[1], bool)
        rest[[int(c) for c in r["x"]]] = False
        assert not q2[i, rest].any() and not q8[i, rest].any()


def test_pow2_and_ue8m0_codes_against_torch():
    s = spec("fp8_t32768", T=96, H=1024)
    x = make_hidden(s)
    xf = O.bf16_to_f32(x)
    x[3, 128:256] = 0                                    # an all-zero group
    # groups of tiny and huge magnitude, down to bf16 subnormals
    tiny = _bf16_bits(xf[4] * np.float32(2.0 ** -128))
    x[4] = tiny
    x[5] = _bf16_bits(xf[5] * np.float32(2.0 ** 100))
    xf = O.bf16_to_f32(x).reshape(96, 8, 128)
    amax = np.abs(xf).max(axis=2).astype(np.float64)
    q2, s2 = O.quantize_rows_fp8(x, "pow2")
    q8, p8 = O.quantize_rows_fp8(x, "ue8m0")
    b8 = O.unpack_ue8m0(p8)
    s8 = np.ldexp(1.0, b8.astype(np.int64) - 127)
    nz = amax > 0
    # every scale is a power of two that keeps the group within +-448
    assert np.all(s2[nz] * 448.0 >= amax[nz] * (1 - 2 ** -23))
    assert np.all(np.frexp(s2[nz].astype(np.float64))[0] == 0.5)
    assert np.all(s8[nz] >= s2[nz]) and np.all(b8[~nz] == 0) and np.all(s2[~nz] == 0)
    # where the power is in UE8M0's range the two formats agree exactly
    inrange = nz & (s2 >= np.float32(2.0 ** -127))
    assert inrange.sum() > 500 and (nz & ~inrange).sum() > 0
    assert np.array_equal(s8[inrange], s2[inrange].astype(np.float64))
    for q, sc in ((q2, s2.astype(np.float64)), (q8, s8)):
        qg = q.reshape(96, 8, 128)
        quot = (xf / np.where(nz, sc, 1.0)[:, :, None].astype(np.float32)).astype(np.float32)
        ref = _torch_e4m3(quot)
        assert np.array_equal(qg[nz], ref[nz])
        assert not qg[~nz].any()


def test_batched_fp8_is_the_gather_of_quantized_rows():
    s = spec("batched_t8192", T=300, H=512).replace(E=16, K=4, P=4)
    idx, _ = make_routing(s)
    x = make_hidden(s)
    first, El, M = 4, 4, 300
    b_x, tpe_ref, trow_ref = O.batched_prepare(x, idx, first, El, M)
    for fmt in O.SCALE_FORMATS:
        b_q, b_s, tpe, trow = O.batched_prepare_fp8(x, idx, first, El, M, fmt)
        assert np.array_equal(tpe, tpe_ref) and np.array_equal(trow, trow_ref)
        # quantizing the bf16 batched buffer (padding rows are zeros) gives the same
        q, sc = O.quantize_rows_fp8(b_x.reshape(El * M, -1), fmt)
        assert np.array_equal(b_q.reshape(El * M, -1), q)
        assert np.array_equal(b_s.reshape(El * M, -1).view(np.uint32), sc.view(np.uint32))
        # and each slot holds its token's quantized row (brute force over tokens)
        qt, st = O.quantize_rows_fp8(x, fmt)
        for e in range(El):
            toks = [t for t in range(idx.shape[0]) if (first + e) in idx[t].tolist()]
            assert tpe[e] == len(toks)
            for slot, t in enumerate(toks):
                assert np.array_equal(b_q[e, slot], qt[t])
                assert np.array_equal(b_s[e, slot].view(np.uint32), st[t].view(np.uint32))
            assert not b_q[e, len(toks):].any() and not b_s[e, len(toks):].any()


def test_scale_storage_orders():
    rng = np.random.default_rng(8)
    b = rng.standard_normal((3, 5, 4)).astype(np.float32)
    flat_c = O.scale_storage(b, True)
    flat_r = O.scale_storage(b, False)
    E, M, G = b.shape
    for e in range(E):
        for s_ in range(M):
            for g in range(G):
                assert flat_c[e * M * G + g * M + s_] == b[e, s_, g]
                assert flat_r[e * M * G + s_ * G + g] == b[e, s_, g]
