"""Pins for the oracle's fp8 row helpers: the dequantized rows an identity
expert hands to combine (``dequantize_rows_fp8``) and the quantize-on-dispatch
send rows (``dispatch_permute_fp8``).

NeMo "uccl_ep.buffer", Buffer.dispatch: fp8 input is a tuple of e4m3 rows
[.., H] and one float scale per token per 128 channels [.., H/128].  The
expected values come from torch's ``float8_e4m3fn`` decode, IEEE float32
multiplication and torch's bf16 conversion, from a row worked by hand from
the OCP E4M3 and bf16 definitions, and from a brute-force loop that
quantizes each send row on its own."""

import numpy as np
import torch

import oracle as O
from epgen import make_hidden, make_routing, spec


def torch_dequant_bits(q, scales):
    """bf16 bits of fl32(decode(q) * scale), every step a torch operation:
    the e4m3 decode (exact in float32), a float32 multiply by the scale of
    the element's 128-channel group, and the bf16 conversion."""
    R, H = q.shape
    vals = torch.from_numpy(np.ascontiguousarray(q, dtype=np.uint8)).view(torch.float8_e4m3fn)
    vals = vals.to(torch.float32).reshape(R, H // 128, 128)
    sc = torch.from_numpy(np.ascontiguousarray(scales, dtype=np.float32)).reshape(R, H // 128, 1)
    prod = (vals * sc).reshape(R, H)
    return prod.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def same_bits_nan_equal(a, b):
    a = np.asarray(a, dtype=np.uint16)
    b = np.asarray(b, dtype=np.uint16)
    nan_a = (a & 0x7FFF) > 0x7F80
    nan_b = (b & 0x7FFF) > 0x7F80
    return np.array_equal(nan_a, nan_b) and np.array_equal(a[~nan_a], b[~nan_b])


def test_dequantize_matches_torch_decode_times_scale():
    # every code in every group, under scales that are exact, inexact,
    # tiny (products in the subnormal range or flushing to zero), huge
    # (products past the largest bf16) and zero; each group its own scale
    codes = np.arange(256, dtype=np.uint8)
    group_scales = np.float32([1.0, 3.0, 1.0 / 3.0, 0.1, 2.0 ** -130, 1e-45, 3.0e36, 7.25e35,
                               0.0, 1.7e-3, 448.0 / 3.0, 2.0 ** 100])
    rows = []
    for r in range(3):
        rng = np.random.default_rng(r)
        rows.append(np.concatenate([rng.permutation(codes) for _ in range(len(group_scales) // 2)]))
    q = np.stack(rows)                                   # [3, 12 * 128]
    scales = np.stack([np.roll(group_scales, r) for r in range(3)])
    with np.errstate(over="ignore"):             # products past float32 become infinities
        got = O.dequantize_rows_fp8(q, scales)
    ref = torch_dequant_bits(q, scales)
    assert got.shape == q.shape and got.dtype == np.uint16
    assert same_bits_nan_equal(got, ref)


def test_dequantize_random_rows_match_torch():
    s = spec("fp8_t32768", T=96, H=1024)
    q, sc = O.quantize_rows_fp8(make_hidden(s))
    assert same_bits_nan_equal(O.dequantize_rows_fp8(q, sc), torch_dequant_bits(q, sc))


def test_dequantize_hand_row():
    # OCP E4M3, bias 7: 0x38 = 0.0111.000 = 2^0 = 1; 0x40 = 0.1000.000 = 2;
    # 0xB8 = -1; 0x01 = subnormal 1/8 * 2^-6 = 2^-9; 0x7E = 0.1111.110 =
    # 1.75 * 2^8 = 448; 0x80 = -0.  Group 0 is scaled by 3, group 1 by 0.5.
    # bf16 (1 sign, 8 exponent bits with bias 127, 7 mantissa bits):
    #   3 = 1.5 * 2^1        -> 0 10000000 1000000 = 0x4040
    #   6 = 1.5 * 2^2        -> 0 10000001 1000000 = 0x40C0
    #  -3                    -> 0xC040
    #   3 * 2^-9 = 1.5*2^-8  -> 0 01110111 1000000 = 0x3BC0
    #   448 * 0.5 = 224 = 1.75 * 2^7 -> 0 10000110 1100000 = 0x4360
    #  -0 * 0.5 = -0         -> 0x8000
    q = np.zeros((1, 256), dtype=np.uint8)
    q[0, :4] = [0x38, 0x40, 0xB8, 0x01]
    q[0, 128:130] = [0x7E, 0x80]
    out = O.dequantize_rows_fp8(q, np.float32([[3.0, 0.5]]))
    assert out[0, :4].tolist() == [0x4040, 0x40C0, 0xC040, 0x3BC0]
    assert out[0, 128:130].tolist() == [0x4360, 0x8000]
    assert not out[0, 4:128].any() and not out[0, 130:].any()


def test_dequantize_rounds_the_float32_product_once_to_bf16():
    # 0x3F = 0.0111.111 = 1.875; scale 1 + 3 * 2^-9 = 1.005859375 (a float32
    # exactly).  Product 1.885986328125 = 241.40625 bf16 steps of 2^-7 above
    # 0: rounds down to 1.8828125 = 1 + 113/128 -> 0x3FF1.  A scale first
    # rounded to bf16 (1.0078125) would give 1.8896484375 = 241.875 steps ->
    # 1.890625 -> 0x3FF2.
    q = np.full((1, 128), 0x3F, dtype=np.uint8)
    sc = np.float32([[1.005859375]])
    out = O.dequantize_rows_fp8(q, sc)
    assert (out == 0x3FF1).all()
    assert same_bits_nan_equal(out, torch_dequant_bits(q, sc))


def _brute_force_permute_fp8(x_bits, send_token_idx):
    """Row by row: send row n is the quantized hidden row of token
    send_token_idx[n], quantized on its own."""
    H = x_bits.shape[1]
    q = np.zeros((len(send_token_idx), H), dtype=np.uint8)
    sc = np.zeros((len(send_token_idx), H // 128), dtype=np.float32)
    for n, t in enumerate(send_token_idx):
        qn, sn = O.quantize_rows_fp8(x_bits[int(t)][None, :])
        q[n], sc[n] = qn[0], sn[0]
    return q, sc


def test_dispatch_permute_fp8_is_each_send_row_quantized():
    s = spec("skewed_t16384", T=40, H=512, E=16, P=4)
    idx, w = make_routing(s)
    x = make_hidden(s)
    x[7, 128:256] = 0                                  # an all-zero group
    sti, srk, _, _, _ = O.build_send_layout(idx, w, s.P, s.E_local)
    q, sc = O.dispatch_permute_fp8(x, sti)
    bq, bsc = _brute_force_permute_fp8(x, sti)
    assert q.shape == (len(sti), s.H) and sc.shape == (len(sti), s.H // 128)
    assert np.array_equal(q, bq)
    assert np.array_equal(sc.view(np.uint32), bsc.view(np.uint32))


def test_dispatch_permute_fp8_follows_any_row_order():
    # an order that is neither ascending nor the identity, with repeats
    rng = np.random.default_rng(5)
    x = make_hidden(spec("fp8_t32768", T=12, H=384))
    sti = np.array([11, 0, 3, 3, 7, 1, 11, 5, 2, 9, 9, 4, 0, 10], dtype=np.int32)
    rng.shuffle(sti)
    q, sc = O.dispatch_permute_fp8(x, sti)
    bq, bsc = _brute_force_permute_fp8(x, sti)
    assert np.array_equal(q, bq)
    assert np.array_equal(sc.view(np.uint32), bsc.view(np.uint32))
