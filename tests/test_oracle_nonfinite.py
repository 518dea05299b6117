"""Pins of the oracle's readings for non-finite values, which the pages leave
open: any NaN rounds to the canonical bf16 quiet NaN 0x7FC0 and to the e4m3
NaN code 0x7F; infinities keep their sign in bf16 and saturate in e4m3; NaN
elements do not count toward an fp8 group's amax; a group holding an
infinity gets an infinite scale.  Checked against torch's conversions and
IEEE division, not against the oracle's own code."""

import numpy as np
import torch

import oracle as O


def _nan_patterns(n=500, seed=0):
    """float32 NaN bit patterns: random payloads and signs, quiet and
    signalling, plus the edge payloads that a rounding carry would turn into
    an infinity or a zero."""
    r = np.random.default_rng(seed)
    mant = r.integers(1, 1 << 23, n, dtype=np.uint32)
    sign = r.integers(0, 2, n, dtype=np.uint32) << np.uint32(31)
    u = sign | np.uint32(0x7F800000) | mant
    edge = np.uint32([0x7F800001, 0x7FFFFFFF, 0xFFFFFFFF, 0x7FC00000, 0xFFC00000,
                      0x7FBFFFFF, 0x7FFF8000, 0xFF800001])
    return np.concatenate([u, edge]).view(np.float32)


def _torch_bf16_bits(values):
    return torch.from_numpy(np.asarray(values, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def test_bf16_nan_is_the_canonical_quiet_nan():
    out = O.f32_to_bf16(_nan_patterns())
    assert (out == 0x7FC0).all()
    as_bf16 = torch.from_numpy(np.uint16([0x7FC0]).view(np.int16)).view(torch.bfloat16)
    assert bool(torch.isnan(as_bf16.float()).all())


def test_bf16_infinities_and_overflow_match_torch():
    # infinities, and the finite values around the largest bf16 (the exact
    # half above it rounds to even, i.e. up to infinity)
    u = np.uint32([0x7F800000, 0xFF800000, 0x7F7F0000, 0x7F7F7FFF, 0x7F7F8000, 0x7F7F8001,
                   0x7F7FFFFF, 0xFF7F8000, 0xFF7FFFFF, 0x7F7E8000])
    v = u.view(np.float32)
    assert np.array_equal(O.f32_to_bf16(v), _torch_bf16_bits(v))


def test_e4m3_nan_code_and_saturation():
    assert (O.e4m3_encode(_nan_patterns()) == 0x7F).all()
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float()
    assert bool(torch.isnan(codes[0x7F])) and bool(torch.isnan(codes[0xFF]))
    # +NaN encodes as torch does
    assert O.e4m3_encode(np.float32([np.nan]))[0] == \
        torch.tensor([float("nan")]).to(torch.float8_e4m3fn).view(torch.uint8).item()
    # infinities take the largest finite magnitude, with their sign
    finite = codes[~torch.isnan(codes)]
    top = float(finite.abs().max())
    inf_codes = O.e4m3_encode(np.float32([np.inf, -np.inf]))
    assert float(codes[int(inf_codes[0])]) == top and float(codes[int(inf_codes[1])]) == -top


def _rows(R=12, H=512, seed=3):
    r = np.random.default_rng(seed)
    x = r.standard_normal((R, H)).astype(np.float32)
    return x


def _bits(x):
    return _torch_bf16_bits(x)


def test_nan_elements_do_not_move_amax():
    x = _rows()
    bits = _bits(x)
    r = np.random.default_rng(4)
    nan_bits = np.uint16([0x7FC0, 0xFFC1, 0x7F81, 0xFF81, 0x7FFF])   # quiet and signalling
    pos = r.choice(x.size, 300, replace=False)
    with_nan = bits.copy().reshape(-1)
    with_nan[pos] = nan_bits[r.integers(0, len(nan_bits), len(pos))]
    with_nan = with_nan.reshape(bits.shape)
    zeroed = with_nan.copy()
    zeroed.reshape(-1)[pos] = 0
    for fmt in O.SCALE_FORMATS:
        qn, sn = O.quantize_rows_fp8(with_nan, fmt)
        qz, sz = O.quantize_rows_fp8(zeroed, fmt)
        assert np.array_equal(sn.view(np.uint32), sz.view(np.uint32)), fmt
        mask = np.zeros(x.size, bool)
        mask[pos] = True
        mask = mask.reshape(x.shape)
        assert (qn[mask] == 0x7F).all(), fmt
        assert np.array_equal(qn[~mask], qz[~mask]), fmt


def test_all_nan_group_keeps_its_nans():
    bits = np.zeros((2, 512), np.uint16)
    bits[0, :128] = 0x7FC0                  # a group of NaNs only
    bits[1, :64] = 0xFF81                   # NaNs and zeros
    for fmt in O.SCALE_FORMATS:
        q, s = O.quantize_rows_fp8(bits, fmt)
        assert (q[0, :128] == 0x7F).all() and (q[0, 128:] == 0).all()
        assert (q[1, :64] == 0x7F).all() and (q[1, 64:] == 0).all()
        assert not np.asarray(s).view(np.uint32).any()          # every scale 0 (byte 0)


def test_infinite_group_gets_an_infinite_scale():
    x = _rows(R=2, H=512)
    x[0, 5] = np.inf
    x[1, 130] = -np.inf
    bits = _bits(x)
    xf = O.bf16_to_f32(bits)
    # IEEE: finite / inf is a signed zero, inf / inf is NaN; torch's e4m3 of
    # the signed zeros gives the codes 0x00 / 0x80
    zeros = torch.from_numpy(np.float32([0.0, -0.0])).to(torch.float8_e4m3fn).view(torch.uint8)
    assert zeros.tolist() == [0x00, 0x80]
    for fmt in O.SCALE_FORMATS:
        q, s = O.quantize_rows_fp8(bits, fmt)
        for row, g in ((0, 0), (1, 1)):
            grp = slice(128 * g, 128 * g + 128)
            vals = xf[row, grp]
            want = np.where(np.isinf(vals), 0x7F, np.where(np.signbit(vals), 0x80, 0x00))
            assert np.array_equal(q[row, grp], want), fmt
        if fmt == "ue8m0":
            b = O.unpack_ue8m0(s)
            assert b[0, 0] == 0xFF and b[1, 1] == 0xFF
            assert 0 < b[0, 1] < 0xFF
        else:
            assert np.isinf(s[0, 0]) and np.isinf(s[1, 1]) and np.isfinite(s[0, 1])
