"""Pins for the oracle's number formats: bf16 rounding and fp8 e4m3fn encode/decode.

The fp8 path must be bit-identical to torch's float8_e4m3fn cast (PR #51772
report, sections 实现拆解 item 1 and 风险与影响 item 3), so torch's CPU cast is
the library routine the encoder is checked against; closed forms from the
format definition and midpoint enumeration pin it independently of torch.
"""
import math

import numpy as np
import pytest
import torch


def all_bf16_patterns():
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)


def torch_f32(bits_u16):
    return torch.from_numpy((bits_u16.astype(np.uint32) << 16).view(np.float32).copy())


# ----------------------------------------------------------------- decode --
def test_e4m3_decode_closed_forms(orc):
    d = orc.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert d[0x7E] == 448.0                   # largest finite
    assert d[0x08] == 2.0 ** -6               # smallest normal
    assert d[0x01] == 2.0 ** -9               # smallest subnormal
    assert d[0x07] == 7 * 2.0 ** -9           # largest subnormal
    assert d[0x38] == 1.0                     # exponent field 7 = bias
    assert d[0x39] == 1.125
    assert d[0xB8] == -1.0
    assert d[0x00] == 0.0 and not math.copysign(1, d[0x00]) < 0
    assert d[0x80] == 0.0 and math.copysign(1, d[0x80]) < 0
    assert math.isnan(d[0x7F]) and math.isnan(d[0xFF])
    assert np.isnan(d).sum() == 2             # no infinities, two NaNs
    pos = d[:0x7F]
    assert np.all(np.diff(pos) > 0)           # codes 0..0x7E strictly increasing


def test_e4m3_decode_matches_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = orc.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(ours[~nan]))


# ----------------------------------------------------------------- encode --
def test_e4m3_encode_closed_forms(orc):
    enc = orc.e4m3_encode_scalar
    assert enc(448.0) == 0x7E
    assert enc(-448.0) == 0xFE
    assert enc(2.0 ** -10) == 0x00            # tie between 0 and 2^-9 -> even code 0
    assert enc(1.5 * 2.0 ** -9) == 0x02       # tie between codes 1 and 2 -> even
    assert enc(2.5 * 2.0 ** -9) == 0x02       # tie between codes 2 and 3 -> even
    assert enc(2.0 ** -11) == 0x00
    assert enc(-2.0 ** -11) == 0x80           # sign kept on underflow
    assert enc(-0.0) == 0x80
    assert enc(0.0) == 0x00
    assert enc(1.0) == 0x38
    assert enc(1.0625) == 0x38                # tie 1.0 / 1.125 -> even (0x38)
    assert enc(1.1875) == 0x3A                # tie 1.125 / 1.25 -> even (0x3A)
    assert enc(7.5 * 2.0 ** -9) == 0x08       # tie across the subnormal/normal edge
    # reading: saturate at +-448 (Inf included), NaN keeps its sign
    for big in (449.0, 463.9, 464.0, 465.0, 480.0, 1e30, math.inf):
        assert enc(big) == 0x7E and enc(-big) == 0xFE
    assert enc(math.nan) == 0x7F
    assert enc(-math.nan) == 0xFF


def test_e4m3_encode_midpoints(orc):
    """Every midpoint between neighbouring finite codes goes to the even code,
    and one float32 ulp either side goes to the nearer code."""
    vals = orc.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    for c in range(0x7E):
        lo, hi = vals[c], vals[c + 1]
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2    # representable in float32
        even = c if c % 2 == 0 else c + 1
        below = np.nextafter(mid, np.float32(-np.inf))
        above = np.nextafter(mid, np.float32(np.inf))
        got = orc.e4m3_encode(np.array([mid, below, above, -mid], np.float32))
        assert got.tolist() == [even, c, c + 1, 0x80 | even], c


def test_e4m3_encode_matches_torch_all_bf16(orc):
    bits = all_bf16_patterns()
    x = torch_f32(bits)
    finite = torch.isfinite(x) & (x.abs() <= 464)
    xs = x[finite]
    ref = xs.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = orc.e4m3_encode(xs.numpy())
    assert np.array_equal(ref, ours)


def test_e4m3_encode_matches_torch_random_f32(orc):
    g = torch.Generator().manual_seed(7)
    u = torch.randint(0, 2 ** 31 - 1, (400_000,), generator=g, dtype=torch.int64)
    u = (u % (0x43E80000)).to(torch.int32)  # |x| < 464 as float bits
    x = u.view(torch.float32) * torch.where(
        torch.rand(u.shape, generator=g) < 0.5, -1.0, 1.0)
    ref = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = orc.e4m3_encode(x.numpy())
    assert np.array_equal(ref, ours)


@pytest.mark.parametrize("scale", [1.0, 0.5, 0.05, 0.1, 0.15, 0.2, 0.25, 0.7312, 1.9999, 0.5000001])
def test_quantize_matches_torch_all_bf16(orc, scale):
    """quantize(x, s) == torch e4m3fn cast of fl32(x) / fl32(s) wherever torch
    and the saturating reading agree (|x/s| <= 464); above that, +-448."""
    bits = all_bf16_patterns()
    x = torch_f32(bits)
    s = torch.tensor(scale, dtype=torch.float32)
    q = x / s
    ours = orc.quantize(bits, float(s))
    ok = torch.isfinite(q) & (q.abs() <= 464)
    ref = q[ok].to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ref, ours[ok.numpy()])
    big = (torch.isinf(q) | (q.abs() > 464)).numpy() & ~np.isnan(q.numpy())
    sign = np.signbit(q.numpy()[big])
    assert np.array_equal(ours[big], np.where(sign, 0xFE, 0x7E).astype(np.uint8))
    nan = np.isnan(q.numpy())
    assert np.array_equal(ours[nan] & 0x7F, np.full(nan.sum(), 0x7F, np.uint8))


def test_quantize_divides_not_reciprocal(orc):
    """The stored code uses fl32(x / s); a reciprocal multiply would differ.
    Find bf16 inputs where the two differ and check the oracle follows division."""
    bits = all_bf16_patterns()
    x = torch_f32(bits)
    s = torch.tensor(0.7312, dtype=torch.float32)
    div = (x / s)
    rec = x * (1.0 / s)
    diff = (div != rec) & torch.isfinite(div) & (div.abs() <= 448)
    assert diff.any()
    sel = diff.nonzero().flatten().numpy()
    ours = orc.quantize(bits[sel], float(s))
    assert np.array_equal(ours, div[diff].to(torch.float8_e4m3fn).view(torch.uint8).numpy())


# ------------------------------------------------------------ dequantize --
@pytest.mark.parametrize("scale", [0.5, 1.0, 0.7312, 1.9999, 0.05])
def test_dequantize_matches_torch(orc, scale):
    codes = np.arange(256, dtype=np.uint8)
    f = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float32)
    ref = (f * torch.tensor(scale, dtype=torch.float32)).to(torch.bfloat16)
    ref = ref.view(torch.int16).numpy().view(np.uint16)
    ours = orc.dequantize(codes, scale)
    fin = np.isfinite(f.numpy())
    assert np.array_equal(ref[fin], ours[fin])
    assert np.all((ours[~fin] & 0x7FC0) == 0x7FC0)  # NaN stays NaN


def test_dequantize_half_scale_is_exact(orc):
    """At scale 0.5 every finite code's value / 2 is exactly representable in bf16."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = orc.e4m3_decode(codes) * 0.5
    ours = orc.dequantize(codes, 0.5)
    back = orc.bf16_to_f32(ours).astype(np.float64)
    assert np.array_equal(back, vals)


# -------------------------------------------------------------- bf16 RNE --
def test_bf16_rounding_matches_torch_f32(orc):
    g = torch.Generator().manual_seed(11)
    u = torch.randint(-2 ** 31, 2 ** 31 - 1, (500_000,), generator=g, dtype=torch.int64)
    x = u.to(torch.int32).view(torch.float32)
    x = x[torch.isfinite(x)]
    ref = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = orc.f64_to_bf16(x.numpy().astype(np.float64))
    assert np.array_equal(ref, ours)


def test_bf16_rounding_closed_forms(orc):
    r = lambda v: int(orc.f64_to_bf16(np.array([v]))[0])
    assert r(1.0) == 0x3F80
    assert r(1.0 + 2.0 ** -8) == 0x3F80                 # tie -> even (down)
    assert r(1.0 + 3 * 2.0 ** -8) == 0x3F82             # tie -> even (up)
    assert r(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81    # just above the tie (not in f32)
    assert r(1.0 + 2.0 ** -8 - 2.0 ** -40) == 0x3F80
    assert r(-2.0) == 0xC000
    assert r(2.0 ** -133) == 0x0001                     # smallest subnormal
    assert r(2.0 ** -134) == 0x0000                     # tie with 0 -> even
    assert r(1.5 * 2.0 ** -133) == 0x0002               # tie -> even
    bmax = (2.0 - 2.0 ** -7) * 2.0 ** 127
    assert r(bmax) == 0x7F7F                            # largest finite bf16
    assert r(bmax + 2.0 ** 119) == 0x7F80               # tie above max -> even = inf
    assert r(bmax + 2.0 ** 118) == 0x7F7F
    assert r(3.5e38) == 0x7F80                          # overflow -> inf
    assert r(-1e300) == 0xFF80
    assert r(math.inf) == 0x7F80
    assert r(math.nan) == 0x7FC0
    assert r(-0.0) == 0x8000
