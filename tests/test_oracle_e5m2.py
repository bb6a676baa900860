"""Pins for the oracle's fp8_e5m2 cache dtype.

Page: "PR #55356 完整报告", 实现拆解 item 3 and 关键源码片段 (cache_kernels.cu):
the dtype whitelist holds "fp8_e5m2", dispatched to its own template
instance (kFp8E5M2) of the same scaled_convert insert; the page's ROCm build
refuses it, this gfx950 build implements it.

The format is OCP e5m2 (torch.float8_e5m2): torch's CPU casts are the
library routine the codec is checked against.  Reading (as for e4m3fn):
saturation at +-57344, so values from 61440 up (and +-Inf) give +-57344
where torch's cast gives +-Inf; everything below agrees with torch.
"""
import numpy as np
import pytest
import torch

from fp8_paged_insert_amd import synth


def u16(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def torch_e5m2(x_f32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x_f32, np.float32)).to(
        torch.float8_e5m2).view(torch.uint8).numpy()


ALL_BF16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def test_decode_all_codes_match_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.e5m2_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[nan]), codes[nan] >= 0x80)


@pytest.mark.parametrize("code,value", [
    (0x7B, 57344.0), (0x7C, np.inf), (0xFC, -np.inf), (0x01, 2.0 ** -16), (0x03, 3 * 2.0 ** -16),
    (0x04, 2.0 ** -14), (0x3C, 1.0), (0x3D, 1.25), (0xC2, -3.0), (0x80, -0.0)])
def test_decode_closed_forms(orc, code, value):
    v = orc.e5m2_decode(np.array([code], np.uint8))[0]
    assert v == value and np.signbit(v) == np.signbit(value)


def test_encode_all_bf16_below_overflow_matches_torch(orc):
    x = orc.bf16_to_f32(ALL_BF16)
    keep = ~np.isnan(x) & (np.abs(x) < 61440.0)
    assert np.array_equal(orc.e5m2_encode(x[keep]), torch_e5m2(x[keep]))


def test_encode_midpoints_and_neighbours_match_torch(orc):
    vals = orc.e5m2_decode(np.arange(0x7C, dtype=np.uint8))      # finite, >= 0
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    for arr in (mids, up, dn, -mids, -up, -dn):
        assert np.array_equal(orc.e5m2_encode(arr), torch_e5m2(arr))


def test_encode_saturation_nan_and_zero(orc):
    x = np.array([57344.0, 61439.0, 61440.0, 1e9, np.inf, -np.inf, -61440.0, np.nan, -np.nan,
                  0.0, -0.0, 2.0 ** -18, -(2.0 ** -17) * 1.5], np.float32)
    want = np.array([0x7B, 0x7B, 0x7B, 0x7B, 0x7B, 0xFB, 0xFB, 0x7F, 0xFF, 0x00, 0x80, 0x00,
                     0x81], np.uint8)
    assert np.array_equal(orc.e5m2_encode(x), want)


@pytest.mark.parametrize("scale", [1.0, 0.5, 0.05, 0.7312, 1.9999, 3.0, -0.7312])
def test_quantize_matches_torch_divide_then_cast(orc, scale):
    x = orc.bf16_to_f32(ALL_BF16)
    with np.errstate(over="ignore", invalid="ignore"):
        q = (x / np.float32(scale)).astype(np.float32)
    keep = ~np.isnan(q) & (np.abs(q) < 61440.0)
    ours = orc.quantize_e5m2(ALL_BF16, scale)
    assert np.array_equal(ours[keep], torch_e5m2(q[keep]))
    big = ~np.isnan(q) & (np.abs(q) >= 61440.0)
    assert np.array_equal(ours[big], np.where(q[big] > 0, 0x7B, 0xFB).astype(np.uint8))


@pytest.mark.parametrize("scale", [1.0, 0.5, 0.7312, 2.0 ** -8, 3.5])
def test_dequantize_matches_torch(orc, scale):
    codes = np.arange(256, dtype=np.uint8)
    f = torch.from_numpy(codes).view(torch.float8_e5m2).float()
    ref = u16((f * torch.tensor(scale)).to(torch.bfloat16))
    ours = orc.dequantize_e5m2(codes, scale)
    nan = np.isnan(f.numpy())
    assert np.array_equal(ours[~nan], ref[~nan])              # Inf codes stay +-Inf
    # NaN codes: the canonical quiet NaN with the code's sign (torch keeps a payload)
    assert np.array_equal(ours[nan], np.where(codes[nan] >= 0x80, 0xFFC0, 0x7FC0))


def test_e5m2_differs_from_e4m3_where_it_must(orc):
    """A format mix-up would pass neither: 1.0 is 0x3C in e5m2 and 0x38 in
    e4m3fn; 448 is representable in both, 57344 only in e5m2."""
    x = np.array([1.0, 448.0, 57344.0], np.float32)
    assert orc.e5m2_encode(x).tolist() == [0x3C, 0x5F, 0x7B]
    assert orc.e4m3_encode(x).tolist() == [0x38, 0x7E, 0x7E]


def test_grouped_insert_e5m2_equals_torch_index_assignment(orc):
    """The e5m2 cache's grouped insert equals torch's index assignment of the
    torch-cast codes, layer by layer (brute force on a small cache)."""
    g = torch.Generator().manual_seed(61)
    L, T, R, P, nb, bs = 3, 11, 32, 16, 4, 4
    kv_c = synth.bf16_normal((L, T, R), g, std=30.0)
    k_pe = synth.bf16_normal((L, T, P), g, std=30.0)
    caches = [synth.random_bytes((nb, bs, R + P), g) for _ in range(L)]
    scales = torch.tensor([0.5, 1.7, 0.031], dtype=torch.float32)
    slots = torch.stack([torch.randperm(nb * bs, generator=g)[:T] for _ in range(L)])
    slots[1, 3] = -1
    ours = [c.numpy().copy() for c in caches]
    orc.insert_grouped(u16(kv_c), u16(k_pe), slots.numpy(), ours, scales.numpy(),
                       fp8_format="e5m2")
    for l in range(L):
        ref = caches[l].clone().view(nb * bs, R + P)
        row = torch.cat([kv_c[l], k_pe[l]], -1).float() / scales[l]
        codes = row.to(torch.float8_e5m2).view(torch.uint8)
        for t in range(T):
            if slots[l, t] >= 0:
                ref[slots[l, t]] = codes[t]
        assert np.array_equal(ours[l].reshape(nb * bs, R + P), ref.numpy()), l


def test_gather_e5m2_matches_torch(orc):
    g = torch.Generator().manual_seed(62)
    nb, bs, W, T = 6, 8, 576, 30
    cache = synth.random_bytes((nb, bs, W), g)
    blocks = torch.randperm(nb, generator=g)[:4]
    slots = synth.block_table_slots(blocks, bs, T)
    rows = cache.view(nb * bs, W)[slots]
    f = rows.view(torch.float8_e5m2).float()
    ref = u16((f * torch.tensor(0.37)).to(torch.bfloat16))
    ours = orc.gather(cache.numpy(), slots.numpy(), scale=0.37, fp8_format="e5m2")
    nan = np.isnan(f.numpy())
    assert nan.any() and np.array_equal(ours[~nan], ref[~nan])
    assert np.all((ours[nan] & 0x7FFF) == 0x7FC0)
    raw = orc.gather(cache.numpy(), slots.numpy(), raw=True, fp8_format="e5m2")
    assert np.array_equal(raw, rows.numpy())
