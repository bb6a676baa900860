"""Pins for the oracle's pack and gather variants: fp16 sources, a k_pe that
arrives as fp8 codes and is copied verbatim, and the raw-code gather.

Page: "PR #51772 完整报告", 关键源码片段 (fused_mla_kv_concat_quant_fp8: a k_pe
that is already fp8 -- the plain fp8 cache's gather does not dequantise -- is
copied into the key as is) and 评论区精华 (the bit-level tests cover bf16 and
fp16 inputs, 0 tokens, 3 and 4 heads, both k_pe dtypes).

What pins each path to something other than the oracle itself:
  * fp16 decode: every one of the 65536 patterns against numpy's float16
    (a library conversion), plus closed-form values of the format.
  * fp16 pack: torch's float8_e4m3fn cast of the fp16 values (library) where
    |x| <= 448, closed-form saturation codes beyond, and agreement with the
    bf16 pack on values both formats hold exactly.
  * raw-k_pe pack: equals the fp8 pack whenever the raw codes are the codes
    the fp8 pack would have produced, and copies NaN codes bit for bit.
  * raw gather: torch indexing of the cache bytes, and dequantising it gives
    the (already pinned) dequantising gather.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_paged_insert_amd import synth


def u16(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def f16_bits(t):
    return t.to(torch.float16).contiguous().view(torch.int16).numpy().view(np.uint16)


# -------------------------------------------------------------- fp16 decode --
def test_f16_decode_every_pattern_matches_numpy(orc):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = orc.f16_to_f32(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    # NaNs keep their sign
    assert np.array_equal(np.signbit(ours[nan]), (bits[nan] >> 15).astype(bool))


@pytest.mark.parametrize("bits,value", [
    (0x3C00, 1.0), (0xC000, -2.0), (0x7BFF, 65504.0), (0x0001, 2.0 ** -24),
    (0x0400, 2.0 ** -14), (0x03FF, 1023 * 2.0 ** -24), (0x3555, 0.333251953125),
    (0x7C00, float("inf")), (0xFC00, float("-inf")), (0x0000, 0.0)])
def test_f16_decode_closed_forms(orc, bits, value):
    assert orc.f16_to_f32(np.array([bits], np.uint16))[0] == np.float32(value)


def test_f16_decode_negative_zero(orc):
    z = orc.f16_to_f32(np.array([0x8000], np.uint16))[0]
    assert z == 0.0 and np.signbit(z)


# ---------------------------------------------------------------- fp16 pack --
@pytest.mark.parametrize("H", [3, 4])
@pytest.mark.parametrize("T", [0, 1, 37])
def test_pack_fp16_fp8_matches_torch_cast(orc, T, H):
    g = torch.Generator().manual_seed(31 + H + T)
    kvb = (torch.randn(T, H, 256, generator=g) * 40).to(torch.float16)
    ws = (torch.randn(T, 576, generator=g) * 40).to(torch.float16)
    kvb = kvb.clamp(-448, 448)
    ws = ws.clamp(-448, 448)
    key_ref = torch.cat([kvb[..., :128], ws[:, None, 512:].expand(T, H, 64)], -1)
    key_ref = key_ref.float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    v_ref = kvb[..., 128:].float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    kb, wb = f16_bits(kvb), f16_bits(ws)
    key, vo = orc.pack(kb[..., :128], wb[:, 512:], kb[..., 128:], mode=orc.PACK_KEY_V_FP8,
                       fp16=True)
    assert np.array_equal(key, key_ref)
    assert np.array_equal(vo, v_ref)


def test_pack_fp16_saturates_and_keeps_nan(orc):
    vals = np.array([65504.0, -65504.0, 500.0, -464.0, np.inf, -np.inf, np.nan, -np.nan,
                     448.0, 2.0 ** -9, -(2.0 ** -10) * 3, 0.0], np.float16)
    want = np.array([0x7E, 0xFE, 0x7E, 0xFE, 0x7E, 0xFE, 0x7F, 0xFF, 0x7E, 0x01, 0x82, 0x00],
                    np.uint8)
    n = vals.size
    kn = np.zeros((1, 1, 16), np.uint16)
    kn[0, 0, :n] = vals.view(np.uint16)
    v = kn.copy()
    key, vo = orc.pack(kn, np.zeros((1, 16), np.uint16), v, mode=orc.PACK_KEY_V_FP8,
                       fp16=True)
    assert np.array_equal(key[0, 0, :n], want)
    assert np.array_equal(vo[0, 0, :n], want)


def test_pack_fp16_equals_bf16_on_shared_values(orc):
    """Values with at most 8 significant bits and a moderate exponent are exact
    in both formats; the fp16 and bf16 packs must then agree code for code."""
    g = torch.Generator().manual_seed(37)
    T, H = 9, 3
    x = torch.randn(T, H, 256, generator=g).to(torch.bfloat16).float()
    pe = torch.randn(T, 576, generator=g).to(torch.bfloat16).float()
    assert torch.equal(x.to(torch.float16).float(), x)
    assert torch.equal(pe.to(torch.float16).float(), pe)
    for ks, vs in [(1.0, 1.0), (0.37, 2.5)]:
        a = orc.pack(u16(x.to(torch.bfloat16))[..., :128], u16(pe.to(torch.bfloat16))[:, 512:],
                     u16(x.to(torch.bfloat16))[..., 128:], mode=orc.PACK_KEY_V_FP8,
                     k_scale=ks, v_scale=vs)
        b = orc.pack(f16_bits(x)[..., :128], f16_bits(pe)[:, 512:], f16_bits(x)[..., 128:],
                     mode=orc.PACK_KEY_V_FP8, k_scale=ks, v_scale=vs, fp16=True)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_pack_fp16_key_mode_is_a_bit_copy(orc):
    g = torch.Generator().manual_seed(41)
    T, H = 6, 4
    kvb = torch.randn(T, H, 256, generator=g).to(torch.float16)
    ws = torch.randn(T, 576, generator=g).to(torch.float16)
    key, _ = orc.pack(f16_bits(kvb)[..., :128], f16_bits(ws)[:, 512:], fp16=True)
    ref = torch.cat([kvb[..., :128], ws[:, None, 512:].expand(T, H, 64)], -1)
    assert np.array_equal(key, f16_bits(ref))


# ----------------------------------------------------------- raw k_pe pack --
@pytest.mark.parametrize("H", [3, 4])
@pytest.mark.parametrize("T", [0, 1, 37])
def test_pack_raw_kpe_equals_fp8_pack_on_its_codes(orc, T, H):
    g = torch.Generator().manual_seed(43 + T + H)
    kvb = torch.randn(T, H, 256, generator=g).to(torch.bfloat16)
    ws = torch.randn(T, 576, generator=g).to(torch.bfloat16)
    ks = 0.625
    kn, kp, v = u16(kvb)[..., :128], u16(ws)[:, 512:], u16(kvb)[..., 128:]
    codes = orc.quantize(np.ascontiguousarray(kp), ks)      # what an fp8 cache would hold
    ws8 = np.zeros((T, 576), np.uint8)                      # raw gather workspace
    ws8[:, 512:] = codes
    a = orc.pack(kn, kp, v, mode=orc.PACK_KEY_V_FP8, k_scale=ks, v_scale=1.5)
    b = orc.pack(kn, ws8[:, 512:], v, mode=orc.PACK_KEY_V_FP8_KPE_RAW, k_scale=ks, v_scale=1.5)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_pack_raw_kpe_copies_every_code(orc):
    T, H = 4, 3
    codes = np.arange(256, dtype=np.uint8).reshape(4, 64)    # includes 0x7F / 0xFF NaNs
    kn = np.zeros((T, H, 128), np.uint16)
    v = np.zeros((T, H, 128), np.uint16)
    key, _ = orc.pack(kn, codes, v, mode=orc.PACK_KEY_V_FP8_KPE_RAW, k_scale=3.0)
    for h in range(H):
        assert np.array_equal(key[:, h, 128:], codes)
    assert not key[:, :, :128].any()


# --------------------------------------------------------------- raw gather --
def test_raw_gather_matches_torch_indexing_and_dequant(orc):
    g = torch.Generator().manual_seed(47)
    nb, bs, W, T = 6, 8, 576, 30
    cache = synth.random_bytes((nb, bs, W), g)
    blocks = torch.randperm(nb, generator=g)[:4]
    slots = synth.block_table_slots(blocks, bs, T)
    raw = orc.gather(cache.numpy(), slots.numpy(), raw=True)
    assert raw.dtype == np.uint8
    assert np.array_equal(raw, cache.view(nb * bs, W)[slots].numpy())
    deq = orc.gather(cache.numpy(), slots.numpy(), scale=0.5)
    assert np.array_equal(orc.dequantize(raw.reshape(-1), 0.5).reshape(T, W), deq)


def test_raw_gather_rejects_bf16_cache(orc):
    cache = np.zeros((2, 4, 576), np.uint16)
    with pytest.raises(oracle.OracleError):
        orc.gather(cache, np.array([0, 1], np.int64), raw=True)
