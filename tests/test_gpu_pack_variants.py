"""GPU parity of the pack and gather variants against the CPU oracle
(bit-exact): fp16 kv_b_proj outputs, a k_pe that arrives as fp8 codes and is
copied into the key unchanged, and the gather that returns an fp8 cache's
codes without dequantising.

Page: "PR #51772 完整报告", 关键源码片段 (fused_mla_kv_concat_quant_fp8: the
plain fp8 cache's gather is not dequantised and its k_pe bytes go into the
key as they are) and 评论区精华 (bit-level tests over bf16 and fp16 inputs,
num_tokens including 0, num_heads 3 and 4, both k_pe dtypes).

Workloads: the pages' test matrix (T in 0, 1, 37, 300; H in 3, 4) on seeded
inputs, fp16 values spread to N(0, 40^2) with planted +-inf / NaN / +-65504
to exercise saturation, grid caps, and the chunked-context shape (fp8 cache
[512, 64, 576], 8192 tokens, kv_b_proj [8192, 64, 256]) through raw gather ->
verbatim-k_pe pack, every byte against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_paged_insert_amd import synth
from gpu_util import DEV, announce, requires_gpu, run_sliced, u16, u8

pytestmark = [pytest.mark.gpu, requires_gpu]


def f16u(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def plant_specials(x):
    """Put +-inf, NaN and +-65504 into the first row of an fp16 tensor."""
    flat = x.view(-1)
    vals = torch.tensor([float("inf"), float("-inf"), float("nan"), 65504.0, -65504.0,
                         500.0, -463.0, 2.0 ** -24], dtype=torch.float16)
    flat[:vals.numel()] = vals
    return x


def gpu_pack(mk, kn, kpe, v, fp8, k_scale=None, v_scale=None, max_blocks=0):
    T, H, nope = kn.shape
    rope = kpe.shape[-1]
    if not fp8:
        key = torch.empty(T, H, nope + rope, dtype=kn.dtype, device=DEV)
        mk.mla_ctx_kv_pack(kn, kpe, key, max_blocks=max_blocks)
        return key, None
    key = torch.empty(T, H, nope + rope, dtype=torch.uint8, device=DEV)
    vo = torch.empty(T, H, v.shape[2], dtype=torch.uint8, device=DEV)
    ks = None if k_scale is None else torch.tensor([k_scale], device=DEV)
    vs = None if v_scale is None else torch.tensor([v_scale], device=DEV)
    mk.mla_ctx_kv_pack(kn, kpe, key, v=v, v_out=vo, mode=mk.MLA_PACK_KEY_V_FP8, k_scale=ks,
                       v_scale=vs, max_blocks=max_blocks)
    return key, vo


# ------------------------------------------------------------ fp16 sources --
@pytest.mark.parametrize("H", [3, 4])
@pytest.mark.parametrize("T", [0, 1, 37, 300])
@pytest.mark.parametrize("fp8", [False, True])
def test_pack_fp16_matrix(mk, T, H, fp8):
    announce("pack fp16 matrix", T, H, fp8)
    g = torch.Generator().manual_seed(200 + T + H)
    kvb = synth.f16_normal((T, H, 256), g, std=40.0)
    ws = synth.f16_normal((T, 576), g, std=40.0)
    if T:
        plant_specials(kvb[0, 0])
        plant_specials(ws[0, 512:])
    dk, dw = kvb.to(DEV), ws.to(DEV)
    key, vo = gpu_pack(mk, dk[..., :128], dw[:, 512:], dk[..., 128:], fp8)
    kb, wb = f16u(kvb), f16u(ws)
    if fp8:
        rk, rv = oracle.pack(kb[..., :128], wb[:, 512:], kb[..., 128:],
                             mode=oracle.PACK_KEY_V_FP8, fp16=True)
        assert np.array_equal(u8(key), rk)
        assert np.array_equal(u8(vo), rv)
    else:
        rk, _ = oracle.pack(kb[..., :128], wb[:, 512:], fp16=True)
        assert np.array_equal(f16u(key), rk)


def test_pack_fp16_scales_and_caps(mk):
    announce("pack fp16 scales / caps")
    g = torch.Generator().manual_seed(211)
    kvb = synth.f16_normal((513, 8, 256), g, std=40.0)
    ws = synth.f16_normal((513, 576), g, std=40.0)
    dk, dw = kvb.to(DEV), ws.to(DEV)
    kb, wb = f16u(kvb), f16u(ws)
    for ks, vs, mb in ((0.7312, 1.37, 0), (0.25, None, 7), (None, -0.1, 1), (3.0e-3, 512.0, 0)):
        key, vo = gpu_pack(mk, dk[..., :128], dw[:, 512:], dk[..., 128:], True, ks, vs, mb)
        rk, rv = oracle.pack(kb[..., :128], wb[:, 512:], kb[..., 128:], mode=oracle.PACK_KEY_V_FP8,
                             k_scale=ks or 1.0, v_scale=vs or 1.0, fp16=True)
        assert np.array_equal(u8(key), rk), (ks, vs, mb)
        assert np.array_equal(u8(vo), rv), (ks, vs, mb)


def test_pack_fp16_every_pattern(mk):
    """All 65536 fp16 bit patterns through the fp8 converter path, as k_nope
    and as V, at scale 1 and at a negative non-power-of-two scale."""
    announce("pack fp16 every pattern")
    bits = torch.arange(1 << 16, dtype=torch.int32).to(torch.int16).view(torch.float16)
    kvb = bits.reshape(256, 1, 256).to(DEV)
    kpe = torch.zeros(256, 64, dtype=torch.float16, device=DEV)
    kb = f16u(kvb)
    for sc in (None, -0.7312):
        key, vo = gpu_pack(mk, kvb[..., :128], kpe, kvb[..., 128:], True, sc, sc)
        rk, rv = oracle.pack(kb[..., :128], f16u(kpe), kb[..., 128:], mode=oracle.PACK_KEY_V_FP8,
                             k_scale=sc or 1.0, v_scale=sc or 1.0, fp16=True)
        assert np.array_equal(u8(key), rk), sc
        assert np.array_equal(u8(vo), rv), sc


# ------------------------------------------------------------ raw gather --
def gpu_gather_raw(mk, cache, slots, max_blocks=0, width=576):
    out = torch.empty(slots.numel(), width, dtype=torch.uint8, device=DEV)
    mk.mla_ctx_latent_gather(cache, slots, out, None, "fp8", max_blocks=max_blocks)
    return out


def test_raw_gather_context_workload_and_caps(mk):
    announce("raw gather C4")
    d = synth.context_pack()
    cache, slots = d["cache"].to(DEV), d["src_slots"].to(DEV)
    ref = oracle.gather(d["cache"].numpy(), d["src_slots"].numpy(), raw=True)
    for mb in (0, 1, 7):
        assert np.array_equal(u8(gpu_gather_raw(mk, cache, slots, mb)), ref), mb


def test_raw_gather_every_code_partial_width_and_empty(mk):
    announce("raw gather codes / width / empty")
    codes = torch.arange(256 * 9, dtype=torch.int32).remainder(256).to(torch.uint8)
    cache = codes.reshape(4, 1, 576)
    slots = torch.tensor([2, 0, 3, 1], dtype=torch.int64)
    out = gpu_gather_raw(mk, cache.to(DEV), slots.to(DEV))
    assert np.array_equal(u8(out), oracle.gather(cache.numpy(), slots.numpy(), raw=True))
    out = gpu_gather_raw(mk, cache.to(DEV), slots.to(DEV), width=512)
    assert np.array_equal(u8(out), oracle.gather(cache.numpy(), slots.numpy(), width=512,
                                                 raw=True))
    empty = gpu_gather_raw(mk, cache.to(DEV), torch.empty(0, dtype=torch.int64, device=DEV))
    assert empty.shape == (0, 576)


def test_raw_gather_rejects_scale_and_bf16_cache(mk):
    announce("raw gather rejects")
    cache = torch.zeros(2, 4, 576, dtype=torch.uint8, device=DEV)
    slots = torch.zeros(2, dtype=torch.int64, device=DEV)
    out = torch.empty(2, 576, dtype=torch.uint8, device=DEV)
    with pytest.raises(RuntimeError, match="does not dequantise"):
        mk.mla_ctx_latent_gather(cache, slots, out, torch.tensor([0.5], device=DEV), "fp8")
    with pytest.raises(RuntimeError, match="needs an fp8 cache"):
        mk.mla_ctx_latent_gather(cache.view(torch.bfloat16), slots, out, None, "bfloat16")


# ----------------------------------------------------------- raw k_pe pack --
@pytest.mark.parametrize("H", [3, 4])
@pytest.mark.parametrize("T", [0, 1, 37, 300])
@pytest.mark.parametrize("fp16", [False, True])
def test_pack_raw_kpe_matrix(mk, T, H, fp16):
    announce("pack raw k_pe matrix", T, H, fp16)
    g = torch.Generator().manual_seed(300 + T + H)
    kvb = (synth.f16_normal if fp16 else synth.bf16_normal)((T, H, 256), g, std=4.0)
    ws8 = synth.random_bytes((T, 576), g)           # every code, NaNs included
    dk = kvb.to(DEV)
    kpe = ws8.to(DEV)[:, 512:]
    ks = 0.625
    key, vo = gpu_pack(mk, dk[..., :128], kpe, dk[..., 128:], True, ks, 1.5)
    kb = f16u(kvb)
    rk, rv = oracle.pack(kb[..., :128], ws8.numpy()[:, 512:], kb[..., 128:],
                         mode=oracle.PACK_KEY_V_FP8_KPE_RAW, k_scale=ks, v_scale=1.5, fp16=fp16)
    assert np.array_equal(u8(key), rk)
    assert np.array_equal(u8(vo), rv)


@pytest.mark.timeout(300)
def test_raw_gather_then_pack_context_workload(mk):
    """The plain-fp8-cache chunk at full size: raw gather of 8192 tokens, then
    the pack with k_pe read as codes straight from the raw workspace (and as
    a float8_e4m3fn view, which the binding routes the same way); every
    workspace, key and V byte against the oracle (token slices on host
    threads)."""
    announce("raw gather -> raw-k_pe pack C4")
    d = synth.context_pack()
    cache, slots = d["cache"].to(DEV), d["src_slots"].to(DEV)
    ws8 = gpu_gather_raw(mk, cache, slots)
    kvb = d["kvb"].to(DEV)
    key, vo = gpu_pack(mk, kvb[..., :128], ws8[:, 512:], kvb[..., 128:], True)
    key2, vo2 = gpu_pack(mk, kvb[..., :128], ws8.view(torch.float8_e4m3fn)[:, 512:],
                         kvb[..., 128:], True)
    torch.cuda.synchronize()
    assert torch.equal(key, key2) and torch.equal(vo, vo2)
    ref_ws = oracle.gather(d["cache"].numpy(), d["src_slots"].numpy(), raw=True)
    assert np.array_equal(u8(ws8), ref_ws)
    kb = u16(d["kvb"])
    parts = run_sliced(lambda a, b: oracle.pack(kb[a:b, :, :128], ref_ws[a:b, 512:],
                                                kb[a:b, :, 128:],
                                                mode=oracle.PACK_KEY_V_FP8_KPE_RAW), 8192)
    assert np.array_equal(u8(key), np.concatenate([p[0] for p in parts]))
    assert np.array_equal(u8(vo), np.concatenate([p[1] for p in parts]))
