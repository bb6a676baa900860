"""GPU parity of mla_ctx_latent_gather and mla_ctx_kv_pack against the CPU
oracle (bit-exact).

Workloads: the chunked-context pack (fp8 cache [512, 64, 576] at scale 0.5
holding 8192 tokens in shuffled blocks; kv_b_proj output [8192, 64, 256];
bf16 key and fp8 key + V), the test matrix of PR #51772 report (评论区精华:
num_heads 3 and 4, num_tokens including 0), grid caps 1 / 7 / default, the
gather -> pack chain, and the long-context pack (131072 tokens as 16 chunks
of 8192 through the capped grid), sampled against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_paged_insert_amd import synth
from gpu_util import DEV, announce, requires_gpu, u16, u8

pytestmark = [pytest.mark.gpu, requires_gpu]


def gpu_gather(mk, cache, slots, scale, dtype="fp8", max_blocks=0, width=576):
    out = torch.empty(slots.numel(), width, dtype=torch.bfloat16, device=DEV)
    sc = None if scale is None else torch.tensor([scale], dtype=torch.float32, device=DEV)
    mk.mla_ctx_latent_gather(cache, slots, out, sc, dtype, max_blocks=max_blocks)
    return out


def gpu_pack(mk, kvb, kpe, fp8, max_blocks=0, k_scale=None, v_scale=None, nope=128):
    T, H, _ = kvb.shape
    rope = kpe.shape[-1]
    if fp8:
        key = torch.empty(T, H, nope + rope, dtype=torch.uint8, device=DEV)
        vo = torch.empty(T, H, kvb.shape[2] - nope, dtype=torch.uint8, device=DEV)
        ks = None if k_scale is None else torch.tensor([k_scale], device=DEV)
        vs = None if v_scale is None else torch.tensor([v_scale], device=DEV)
        mk.mla_ctx_kv_pack(kvb[..., :nope], kpe, key, v=kvb[..., nope:], v_out=vo,
                           mode=mk.MLA_PACK_KEY_V_FP8, k_scale=ks, v_scale=vs,
                           max_blocks=max_blocks)
        return key, vo
    key = torch.empty(T, H, nope + rope, dtype=torch.bfloat16, device=DEV)
    mk.mla_ctx_kv_pack(kvb[..., :nope], kpe, key, max_blocks=max_blocks)
    return key, None


def oracle_pack(kvb_np, kpe_np, fp8, k_scale=1.0, v_scale=1.0, nope=128):
    if fp8:
        return oracle.pack(kvb_np[..., :nope], kpe_np, kvb_np[..., nope:],
                           mode=oracle.PACK_KEY_V_FP8, k_scale=k_scale, v_scale=v_scale)
    return oracle.pack(kvb_np[..., :nope], kpe_np)


# ------------------------------------------------------------------ gather --
def test_gather_context_pack_workload(mk):
    announce("gather C4")
    d = synth.context_pack()
    cache = d["cache"].to(DEV)
    slots = d["src_slots"].to(DEV)
    ws = gpu_gather(mk, cache, slots, 0.5)
    ref = oracle.gather(d["cache"].numpy(), d["src_slots"].numpy(), 0.5)
    assert np.array_equal(u16(ws), ref)


@pytest.mark.parametrize("scale", [0.5, 1.0, 0.7312, 1.9999, 0.05, 3.0e-3])
def test_gather_every_code(mk, scale):
    """All 256 e4m3fn codes (NaN included) dequantised at several scales."""
    announce("gather codes", scale)
    codes = torch.arange(256 * 9, dtype=torch.int32).remainder(256).to(torch.uint8)
    cache = codes.reshape(4, 1, 576)
    slots = torch.tensor([2, 0, 3, 1], dtype=torch.int64)
    out = gpu_gather(mk, cache.to(DEV), slots.to(DEV), scale)
    ref = oracle.gather(cache.numpy(), slots.numpy(), scale)
    assert np.array_equal(u16(out), ref)


def test_gather_bf16_cache_and_grid_caps(mk):
    announce("gather bf16 + caps")
    g = torch.Generator().manual_seed(31)
    cache = synth.random_bf16_bits((64, 16, 576), g)
    blocks = torch.randperm(64, generator=g)[:40]
    slots = synth.block_table_slots(blocks, 16, 630)
    ref = oracle.gather(u16(cache).reshape(64, 16, 576), slots.numpy())
    gc, gs = cache.to(DEV), slots.to(DEV)
    for mb in (1, 7, 0):
        out = gpu_gather(mk, gc, gs, None, dtype="bfloat16", max_blocks=mb)
        assert np.array_equal(u16(out), ref), mb


def test_gather_partial_width_and_zero_tokens(mk):
    announce("gather width / empty")
    d = synth.context_cache(num_blocks=16, num_ctx=300)
    cache = d["cache"].to(DEV)
    out = gpu_gather(mk, cache, d["src_slots"].to(DEV), 0.5, width=512)
    ref = oracle.gather(d["cache"].numpy(), d["src_slots"].numpy(), 0.5, width=512)
    assert np.array_equal(u16(out), ref)
    empty = gpu_gather(mk, cache, torch.empty(0, dtype=torch.int64, device=DEV), 0.5)
    assert empty.shape == (0, 576)


# -------------------------------------------------------------------- pack --
@pytest.mark.parametrize("H", [3, 4])
@pytest.mark.parametrize("T", [0, 1, 37, 300])
@pytest.mark.parametrize("fp8", [False, True])
def test_pack_small_matrix(mk, T, H, fp8):
    announce("pack matrix", T, H, fp8)
    g = torch.Generator().manual_seed(100 + T + H)
    kvb = synth.bf16_normal((T, H, 256), g)
    ws = synth.bf16_normal((T, 576), g)
    key, vo = gpu_pack(mk, kvb.to(DEV), ws.to(DEV)[:, 512:], fp8)
    rk, rv = oracle_pack(u16(kvb), u16(ws)[:, 512:], fp8)
    assert np.array_equal(u8(key) if fp8 else u16(key), rk)
    if fp8:
        assert np.array_equal(u8(vo), rv)


@pytest.mark.parametrize("fp8", [False, True])
def test_pack_grid_cap_independent(mk, fp8):
    announce("pack caps", fp8)
    g = torch.Generator().manual_seed(7)
    kvb = synth.bf16_normal((513, 8, 256), g).to(DEV)
    ws = synth.bf16_normal((513, 576), g).to(DEV)
    outs = [gpu_pack(mk, kvb, ws[:, 512:], fp8, max_blocks=mb) for mb in (1, 7, 0)]
    for k, v in outs[1:]:
        assert torch.equal(k, outs[0][0])
        if fp8:
            assert torch.equal(v, outs[0][1])


def test_pack_fp8_with_scales(mk):
    announce("pack scales")
    g = torch.Generator().manual_seed(8)
    kvb = synth.bf16_normal((64, 4, 256), g, std=40.0)
    ws = synth.bf16_normal((64, 576), g, std=40.0)
    for ks, vs in ((0.7312, 1.37), (0.25, None), (None, 0.1)):
        key, vo = gpu_pack(mk, kvb.to(DEV), ws.to(DEV)[:, 512:], True, k_scale=ks, v_scale=vs)
        rk, rv = oracle_pack(u16(kvb), u16(ws)[:, 512:], True, ks or 1.0, vs or 1.0)
        assert np.array_equal(u8(key), rk) and np.array_equal(u8(vo), rv), (ks, vs)


@pytest.mark.parametrize("fp8", [False, True])
def test_pack_context_workload_sampled(mk, fp8):
    """8192 tokens x 64 heads at full size: 192 sampled tokens against the
    oracle, plus the k_pe broadcast over heads checked on every token."""
    announce("pack C4 full", fp8)
    d = synth.context_pack()
    kvb = d["kvb"].to(DEV)
    ws = d["workspace"].to(DEV)
    key, vo = gpu_pack(mk, kvb, ws[:, 512:], fp8)
    torch.cuda.synchronize()
    assert torch.equal(key[:, :, 128:], key[:, :1, 128:].expand_as(key[:, :, 128:]))
    g = torch.Generator().manual_seed(5)
    pick = torch.randperm(8192, generator=g)[:192]
    rk, rv = oracle_pack(u16(d["kvb"][pick]), u16(d["workspace"][pick])[:, 512:], fp8)
    got_k = u8(key[pick.to(DEV)]) if fp8 else u16(key[pick.to(DEV)])
    assert np.array_equal(got_k, rk)
    if fp8:
        assert np.array_equal(u8(vo[pick.to(DEV)]), rv)


@pytest.mark.parametrize("fp8", [False, True])
def test_gather_then_pack_chain(mk, fp8):
    """One chunk end to end: cache -> gather -> pack on the GPU equals the
    oracle's gather -> pack from the same cache."""
    announce("gather->pack chain", fp8)
    d = synth.context_pack(num_ctx=1024, heads=16)
    cache, slots = d["cache"].to(DEV), d["src_slots"].to(DEV)
    ws = gpu_gather(mk, cache, slots, 0.5)
    key, vo = gpu_pack(mk, d["kvb"].to(DEV), ws[:, 512:], fp8)
    ref_ws = oracle.gather(d["cache"].numpy(), d["src_slots"].numpy(), 0.5)
    rk, rv = oracle_pack(u16(d["kvb"]), ref_ws[:, 512:], fp8)
    assert np.array_equal(u8(key) if fp8 else u16(key), rk)
    if fp8:
        assert np.array_equal(u8(vo), rv)


def test_long_context_pack_16_chunks_sampled(mk):
    """131072 context tokens in a [4096, 64, 576] cache, 16 chunks of 8192:
    gather + fp8 pack per chunk; 16 sampled tokens per chunk vs the oracle."""
    announce("long-context pack 16 chunks")
    d = synth.context_cache(seed=55, num_blocks=4096, num_ctx=131072)
    cache, slots = d["cache"].to(DEV), d["src_slots"].to(DEV)
    gk = torch.Generator(device=DEV)
    gk.manual_seed(555)
    g = torch.Generator().manual_seed(56)
    ws = torch.empty(8192, 576, dtype=torch.bfloat16, device=DEV)
    key = torch.empty(8192, 64, 192, dtype=torch.uint8, device=DEV)
    vo = torch.empty(8192, 64, 128, dtype=torch.uint8, device=DEV)
    for c in range(16):
        kvb = torch.randn(8192, 64, 256, generator=gk, device=DEV).to(torch.bfloat16)
        mk.mla_ctx_latent_gather(cache, slots[c * 8192:(c + 1) * 8192], ws,
                                 torch.tensor([0.5], device=DEV), "fp8")
        mk.mla_ctx_kv_pack(kvb[..., :128], ws[:, 512:], key, v=kvb[..., 128:], v_out=vo,
                           mode=mk.MLA_PACK_KEY_V_FP8)
        pick = torch.randperm(8192, generator=g)[:16]
        sl = d["src_slots"][c * 8192:(c + 1) * 8192][pick].numpy()
        ref_ws = oracle.gather(d["cache"].numpy(), sl, 0.5)
        rk, rv = oracle_pack(u16(kvb[pick.to(DEV)]), ref_ws[:, 512:], True)
        torch.cuda.synchronize()
        assert np.array_equal(u8(key[pick.to(DEV)]), rk), c
        assert np.array_equal(u8(vo[pick.to(DEV)]), rv), c


def test_launch_events_bracket_one_kernel(mk):
    """mla_set_launch_events: the next launch records the pair, later ones don't."""
    announce("launch events")
    g = torch.Generator().manual_seed(21)
    kvb = synth.bf16_normal((2048, 16, 256), g).to(DEV)
    ws = synth.bf16_normal((2048, 576), g).to(DEV)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()
    torch.cuda.synchronize()
    mk.set_launch_events(e0, e1)
    key, _ = gpu_pack(mk, kvb, ws[:, 512:], False)
    torch.cuda.synchronize()
    t1 = e0.elapsed_time(e1)
    assert t1 > 0.0
    gpu_pack(mk, kvb, ws[:, 512:], False)        # not armed: the pair is untouched
    torch.cuda.synchronize()
    assert e0.elapsed_time(e1) == t1
    with pytest.raises(mk.MlaError):
        mk.set_launch_events(e0, None)
