"""GPU parity of mla_ctx_latent_gather and mla_ctx_kv_pack against the CPU
oracle (bit-exact).

Workloads: the chunked-context pack (fp8 cache [512, 64, 576] at scale 0.5
holding 8192 tokens in shuffled blocks; kv_b_proj output [8192, 64, 256];
bf16 key and fp8 key + V), the test matrix of PR #51772 report (评论区精华:
num_heads 3 and 4, num_tokens including 0), grid caps 1 / 7 / default, the
gather -> pack chain, the chunked-context pack at full size, and the
long-context pack (131072 tokens as 16 chunks of 8192, on the default grid,
on the capped grid-stride grid and through the joint pack + next-gather
launch), the joint launch for every gather kind and pack mode, every output
byte against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_paged_insert_amd import synth
from gpu_util import DEV, announce, requires_gpu, run_sliced, u16, u8

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



@pytest.mark.parametrize("kind", ["fp8", "raw", "bfloat16"])
@pytest.mark.parametrize("layout", ["padded_entries", "padded_blocks", "block_size_one"])
def test_gather_padded_layouts(mk, kind, layout):
    """Cache views whose entries or blocks are padded (entry stride 640 with
    the row at byte offset 32 of the entry; 16 of 17 entries used per block)
    and a block size of 1, read through the view's strides: every row equals
    the oracle's gather of the same logical [num_blocks, block_size, 576]
    cache (raw: the codes themselves)."""
    announce("gather layout", kind, layout)
    g = torch.Generator().manual_seed(400 + len(kind) * 7 + len(layout))
    bf16 = kind == "bfloat16"
    shape = {"padded_entries": (24, 32, 640), "padded_blocks": (40, 17, 576),
             "block_size_one": (700, 1, 576 + 64)}[layout]
    buf = synth.random_bf16_bits(shape, g) if bf16 else synth.random_bytes(shape, g)
    view = {"padded_entries": lambda b: b[:, :, 16 if bf16 else 32:][:, :, :576],
            "padded_blocks": lambda b: b[:, :16, :],
            "block_size_one": lambda b: b[:, :, :576]}[layout]
    host = view(buf)
    nb, bs = host.shape[0], host.shape[1]
    slots = torch.randperm(nb * bs, generator=g)[:min(600, nb * bs)].to(torch.int64)
    dev = view(buf.to(DEV))
    assert dev.stride() == host.stride()
    logical = (u16(host) if bf16 else u8(host)).copy()
    if kind == "raw":
        out = torch.empty(slots.numel(), 576, dtype=torch.uint8, device=DEV)
        mk.mla_ctx_latent_gather(dev, slots.to(DEV), out, None, "fp8")
        ref = logical.reshape(-1, 576)[slots.numpy()]
        assert np.array_equal(u8(out), ref)
        return
    scale = None if bf16 else 0.7312
    out = gpu_gather(mk, dev, slots.to(DEV), scale, dtype="bfloat16" if bf16 else "fp8")
    ref = oracle.gather(logical, slots.numpy(), scale) if scale else oracle.gather(logical,
                                                                                slots.numpy())
    assert np.array_equal(u16(out), ref)


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


def oracle_pack_full(kvb_np, kpe_np, fp8):
    """The oracle's pack over every token, token slices on host threads."""
    parts = run_sliced(lambda a, b: oracle_pack(kvb_np[a:b], kpe_np[a:b], fp8),
                       kvb_np.shape[0])
    key = np.concatenate([p[0] for p in parts])
    return key, (np.concatenate([p[1] for p in parts]) if fp8 else None)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("fp8", [False, True])
def test_pack_context_workload_full(mk, fp8):
    """8192 tokens x 64 heads at full size, every output byte against the
    oracle; the k_pe broadcast over heads checked on its own as well."""
    announce("pack C4 full", fp8)
    d = synth.context_pack()
    kvb = d["kvb"].to(DEV)
    ws = d["workspace"].to(DEV)
    key, vo = gpu_pack(mk, kvb, ws[:, 512:], fp8)
    torch.cuda.synchronize()
    assert torch.equal(key[:, :, 128:], key[:, :1, 128:].expand_as(key[:, :, 128:]))
    rk, rv = oracle_pack_full(u16(d["kvb"]), u16(d["workspace"])[:, 512:], fp8)
    assert np.array_equal(u8(key) if fp8 else u16(key), rk)
    if fp8:
        assert np.array_equal(u8(vo), rv)


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


@pytest.mark.timeout(600)
def test_long_context_pack_16_chunks_full(mk):
    """131072 context tokens in a [4096, 64, 576] cache, 16 chunks of 8192.
    Per chunk, on the GPU: the gather, the fp8 pack on the default grid and on
    a capped grid of 16 workgroups per compute unit (a grid-stride loop of
    about 10 passes), and the chunk loop with the joint launch (pack of chunk
    c + gather of chunk c + 1 into the other of two workspaces), its pack
    capped at 64 workgroups per compute unit.  Every
    workspace row and every key and V byte of every chunk, from each path,
    against the oracle's gather -> pack of the same cache."""
    announce("long-context pack 16 chunks, full")
    d = synth.context_cache(seed=55, num_blocks=4096, num_ctx=131072)
    cache, slots = d["cache"].to(DEV), d["src_slots"].to(DEV)
    cache_np, slots_np = d["cache"].numpy(), d["src_slots"].numpy()
    cap = 16 * torch.cuda.get_device_properties(DEV).multi_processor_count
    gk = torch.Generator(device=DEV)
    gk.manual_seed(555)
    ws = torch.empty(8192, 576, dtype=torch.bfloat16, device=DEV)
    ws2 = [torch.empty(8192, 576, dtype=torch.bfloat16, device=DEV) for _ in range(2)]
    outs = {k: (torch.empty(8192, 64, 192, dtype=torch.uint8, device=DEV),
                torch.empty(8192, 64, 128, dtype=torch.uint8, device=DEV))
            for k in ("default grid", "capped grid", "joint launch, capped pack")}
    sc = torch.tensor([0.5], device=DEV)
    chunk = lambda c: slots[c * 8192:(c + 1) * 8192]
    mk.mla_ctx_latent_gather(cache, chunk(0), ws2[0], sc, "fp8")
    for c in range(16):
        kvb = torch.randn(8192, 64, 256, generator=gk, device=DEV).to(torch.bfloat16)
        kn, v = kvb[..., :128], kvb[..., 128:]
        mk.mla_ctx_latent_gather(cache, chunk(c), ws, sc, "fp8")
        k, vo = outs["default grid"]
        mk.mla_ctx_kv_pack(kn, ws[:, 512:], k, v=v, v_out=vo, mode=mk.MLA_PACK_KEY_V_FP8)
        k, vo = outs["capped grid"]
        mk.mla_ctx_kv_pack(kn, ws[:, 512:], k, v=v, v_out=vo, mode=mk.MLA_PACK_KEY_V_FP8,
                           max_blocks=cap)
        torch.cuda.synchronize()
        joint_ws = u16(ws2[c % 2])            # gathered by the previous joint launch
        k, vo = outs["joint launch, capped pack"]
        if c < 15:
            mk.mla_ctx_kv_pack_gather(kn, ws2[c % 2][:, 512:], k, cache, chunk(c + 1),
                                      ws2[(c + 1) % 2], v=v, v_out=vo,
                                      mode=mk.MLA_PACK_KEY_V_FP8, cache_scale=sc,
                                      max_blocks=4 * cap)
        else:
            mk.mla_ctx_kv_pack(kn, ws2[c % 2][:, 512:], k, v=v, v_out=vo,
                               mode=mk.MLA_PACK_KEY_V_FP8, max_blocks=4 * cap)
        torch.cuda.synchronize()
        sl = slots_np[c * 8192:(c + 1) * 8192]
        ref_ws = np.concatenate(run_sliced(lambda a, b: oracle.gather(cache_np, sl[a:b], 0.5),
                                           8192))
        assert np.array_equal(u16(ws), ref_ws), f"chunk {c}: workspace"
        assert np.array_equal(joint_ws, ref_ws), f"chunk {c}: workspace of the joint launch"
        rk, rv = oracle_pack_full(u16(kvb), ref_ws[:, 512:], True)
        for name, (k, vo) in outs.items():
            assert np.array_equal(u8(k), rk), f"chunk {c}: key, {name}"
            assert np.array_equal(u8(vo), rv), f"chunk {c}: V, {name}"
        announce(f"chunk {c}: identical")


@pytest.mark.parametrize("kind", ["fp8", "fp8_e5m2", "bfloat16", "raw"])
@pytest.mark.parametrize("mode", ["bf16", "fp8", "fp8_scaled"])
@pytest.mark.parametrize("max_blocks", [0, 2])
def test_pack_gather_joint_launch(mk, kind, mode, max_blocks):
    """The joint launch against the oracle's pack of one chunk and gather of
    the next, for every gather kind and both 16-bit-source pack modes, on a
    ragged shape (300 tokens x 3 heads packed, 437 tokens gathered), with the
    full pack grid (the gather's workgroups first) and with the pack part
    capped at 2 workgroups (grid-stride; the gather's workgroups last)."""
    announce("pack + gather joint launch", kind, mode, max_blocks)
    g = torch.Generator().manual_seed(300 + len(kind) + len(mode))
    T, H, Tg = 300, 3, 437
    kvb = synth.bf16_normal((T, H, 256), g, std=40.0 if mode == "fp8_scaled" else 1.0)
    ws = synth.bf16_normal((T, 576), g)
    if kind == "bfloat16":
        cache = synth.random_bf16_bits((16, 64, 576), g)
        cache_np = u16(cache).reshape(16, 64, 576)
    else:
        cache = synth.random_bytes((16, 64, 576), g)
        cache_np = cache.numpy()
    blocks = torch.randperm(16, generator=g)[:7]
    sl = synth.block_table_slots(blocks, 64, Tg)
    dkvb, dws = kvb.to(DEV), ws.to(DEV)
    fp8 = mode != "bf16"
    key = torch.empty(T, H, 192, dtype=torch.uint8 if fp8 else torch.bfloat16, device=DEV)
    vo = torch.empty(T, H, 128, dtype=torch.uint8, device=DEV) if fp8 else None
    out = torch.empty(Tg, 576, dtype=torch.uint8 if kind == "raw" else torch.bfloat16,
                      device=DEV)
    ks = torch.tensor([0.7312], device=DEV) if mode == "fp8_scaled" else None
    vs = torch.tensor([1.37], device=DEV) if mode == "fp8_scaled" else None
    cs = None if kind in ("bfloat16", "raw") else torch.tensor([0.8125], device=DEV)
    dt = {"raw": "fp8", "fp8": "fp8", "fp8_e5m2": "fp8_e5m2", "bfloat16": "bfloat16"}[kind]
    kw = dict(v=dkvb[..., 128:], v_out=vo, mode=mk.MLA_PACK_KEY_V_FP8, k_scale=ks,
              v_scale=vs) if fp8 else {}
    mk.mla_ctx_kv_pack_gather(dkvb[..., :128], dws[:, 512:], key, cache.to(DEV), sl.to(DEV), out,
                              cache_scale=cs, kv_cache_dtype=dt, max_blocks=max_blocks, **kw)
    torch.cuda.synchronize()
    fmt = "e5m2" if kind == "fp8_e5m2" else "e4m3"
    ref_g = oracle.gather(cache_np, sl.numpy(), 0.8125 if cs is not None else 1.0,
                          raw=kind == "raw", fp8_format=fmt)
    assert np.array_equal(u8(out) if kind == "raw" else u16(out), ref_g), "gather part"
    rk, rv = oracle_pack(u16(kvb), u16(ws)[:, 512:], fp8, 0.7312 if ks is not None else 1.0,
                         1.37 if vs is not None else 1.0)
    assert np.array_equal(u8(key) if fp8 else u16(key), rk), "pack key"
    if fp8:
        assert np.array_equal(u8(vo), rv), "pack V"


@pytest.mark.timeout(300)
def test_pack_gather_joint_launch_context_workload(mk):
    """The chunked-context shape (8192 tokens x 64 heads packed, 8192 tokens
    gathered from a [512, 64, 576] fp8 cache): every byte against the oracle."""
    announce("pack + gather joint launch, C4 shape")
    d = synth.context_pack()
    kvb, ws = d["kvb"].to(DEV), d["workspace"].to(DEV)
    key = torch.empty(8192, 64, 192, dtype=torch.uint8, device=DEV)
    vo = torch.empty(8192, 64, 128, dtype=torch.uint8, device=DEV)
    out = torch.empty(8192, 576, dtype=torch.bfloat16, device=DEV)
    mk.mla_ctx_kv_pack_gather(kvb[..., :128], ws[:, 512:], key, d["cache"].to(DEV),
                              d["src_slots"].to(DEV), out, v=kvb[..., 128:], v_out=vo,
                              mode=mk.MLA_PACK_KEY_V_FP8,
                              cache_scale=torch.tensor([0.5], device=DEV))
    torch.cuda.synchronize()
    ref_g = oracle.gather(d["cache"].numpy(), d["src_slots"].numpy(), 0.5)
    assert np.array_equal(u16(out), ref_g)
    rk, rv = oracle_pack_full(u16(d["kvb"]), u16(d["workspace"])[:, 512:], True)
    assert np.array_equal(u8(key), rk) and np.array_equal(u8(vo), rv)


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
