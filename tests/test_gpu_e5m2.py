"""GPU parity of the fp8_e5m2 cache dtype against the CPU oracle.

Page: "PR #55356 完整报告", 实现拆解 item 3 and 关键源码片段 (cache_kernels.cu,
test_cache.py): the grouped insert dispatches "fp8_e5m2" to its own template
instance and its test covers auto / fp8 / fp8_e5m2 bit for bit against the
per-layer insert; the page's ROCm build refuses the dtype, gfx950 converts it
natively (v_cvt_pk_bf8_f32 / v_cvt_pk_f32_bf8).

Bars: insert and gather bit-exact; the epilogue as for e4m3fn (rows within
1 bf16 ulp, codes within 1 code, identical codes wherever the rows agree).
Workloads: every bf16 bit pattern through the converter at 8 scales (one
negative, one small enough to saturate), the grouped-insert test shape of the
page, the long-context insert at full size (every byte), non-MLA row shapes, the
fused epilogue shape, and the gather of every code at 6 scales.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_paged_insert_amd import synth
from gpu_util import (DEV, announce, bf16_ulps, check_slots, fp8_codes_apart, requires_gpu,
                      run_sliced, to_dev, u16, u8)

pytestmark = [pytest.mark.gpu, requires_gpu]

E5 = "fp8_e5m2"


def run_insert(mk, d):
    g = to_dev(d)
    caches = g["caches"]
    check_slots(d["slot_mapping"], d["caches"][0].shape[0] * d["block_size"])
    mk.mla_kv_insert_grouped(g["kv_c"], g["k_pe"], caches, g["slot_mapping"], g["block_size"],
                             caches[0].stride(0), caches[0].stride(1), g["scales"], E5)
    torch.cuda.synchronize()
    return caches


def oracle_insert(d):
    caches = [u8(c).copy() for c in d["caches"]]
    oracle.insert_grouped(u16(d["kv_c"]), u16(d["k_pe"]), d["slot_mapping"].numpy(), caches,
                          d["scales"].numpy(), fp8_format="e5m2")
    return caches


def assert_same(gpu, ref):
    for l, (g, r) in enumerate(zip(gpu, ref)):
        gn = u8(g)
        if not np.array_equal(gn, r):
            bad = np.argwhere(gn != r)
            raise AssertionError(f"layer {l}: {len(bad)} bytes differ, first at {bad[0]}")


# ------------------------------------------------------------------ insert --
def test_every_bf16_pattern_through_the_e5m2_converter(mk):
    announce("e5m2 exhaustive converter")
    scales = torch.tensor([1.0, 0.5, 0.05, 0.7312, 1.9999, 1.3, -0.7312, 3.0e-3],
                          dtype=torch.float32)
    L = scales.numel()
    rows = 65536 // 512 + 1
    bits = np.arange(rows * 576, dtype=np.int64) % 65536
    x = torch.from_numpy(bits.astype(np.int32)).to(torch.int16).view(torch.bfloat16)
    x = x.reshape(rows, 576)
    d = dict(kv_c=x[:, :512].unsqueeze(0).expand(L, rows, 512),
             k_pe=x[:, 512:].unsqueeze(0).expand(L, rows, 64),
             caches=[torch.zeros(rows, 1, 576, dtype=torch.uint8) for _ in range(L)],
             scales=scales,
             slot_mapping=torch.arange(rows, dtype=torch.int64).reshape(1, rows).expand(L, rows),
             num_layers=L, num_tokens=rows, block_size=1)
    gpu = run_insert(mk, d)
    for l in range(L):
        ref = oracle.quantize_e5m2(u16(x), float(scales[l])).reshape(rows, 1, 576)
        got = u8(gpu[l])
        if not np.array_equal(got, ref):
            i = np.argwhere(got != ref)[0]
            b = int(u16(x)[i[0], i[2]])
            raise AssertionError(f"scale {float(scales[l])}: bf16 0x{b:04x} -> "
                                 f"gpu 0x{got[tuple(i)]:02x}, oracle 0x{ref[tuple(i)]:02x}")


@pytest.mark.parametrize("shared", [False, True])
def test_grouped_test_shape(mk, shared):
    announce("e5m2 grouped test shape", shared)
    d = synth.grouped_test_shape(shared=shared, fp8=True)
    gpu = run_insert(mk, d)
    assert_same(gpu, oracle_insert(d))
    # grouped == one single-layer launch per layer (the page's reference)
    per = [c.clone().to(DEV) for c in d["caches"]]
    g = to_dev(d)
    for l in range(d["num_layers"]):
        mk.mla_kv_insert_grouped(g["kv_c"][l:l + 1], g["k_pe"][l:l + 1], [per[l]],
                                 g["slot_mapping"][l:l + 1].contiguous(), 16, per[l].stride(0),
                                 per[l].stride(1), g["scales"][l:l + 1].contiguous(), E5)
    torch.cuda.synchronize()
    for a, b in zip(gpu, per):
        assert torch.equal(a, b)


@pytest.mark.timeout(300)
def test_long_context_insert_full_size(mk):
    """5 x 16384 tokens into [4096, 64, 576] e5m2 caches: every byte of the
    five caches against the oracle, one layer per host thread."""
    announce("e5m2 long-context insert")
    d = synth.long_context_insert()
    gpu = run_insert(mk, d)
    caches = [u8(c).copy() for c in d["caches"]]
    kv, pe, sm = u16(d["kv_c"]), u16(d["k_pe"]), d["slot_mapping"].numpy()
    sc = d["scales"].numpy()

    def layers(a, b):
        for l in range(a, b):
            oracle.insert_grouped(kv[l:l + 1], pe[l:l + 1], sm[l:l + 1], [caches[l]],
                                  sc[l:l + 1], fp8_format="e5m2")
    run_sliced(layers, d["num_layers"], parts=d["num_layers"])
    assert_same(gpu, caches)


@pytest.mark.parametrize("R,P", [(256, 32), (512, 16)])
def test_other_row_shapes(mk, R, P):
    announce("e5m2 other row shapes", R, P)
    g = synth.gen(200 + R + P)
    L, T, bs, nb = 3, 37, 16, 8
    slots = torch.stack([synth.randperm(nb * bs, g)[:T] for _ in range(L)])
    slots[:, 5] = -1
    d = dict(kv_c=synth.bf16_normal((L, T, R), g, std=500.0),
             k_pe=synth.bf16_normal((L, T, P), g, std=500.0),
             caches=[synth.random_bytes((nb, bs, R + P + 16), g) for _ in range(L)],
             scales=torch.tensor([0.3, 1.7, -0.009], dtype=torch.float32),
             slot_mapping=slots, num_layers=L, num_tokens=T, block_size=bs)
    assert_same(run_insert(mk, d), oracle_insert(d))


# ---------------------------------------------------------------- epilogue --
def test_epilogue_context_shape(mk):
    announce("e5m2 epilogue C3 shape")
    d = synth.context_epilogue(with_gemm=False, fp8=True)
    L, T = d["num_layers"], d["num_tokens"]
    g = to_dev(d)
    cs = torch.empty(T, 2 * 64, dtype=torch.float32, device=DEV)
    mk.mla_rope_cos_sin_cache(cs, T, 64, d["rope_base"])
    rows = torch.empty(L, T, 576, dtype=torch.bfloat16, device=DEV)
    caches = g["caches"]
    mk.mla_ctx_kv_epilogue(g["all_kv"], g["gamma"], d["eps"], g["positions"], cs, caches,
                           g["slot_mapping"], 64, caches[0].stride(0), caches[0].stride(1),
                           g["scales"], E5, dbg_rows=rows)
    torch.cuda.synchronize()
    ref_caches = [u8(c).copy() for c in d["caches"]]
    ref_rows = oracle.ctx_kv_epilogue(u16(d["all_kv"]), u16(d["gamma"]), d["eps"],
                                      d["positions"].numpy(), d["slot_mapping"].numpy(),
                                      ref_caches, d["scales"].numpy(), rope_base=d["rope_base"],
                                      fp8_format="e5m2")
    got_rows = u16(rows)
    assert bf16_ulps(got_rows, ref_rows).max() <= 1
    sm = d["slot_mapping"].numpy()
    for l in range(L):
        got = u8(caches[l]).reshape(-1, 576)
        ref = ref_caches[l].reshape(-1, 576)
        init = u8(d["caches"][l]).reshape(-1, 576)
        touched = np.zeros(got.shape[0], bool)
        touched[sm[l]] = True
        assert np.array_equal(got[~touched], init[~touched]), f"layer {l}: stray writes"
        g_rows, r_rows = got[sm[l]], ref[sm[l]]
        assert fp8_codes_apart(g_rows, r_rows).max() <= 1, f"layer {l}"
        agree = got_rows[l] == ref_rows[l]
        assert np.array_equal(g_rows[agree], r_rows[agree]), f"layer {l}"
    # quantisation and scatter on their own: the oracle's e5m2 insert of the
    # GPU's own rows gives the GPU's caches bit for bit
    dbg = [u8(c).copy() for c in d["caches"]]
    oracle.insert_grouped(got_rows[:, :, :512], got_rows[:, :, 512:], sm, dbg,
                          d["scales"].numpy(), fp8_format="e5m2")
    for l in range(L):
        assert np.array_equal(u8(caches[l]), dbg[l]), f"layer {l}: insert of the GPU rows"


# ------------------------------------------------------------------ gather --
@pytest.mark.parametrize("scale", [0.5, 1.0, 0.7312, 1.9999, 3.0e-3, -0.37])
def test_gather_every_code(mk, scale):
    """All 256 e5m2 codes (both infinities and the NaNs included) dequantised."""
    announce("e5m2 gather codes", scale)
    codes = torch.arange(256 * 9, dtype=torch.int32).remainder(256).to(torch.uint8)
    cache = codes.reshape(4, 1, 576)
    slots = torch.tensor([2, 0, 3, 1], dtype=torch.int64)
    out = torch.empty(4, 576, dtype=torch.bfloat16, device=DEV)
    mk.mla_ctx_latent_gather(cache.to(DEV), slots.to(DEV), out,
                             torch.tensor([scale], dtype=torch.float32, device=DEV), E5)
    ref = oracle.gather(cache.numpy(), slots.numpy(), scale, fp8_format="e5m2")
    got = u16(out)
    if not np.array_equal(got, ref):
        i = np.argwhere(got != ref)[0]
        code = int(cache.view(4, 576).numpy()[slots[i[0]], i[1]])
        raise AssertionError(f"code 0x{code:02x}: gpu 0x{got[tuple(i)]:04x}, "
                             f"oracle 0x{ref[tuple(i)]:04x}")


def test_gather_workload_and_raw(mk):
    announce("e5m2 gather workload + raw")
    d = synth.context_pack()
    cache, slots = d["cache"].to(DEV), d["src_slots"].to(DEV)
    ws = torch.empty(8192, 576, dtype=torch.bfloat16, device=DEV)
    mk.mla_ctx_latent_gather(cache, slots, ws, torch.tensor([0.5], device=DEV), E5)
    ref = oracle.gather(d["cache"].numpy(), d["src_slots"].numpy(), 0.5, fp8_format="e5m2")
    assert np.array_equal(u16(ws), ref)
    raw = torch.empty(8192, 576, dtype=torch.uint8, device=DEV)
    mk.mla_ctx_latent_gather(cache, slots, raw, None, E5)
    assert np.array_equal(u8(raw), oracle.gather(d["cache"].numpy(), d["src_slots"].numpy(),
                                                 raw=True, fp8_format="e5m2"))
    with pytest.raises(RuntimeError):          # e4m3fn-typed output for an e5m2 cache
        mk.mla_ctx_latent_gather(cache, slots, raw.view(torch.float8_e4m3fn), None, E5)
