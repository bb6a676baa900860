"""GPU parity of mla_kv_insert_grouped against the CPU oracle (bit-exact).

Workloads: the single-layer bf16 insert (16 tokens), the small-batch grouped
fp8 insert (5 layers x 4 tokens, token-major, shared slots with a -1), the
grouped-insert test shape of PR #55356 report (关键源码片段, test_cache.py:
5 layers, 42 tokens, block 16, 8 blocks, linspace scales, shared or not, auto /
fp8 / fp8_e4m3), the long-context insert at full size (5 x 16384 tokens into
[4096, 64, 576] caches, every cache byte against the oracle), and edge cases.  The exhaustive test feeds every
bf16 bit pattern through the gfx950 converter path.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_paged_insert_amd import synth
from gpu_util import DEV, announce, check_slots, requires_gpu, run_sliced, to_dev, u16, u8

pytestmark = [pytest.mark.gpu, requires_gpu]


def run_gpu(mk, d, dtype, check_strides=False):
    g = to_dev(d)
    if check_strides:
        assert g["kv_c"].stride() == d["kv_c"].stride()
        assert g["slot_mapping"].stride() == d["slot_mapping"].stride()
    caches = g["caches"]
    check_slots(d["slot_mapping"], d["caches"][0].shape[0] * d["block_size"])
    mk.mla_kv_insert_grouped(g["kv_c"], g["k_pe"], caches, g["slot_mapping"], g["block_size"],
                             caches[0].stride(0), caches[0].stride(1),
                             g["scales"] if dtype.startswith("fp8") else None, dtype)
    torch.cuda.synchronize()
    return caches


def np_cache(c):
    return u16(c) if c.dtype == torch.bfloat16 else u8(c)


def run_oracle(d, dtype):
    caches = [np_cache(c).copy() for c in d["caches"]]
    sm = d["slot_mapping"].numpy()
    oracle.insert_grouped(u16(d["kv_c"]), u16(d["k_pe"]), sm, caches,
                          d["scales"].numpy() if dtype.startswith("fp8") else None)
    return caches


def assert_same(gpu_caches, ref_caches):
    for l, (g, r) in enumerate(zip(gpu_caches, ref_caches)):
        gn = np_cache(g)
        if not np.array_equal(gn, r):
            bad = np.argwhere(gn != r)
            raise AssertionError(f"layer {l}: {len(bad)} elements differ, first at {bad[0]}")


@pytest.mark.parametrize("dtype", ["auto", "bfloat16"])
def test_single_layer_bf16(mk, dtype):
    announce("single_layer_bf16", dtype)
    d = synth.single_layer_bf16()
    assert_same(run_gpu(mk, d, dtype), run_oracle(d, dtype))


def test_small_batch_fp8_token_major_shared(mk):
    announce("small_batch_fp8")
    d = synth.small_batch_fp8()
    assert d["kv_c"].stride(0) == 512 and d["kv_c"].stride(1) == 2560   # token-major
    assert d["slot_mapping"].stride(0) == 0 and d["slot_mapping"][0, -1] == -1
    assert_same(run_gpu(mk, d, "fp8", check_strides=True), run_oracle(d, "fp8"))


@pytest.mark.parametrize("shared", [False, True])
@pytest.mark.parametrize("dtype", ["auto", "fp8", "fp8_e4m3"])
def test_grouped_test_shape(mk, shared, dtype):
    announce("grouped_test_shape", shared, dtype)
    d = synth.grouped_test_shape(shared=shared, fp8=dtype != "auto")
    gpu = run_gpu(mk, d, dtype)
    assert_same(gpu, run_oracle(d, dtype))
    # grouped == one single-layer launch per layer (the page's reference)
    per = [c.clone().to(DEV) for c in d["caches"]]
    for l in range(d["num_layers"]):
        mk.mla_kv_insert_grouped(
            d["kv_c"][l:l + 1].to(DEV), d["k_pe"][l:l + 1].to(DEV),
            [per[l]], d["slot_mapping"][l].contiguous().to(DEV), 16,
            per[l].stride(0), per[l].stride(1),
            d["scales"][l:l + 1].to(DEV) if dtype != "auto" else None, dtype)
    torch.cuda.synchronize()
    for a, b in zip(gpu, per):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


@pytest.mark.parametrize("R,P", [(256, 32), (128, 16), (512, 16), (512, 0)])
@pytest.mark.parametrize("dtype", ["bfloat16", "fp8"])
def test_other_row_shapes(mk, R, P, dtype):
    """Row shapes other than 512 + 64 (any multiples of 16) take the flat
    chunk kernel; 3 layers x 37 tokens, block 16, one skipped slot per layer."""
    announce("other_row_shapes", R, P, dtype)
    g = synth.gen(100 + R + P)
    L, T, bs, nb = 3, 37, 16, 8
    fp8 = dtype == "fp8"
    fill = synth.random_bytes if fp8 else synth.random_bf16_bits
    slots = torch.stack([synth.randperm(nb * bs, g)[:T] for _ in range(L)])
    slots[:, 5] = -1
    d = dict(kv_c=synth.bf16_normal((L, T, R), g), k_pe=synth.bf16_normal((L, T, P), g),
             caches=[fill((nb, bs, R + P + 16), g) for _ in range(L)],
             scales=torch.tensor([0.3, 1.7, -0.9], dtype=torch.float32) if fp8 else None,
             slot_mapping=slots, num_layers=L, num_tokens=T, block_size=bs)
    assert_same(run_gpu(mk, d, dtype), run_oracle(d, dtype))


def test_invalid_scales_raise(mk):
    """Scales on the host, non-contiguous, wrong count or dtype are refused."""
    announce("invalid_scales")
    d = to_dev(synth.grouped_test_shape(fp8=True))
    caches = d["caches"]
    ptrs = mk.cache_ptr_table(caches)     # the raw device table form
    before = [c.clone() for c in caches]

    def run(sc, dtype="fp8"):
        mk.mla_kv_insert_grouped(d["kv_c"], d["k_pe"], ptrs, d["slot_mapping"], 16,
                                 caches[0].stride(0), caches[0].stride(1), sc, dtype)

    for bad, msg in ((d["scales"].cpu(), "same CUDA device"),
                     (torch.ones(5, 2, device=DEV)[:, 0], "must be contiguous"),
                     (torch.ones(4, device=DEV), "one scale per layer"),
                     (torch.ones(5, device=DEV, dtype=torch.float64), "float32"),
                     (None, "needs kv_scales")):
        with pytest.raises(RuntimeError, match=msg):
            run(bad)
    with pytest.raises(RuntimeError, match="takes no kv_scales"):
        run(d["scales"], "auto")
    torch.cuda.synchronize()
    for a, b in zip(caches, before):
        assert torch.equal(a, b)


def test_exhaustive_bf16_patterns_through_fp8_converter(mk):
    """All 65536 bf16 bit patterns (NaN, Inf, subnormals, +-0 included),
    quantised with several per-layer scales, equal the oracle bit for bit."""
    announce("exhaustive_converter")
    scales = torch.tensor([1.0, 0.5, 0.05, 0.25, 0.7312, 1.9999, 1.3, -0.7312], dtype=torch.float32)
    L = scales.numel()
    rows = 65536 // 512 + 1
    bits = np.arange(rows * 576, dtype=np.int64) % 65536
    x = torch.from_numpy(bits.astype(np.int32)).to(torch.int16).view(torch.bfloat16).reshape(rows, 576)
    kv_c = x[:, :512].unsqueeze(0).expand(L, rows, 512)
    k_pe = x[:, 512:].unsqueeze(0).expand(L, rows, 64)
    caches = [torch.zeros(rows, 1, 576, dtype=torch.uint8) for _ in range(L)]
    sm = torch.arange(rows, dtype=torch.int64).reshape(1, rows).expand(L, rows)
    d = dict(kv_c=kv_c, k_pe=k_pe, caches=caches, scales=scales, slot_mapping=sm,
             num_layers=L, num_tokens=rows, block_size=1)
    gpu = run_gpu(mk, d, "fp8")
    for l in range(L):
        ref = oracle.quantize(u16(x), float(scales[l])).reshape(rows, 1, 576)
        got = np_cache(gpu[l])
        if not np.array_equal(got, ref):
            i = np.argwhere(got != ref)[0]
            b = int(u16(x)[i[0], i[2]])
            raise AssertionError(f"scale {float(scales[l])}: bf16 0x{b:04x} -> "
                                 f"gpu 0x{got[tuple(i)]:02x}, oracle 0x{ref[tuple(i)]:02x}")



@pytest.mark.parametrize("dtype", ["fp8", "fp8_e5m2"])
def test_extreme_scales_through_fp8_converter(mk, dtype):
    """All 65536 bf16 patterns quantised with scales at and inside the edges
    of the range where the quotient is exact (2^-85 <= |s| < 2^126, the
    stated precondition): the smallest, the largest fp32 below 2^126, odd
    significands and a negative scale; e4m3fn and e5m2 codes equal the
    oracle's (one IEEE fp32 division, then the format's rounding) bit for
    bit, so the device's reciprocal-and-FMA quotient, its subnormal results
    and the saturation behave as on the host across the whole range."""
    announce("extreme scales", dtype)
    f = np.float32
    scales = torch.tensor([f(2.0 ** -85), f(1.5 * 2.0 ** -85), f(1e-20), f(3e-9),
                           f(1.2345678 * 2.0 ** 40), f(1e30),
                           np.nextafter(f(2.0 ** 126), f(0)), f(-1.7 * 2.0 ** -85)],
                          dtype=torch.float32)
    assert float(scales.abs().min()) >= 2.0 ** -85 and float(scales.abs().max()) < 2.0 ** 126
    L = scales.numel()
    rows = 65536 // 512 + 1
    bits = np.arange(rows * 576, dtype=np.int64) % 65536
    x = torch.from_numpy(bits.astype(np.int32)).to(torch.int16).view(torch.bfloat16).reshape(rows, 576)
    d = dict(kv_c=x[:, :512].unsqueeze(0).expand(L, rows, 512),
             k_pe=x[:, 512:].unsqueeze(0).expand(L, rows, 64),
             caches=[torch.zeros(rows, 1, 576, dtype=torch.uint8) for _ in range(L)],
             scales=scales, slot_mapping=torch.arange(rows, dtype=torch.int64).reshape(1, rows)
             .expand(L, rows), num_layers=L, num_tokens=rows, block_size=1)
    gpu = run_gpu(mk, d, dtype)
    quant = oracle.quantize if dtype == "fp8" else oracle.quantize_e5m2
    for l in range(L):
        ref = quant(u16(x), float(scales[l])).reshape(rows, 1, 576)
        got = np_cache(gpu[l])
        if not np.array_equal(got, ref):
            i = np.argwhere(got != ref)[0]
            b = int(u16(x)[i[0], i[2]])
            raise AssertionError(f"scale {float(scales[l])!r}: bf16 0x{b:04x} -> "
                                 f"gpu 0x{got[tuple(i)]:02x}, oracle 0x{ref[tuple(i)]:02x}")
        announce(f"scale {float(scales[l]):.4g}: {int((ref & 0x7F).astype(bool).sum())} "
                 "nonzero codes, all equal")


def test_padded_layout_and_block_size_one(mk):
    announce("padded_layout")
    g = torch.Generator().manual_seed(77)
    L, T = 3, 50
    big = [torch.randint(0, 256, (12, 5, 640), generator=g, dtype=torch.int32).to(torch.uint8)
           for _ in range(L)]
    views = [b[:, :4, :] for b in big]           # block stride 5*640, entry stride 640
    kv = synth.bf16_normal((T, L, 512), g)       # token-major
    pe = synth.bf16_normal((T, L, 64), g)
    T = 40
    kv, pe = kv[:T], pe[:T]
    sm = torch.stack([torch.randperm(48, generator=g)[:T] for _ in range(L)])
    sm[:, ::7] = -3
    d = dict(kv_c=kv.permute(1, 0, 2), k_pe=pe.permute(1, 0, 2), caches=views,
             scales=torch.tensor([0.9, 1.1, 0.6]), slot_mapping=sm, num_layers=L,
             num_tokens=T, block_size=4)
    gbig = [b.to(DEV) for b in big]
    gv = [b[:, :4, :] for b in gbig]
    check_slots(sm, 12 * 4)
    mk.mla_kv_insert_grouped(d["kv_c"].to(DEV), d["k_pe"].to(DEV), gv,
                             sm.to(DEV), 4, gv[0].stride(0), gv[0].stride(1),
                             d["scales"].to(DEV), "fp8")
    torch.cuda.synchronize()
    ref = [b.numpy().copy() for b in big]
    oracle.insert_grouped(u16(d["kv_c"]), u16(d["k_pe"]), sm.numpy(),
                          [r[:, :4, :] for r in ref], d["scales"].numpy())
    for l in range(L):
        assert np.array_equal(u8(gbig[l]), ref[l])

    # block_size 1, bf16 cache, every slot skipped but one
    c = torch.zeros(8, 1, 576, dtype=torch.bfloat16, device=DEV)
    s = torch.full((1, 3), -1, dtype=torch.int64, device=DEV)
    s[0, 1] = 5
    kvc = torch.randn(1, 3, 512, device=DEV).to(torch.bfloat16)
    kpe = torch.randn(1, 3, 64, device=DEV).to(torch.bfloat16)
    mk.mla_kv_insert_grouped(kvc, kpe, [c], s, 1, 576, 576, None, "auto")
    torch.cuda.synchronize()
    assert torch.equal(c[5, 0, :512], kvc[0, 1]) and torch.equal(c[5, 0, 512:], kpe[0, 1])
    assert int((c.view(torch.int16) != 0).any(dim=-1).sum()) == 1


def test_zero_tokens_is_a_noop(mk):
    announce("zero_tokens")
    c = torch.zeros(2, 4, 576, dtype=torch.uint8, device=DEV)
    mk.mla_kv_insert_grouped(torch.empty(5, 0, 512, dtype=torch.bfloat16, device=DEV),
                             torch.empty(5, 0, 64, dtype=torch.bfloat16, device=DEV),
                             [c] * 5, torch.empty(5, 0, dtype=torch.int64, device=DEV),
                             4, c.stride(0), c.stride(1), torch.ones(5, device=DEV), "fp8")
    torch.cuda.synchronize()
    assert not c.any()


def oracle_insert_layers_threaded(d, fp8_format="e4m3"):
    """The oracle's grouped insert, one layer per host thread (the grouped
    insert is L independent single-layer inserts, which the oracle's own
    pins establish), into copies of the initial caches."""
    caches = [np_cache(c).copy() for c in d["caches"]]
    kv, pe, sm = u16(d["kv_c"]), u16(d["k_pe"]), d["slot_mapping"].numpy()
    sc = d["scales"].numpy()

    def layers(a, b):
        for l in range(a, b):
            oracle.insert_grouped(kv[l:l + 1], pe[l:l + 1], sm[l:l + 1], [caches[l]],
                                  sc[l:l + 1], fp8_format=fp8_format)
    run_sliced(layers, d["num_layers"], parts=d["num_layers"])
    return caches


@pytest.mark.timeout(300)
def test_long_context_insert_full_size(mk):
    """5 layers x 16384 tokens into [4096, 64, 576] fp8 caches: every byte of
    the five 151 MB caches against the oracle (written rows and untouched
    ones)."""
    announce("long_context_insert_full")
    d = synth.long_context_insert()
    gpu = run_gpu(mk, d, "fp8")
    assert_same(gpu, oracle_insert_layers_threaded(d))


def test_prepared_insert_matches_and_follows_contents(mk):
    """PreparedInsert re-enqueues the checked insert; new input contents are
    picked up on every call."""
    announce("prepared insert")
    d = to_dev(synth.small_batch_fp8())
    caches = d["caches"]
    a = [c.clone() for c in caches]
    plan = mk.prepare_insert_grouped(d["kv_c"], d["k_pe"], a, d["slot_mapping"], 64,
                                     a[0].stride(0), a[0].stride(1), d["scales"], "fp8")
    plan()
    b = [c.clone() for c in caches]
    mk.mla_kv_insert_grouped(d["kv_c"], d["k_pe"], b, d["slot_mapping"], 64, b[0].stride(0),
                             b[0].stride(1), d["scales"], "fp8")
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    d["kv_c"].mul_(-1)            # same storage, new contents
    plan()
    mk.mla_kv_insert_grouped(d["kv_c"], d["k_pe"], b, d["slot_mapping"], 64, b[0].stride(0),
                             b[0].stride(1), d["scales"], "fp8")
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
