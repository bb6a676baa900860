"""Largest launches each entry point accepts: the work-item counters are 32-bit,
so the pack, the gather and the merge are run with just under 2^31 items
(85-105 GB of device memory each) and sampled outputs -- the first rows, the
last rows and rows past 2^30 items -- are compared with the CPU oracle.  An
index overflow anywhere in the item -> (token, head, chunk) -> address chain
would put some of these rows in the wrong place.  Skipped when the device has
not enough free memory.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, announce, requires_gpu, u16, u8
from test_gpu_merge import merge_close

pytestmark = [pytest.mark.gpu, requires_gpu]

GB = 1 << 30


def need(nbytes):
    free, _ = torch.cuda.mem_get_info(DEV)
    if free < nbytes + 8 * GB:
        pytest.skip(f"needs {nbytes / GB:.0f} GiB free on the device, {free / GB:.0f} GiB free")


def random_bits(shape, dtype):
    """Random 16-bit patterns (bf16 view) or bytes, generated on the device."""
    if dtype == torch.bfloat16:
        return torch.randint(-32768, 32768, shape, dtype=torch.int16, device=DEV).view(dtype)
    return torch.randint(0, 256, shape, dtype=torch.uint8, device=DEV)


def sample(n, count, seed):
    r = np.random.default_rng(seed)
    idx = np.concatenate([np.arange(4), n - 1 - np.arange(4), r.integers(n // 2, n, count)])
    return np.unique(idx)


def test_pack_just_below_2_31_chunks(mk):
    T, H = 1677721, 64                         # T * H * (12 + 8) = 2^31 - 768 chunks
    assert T * H * 20 < (1 << 31)
    need(T * H * (512 + 320) + T * 128)
    announce("pack at the 2^31-chunk limit", T, H)
    torch.manual_seed(11)
    kvb = random_bits((T, H, 256), torch.bfloat16)
    kpe = random_bits((T, 64), torch.bfloat16)
    key = torch.empty(T, H, 192, dtype=torch.uint8, device=DEV)
    v8 = torch.empty(T, H, 128, dtype=torch.uint8, device=DEV)
    mk.mla_ctx_kv_pack(kvb[..., :128], kpe, key, v=kvb[..., 128:], v_out=v8,
                       mode=mk.MLA_PACK_KEY_V_FP8)
    torch.cuda.synchronize()
    rows = torch.from_numpy(sample(T, 60, 1)).to(DEV)
    kn = u16(kvb[rows])
    rk, rv = oracle.pack(kn[..., :128], u16(kpe[rows]), kn[..., 128:], mode=oracle.PACK_KEY_V_FP8)
    assert np.array_equal(u8(key[rows]), rk)
    assert np.array_equal(u8(v8[rows]), rv)
    del kvb, kpe, key, v8
    torch.cuda.empty_cache()


def test_gather_just_below_2_31_chunks(mk):
    T = (1 << 31) // 36 - 1                    # 36 chunks of 16 codes per 576-byte row
    nb = (T + 63) // 64
    need(nb * 64 * 576 + T * (1152 + 8))
    announce("gather at the 2^31-chunk limit", T)
    torch.manual_seed(12)
    cache = random_bits((nb, 64, 576), torch.uint8)
    slots = torch.randperm(nb * 64, device=DEV)[:T].contiguous()
    out = torch.empty(T, 576, dtype=torch.bfloat16, device=DEV)
    scale = torch.tensor([0.625], dtype=torch.float32, device=DEV)
    mk.mla_ctx_latent_gather(cache, slots, out, scale, "fp8")
    torch.cuda.synchronize()
    js = torch.from_numpy(sample(T, 60, 2)).to(DEV)
    src = cache.view(nb * 64, 576)[slots[js]]                # the sampled rows, in order
    mini = u8(src).reshape(-1, 1, 576)
    ref = oracle.gather(mini, np.arange(mini.shape[0], dtype=np.int64), 0.625)
    assert np.array_equal(u16(out[js]), ref)
    del cache, slots, out
    torch.cuda.empty_cache()


def test_merge_just_below_2_31_rows(mk):
    H, D = 64, 8
    T = ((1 << 31) - 32) // H                  # T * H = 2^31 - 64 rows
    need(2 * T * H * D * 2 + 2 * T * H * 4)
    announce("merge at the 2^31-row limit", T, H, D)
    torch.manual_seed(13)
    acc = torch.randn(T, H, D, dtype=torch.bfloat16, device=DEV)
    part = torch.randn(T, H, D, dtype=torch.bfloat16, device=DEV)
    lse = 3.0 * torch.randn(H, T, device=DEV)
    plse = 3.0 * torch.randn(H, T, device=DEV)
    ts = torch.from_numpy(sample(T, 40, 3)).to(DEV)
    a0, l0 = acc[ts].cpu(), lse[:, ts].cpu().numpy()
    mk.mla_ctx_merge_chunk(acc, lse, part, plse, mk.MLA_MERGE_ACCUMULATE)
    torch.cuda.synchronize()
    p0, pl0 = part[ts].cpu(), plse[:, ts].cpu().numpy()
    ro, rl = u16(a0).copy(), l0.copy()
    oracle.merge_chunk(ro, rl, u16(p0), pl0, oracle.MERGE_ACCUMULATE)
    merge_close(u16(acc[ts]), ro, a0, p0, l0, pl0)
    assert np.allclose(lse[:, ts].cpu().numpy(), rl, rtol=1e-6, atol=1e-6)
    del acc, part, lse, plse
    torch.cuda.empty_cache()


def test_stream_copy_is_a_byte_copy(mk):
    """The measurement copy moves every byte (sizes with a partial last
    workgroup, and one empty copy)."""
    announce("stream copy")
    g = torch.Generator(device=DEV)
    g.manual_seed(77)
    for n in (16, 4096 + 48, (1 << 24) + 16 * 37):
        src = torch.randint(0, 256, (n,), generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)
        dst = torch.zeros_like(src)
        mk.mla_stream_copy(dst, src)
        torch.cuda.synchronize()
        assert torch.equal(dst, src), n
    mk.mla_stream_copy(src[:0], dst[:0])


def test_stream_mix_is_a_chunk_xor(mk):
    """The mixed read:write measurement kernel: output chunk i is the XOR of
    input chunks r i .. r i + r - 1, for r = 1 to 4, with a partial last
    workgroup."""
    announce("stream mix")
    g = torch.Generator(device=DEV)
    g.manual_seed(78)
    n = 4096 + 48
    for r in (1, 2, 3, 4):
        src = torch.randint(-2**31, 2**31 - 1, (n * r // 4,), generator=g, device=DEV,
                            dtype=torch.int64).to(torch.int32)
        dst = torch.zeros(n // 4, dtype=torch.int32, device=DEV)
        mk.mla_stream_mix(dst, src, r)
        torch.cuda.synchronize()
        chunks = src.view(-1, r, 4).cpu()
        ref = chunks[:, 0].clone()
        for k in range(1, r):
            ref ^= chunks[:, k]
        assert torch.equal(dst.view(-1, 4).cpu(), ref), r


def test_mfma_rate_clock_readings(mk):
    """The matrix-core rate probe: every wavefront of every workgroup writes
    increasing shader-clock and real-time readings, and the issue interval
    and clock derived from them are in a physical range."""
    announce("mfma rate probe")
    cus = torch.cuda.get_device_properties(DEV).multi_processor_count
    clocks = torch.zeros(16 * cus, dtype=torch.int64, device=DEV)
    iters = 256
    mk.mla_mfma_rate(clocks, iters)
    torch.cuda.synchronize()
    c = clocks.view(-1, 4).cpu().numpy()
    assert (c[:, 1] > c[:, 0]).all() and (c[:, 3] > c[:, 2]).all()
    cycles = (c[:, 1] - c[:, 0]).astype(float)
    per_mfma = cycles.mean() / (iters * 12)
    ghz = cycles.sum() / (c[:, 3] - c[:, 2]).astype(float).sum() * 0.1
    announce(f"{per_mfma:.1f} cycles per MFMA at {ghz:.2f} GHz")
    assert 8 <= per_mfma <= 256 and 0.3 <= ghz <= 3.5
