"""Pins for the oracle's projection, RMSNorm, RoPE, epilogue, gather and pack.

Closed forms and invariants chosen so a dropped term, a wrong sign, a wrong
pairing or index, or a transposed operand fails at least one test:
  * RMSNorm: one-hot rows (pin the mean over n and the gamma index), exact
    power-of-two scale invariance at eps = 0, the eps term on a constant row.
  * RoPE: position 0 is the identity; one-hot inputs at pairs whose angle is
    exactly 1 rad pin the frequency exponent, the (i, i + d/2) pairing and the
    rotation's sign; rotation composes and preserves pair norms.
  * Projection: float64 matmul (library), one-hot selection weights (exact
    column copies), [N, K] vs [K, N] addressing.
  * Gather / pack: torch indexing, concat and e4m3fn casts (library routines).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from fp8_paged_insert_amd import synth

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))


def u16(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf(v):
    """bf16 bits of a float value (library cast of an f32 value)."""
    return int(torch.tensor([v], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)[0])


def bf16_ulp_dist(a, b):
    """Distance in bf16 ulps between bit patterns (ordered-integer mapping)."""
    def key(x):
        x = np.asarray(x, np.int64)
        return np.where(x & 0x8000, 0x8000 - (x & 0x7FFF), 0x8000 + (x & 0x7FFF))
    return np.abs(key(a) - key(b))


# ------------------------------------------------------------------ RMSNorm --
def test_rmsnorm_one_hot(orc):
    n = 512
    gamma = np.full(n, bf(1.0), np.uint16)
    gamma[7] = bf(0.75)
    for k, c in [(7, 3.0), (100, -0.5), (511, 2.0 ** -10)]:
        x = np.zeros(n, np.uint16)
        x[k] = bf(c)
        y = orc.rmsnorm_row(x, gamma, 0.0)
        g = f32(gamma[k])
        expect = math.copysign(math.sqrt(n), c) * g   # c / sqrt(c^2 / n) * g
        assert y[k] == orc.f64_to_bf16(np.array([expect]))[0]
        assert not np.delete(y, k).any() or np.all((np.delete(y, k) & 0x7FFF) == 0)


def test_rmsnorm_constant_row_eps(orc):
    """Constant row c: y = c / sqrt(c^2 + eps) * gamma, eps visible for small c."""
    n = 512
    gamma = np.full(n, bf(1.25), np.uint16)
    eps = np.float32(1e-6)
    for c in [1.0, 2.0 ** -9, 2.0 ** -11]:
        x = np.full(n, bf(c), np.uint16)
        y = orc.rmsnorm_row(x, gamma, float(eps))
        expect = c / math.sqrt(c * c + float(eps)) * 1.25
        assert np.all(y == orc.f64_to_bf16(np.array([expect]))[0])
    # the eps term matters: at c = 2^-11 (c^2 ~ 2.4e-7 < eps) y is far below 1.25
    assert f32(y[0]) < 0.6          # 1.25 without eps


def test_rmsnorm_power_of_two_scale_invariance(orc):
    g = torch.Generator().manual_seed(3)
    x = u16(torch.randn(512, generator=g).to(torch.bfloat16))
    gamma = u16(torch.empty(512).uniform_(0.8, 1.2, generator=g).to(torch.bfloat16))
    y1 = orc.rmsnorm_row(x, gamma, 0.0)
    for k in (-3, 1, 4):
        xs = u16((torch.from_numpy(f32(x).copy()) * 2.0 ** k).to(torch.bfloat16))
        assert np.array_equal(orc.rmsnorm_row(xs, gamma, 0.0), y1)


def test_rmsnorm_matches_f64_formula(orc):
    g = torch.Generator().manual_seed(4)
    for _ in range(20):
        x = torch.randn(512, generator=g).to(torch.bfloat16)
        gm = torch.empty(512).uniform_(0.8, 1.2, generator=g).to(torch.bfloat16)
        x64, g64 = x.double(), gm.double()
        ref = x64 * torch.rsqrt((x64 * x64).mean() + float(np.float32(1e-6))) * g64
        ours = orc.rmsnorm_row(u16(x), u16(gm), 1e-6)
        assert bf16_ulp_dist(ours, orc.f64_to_bf16(ref.numpy())).max() == 0



def test_rmsnorm_special_values(orc):
    """IEEE consequences of the definition x * (mean x^2 + eps)^-1/2 * gamma:
    an all-zero row gives zeros carrying the signs of x * gamma; a NaN makes
    every output NaN; an infinite element makes the scale 0, so it becomes
    NaN (Inf * 0) and every finite element a signed zero."""
    n = 512
    gamma = np.full(n, bf(1.0), np.uint16)
    gamma[3] = bf(-2.0)
    nan_bits = lambda y: ((y & 0x7F80) == 0x7F80) & ((y & 0x7F) != 0)
    x = np.zeros(n, np.uint16)
    x[1::2] = 0x8000                                  # -0
    y = orc.rmsnorm_row(x, gamma, 1e-6)
    sign = (x >> 15) ^ (gamma >> 15)
    assert np.array_equal(y, (sign << 15).astype(np.uint16))
    g = torch.Generator().manual_seed(6)
    base = u16(torch.randn(n, generator=g).to(torch.bfloat16))
    xn = base.copy()
    xn[200] = 0x7FC0
    assert nan_bits(orc.rmsnorm_row(xn, gamma, 1e-6)).all()
    for inf in (0x7F80, 0xFF80):
        xi = base.copy()
        xi[10] = inf
        y = orc.rmsnorm_row(xi, gamma, 1e-6)
        assert nan_bits(y[10])
        rest = np.delete(np.arange(n), 10)
        assert not (y[rest] & 0x7FFF).any()
        assert np.array_equal(y[rest] >> 15, (xi[rest] >> 15) ^ (gamma[rest] >> 15))


# --------------------------------------------------------------------- RoPE --
def test_rope_position_zero_is_identity(orc):
    g = torch.Generator().manual_seed(5)
    x = u16(torch.randn(64, generator=g).to(torch.bfloat16))
    assert np.array_equal(orc.rope_row(x, 0), x)


@pytest.mark.parametrize("i,pos", [(0, 1), (8, 10), (16, 100), (24, 1000)])
def test_rope_one_hot_unit_angle(orc, i, pos):
    """theta_i = pos * 10000^(-2i/64) = 1 rad for these (i, pos) pairs."""
    d, half = 64, 32
    c, s = math.cos(1.0), math.sin(1.0)
    x = np.zeros(d, np.uint16)
    x[i] = bf(1.0)
    y = orc.rope_row(x, pos)
    expect = np.zeros(d, np.uint16)
    expect[i] = orc.f64_to_bf16(np.array([c]))[0]
    expect[i + half] = orc.f64_to_bf16(np.array([s]))[0]
    assert np.array_equal(y & 0x7FFF, expect & 0x7FFF) and (y[i + half] & 0x8000) == 0
    x = np.zeros(d, np.uint16)
    x[i + half] = bf(1.0)
    y = orc.rope_row(x, pos)
    assert y[i] == orc.f64_to_bf16(np.array([-s]))[0]
    assert y[i + half] == orc.f64_to_bf16(np.array([c]))[0]


def test_rope_last_pair_frequency(orc):
    """Pair 31 turns at 10000^(-62/64) rad per position."""
    pos = 4095
    theta = pos * 10000.0 ** (-62.0 / 64.0)
    x = np.zeros(64, np.uint16)
    x[31] = bf(1.0)
    y = orc.rope_row(x, pos)
    assert y[31] == orc.f64_to_bf16(np.array([math.cos(theta)]))[0]
    assert y[63] == orc.f64_to_bf16(np.array([math.sin(theta)]))[0]


def test_rope_norm_and_composition(orc):
    g = torch.Generator().manual_seed(6)
    for _ in range(20):
        x = u16(torch.randn(64, generator=g).to(torch.bfloat16))
        p1, p2 = [int(v) for v in torch.randint(0, 2048, (2,), generator=g)]
        y = orc.rope_row(x, p1)
        xf, yf = f32(x).astype(np.float64), f32(y).astype(np.float64)
        n_in = xf[:32] ** 2 + xf[32:] ** 2
        n_out = yf[:32] ** 2 + yf[32:] ** 2
        assert np.all(np.abs(n_out - n_in) <= 2 ** -7 * n_in + 1e-30)
        z = orc.rope_row(y, p2)
        w = orc.rope_row(x, p1 + p2)
        assert np.all(np.abs(f32(z) - f32(w)) <= 2 ** -6 * np.abs(f32(w)) + 2 ** -6 * np.abs(xf).max())


# --------------------------------------------------------------- projection --
def test_gemm_matches_f64_matmul(orc):
    g = torch.Generator().manual_seed(8)
    T, K, N = 9, 200, 37
    x = torch.randn(T, K, generator=g).to(torch.bfloat16)
    w = (0.02 * torch.randn(K, N, generator=g)).to(torch.bfloat16)
    ref = orc.f64_to_bf16((x.double() @ w.double()).numpy())
    ours = orc.gemm_rows(u16(x), u16(w))
    assert bf16_ulp_dist(ours, ref).max() <= 1
    assert (ours == ref).mean() > 0.99


def test_gemm_selection_matrix_copies_columns(orc):
    g = torch.Generator().manual_seed(9)
    T, K, N = 6, 64, 48
    x = torch.randn(T, K, generator=g).to(torch.bfloat16)
    perm = torch.randperm(K, generator=g)[:N]
    w = torch.zeros(K, N)
    w[perm, torch.arange(N)] = 1.0
    ours = orc.gemm_rows(u16(x), u16(w.to(torch.bfloat16)))
    assert np.array_equal(ours, u16(x)[:, perm.numpy()])


def test_gemm_nk_layout_and_row_subset(orc):
    g = torch.Generator().manual_seed(10)
    T, K, N = 8, 96, 40
    x = u16(torch.randn(T, K, generator=g).to(torch.bfloat16))
    w_kn = u16((0.05 * torch.randn(K, N, generator=g)).to(torch.bfloat16))
    w_nk = np.ascontiguousarray(w_kn.T)
    full = orc.gemm_rows(x, w_kn)
    via_nk = orc.gemm_rows(x, w_nk.T)      # same matrix through [N, K] storage
    assert np.array_equal(full, via_nk)
    rows = np.array([7, 0, 3], np.int64)
    assert np.array_equal(orc.gemm_rows(x, w_kn, rows), full[rows])


def test_fused_projection_flop_reduction_closed_form():
    """One KV-only projection (L x 576 rows) instead of L full Q+KV ones (L x 2112)."""
    v = GOLDEN["fused_projection_rows"]
    red = 1 - (v["layers"] * v["kv_width"]) / (v["layers"] * v["qkv_a_width"])
    assert round(100 * red, 1) == v["flop_reduction_percent"]


# ----------------------------------------------------------------- epilogue --
def test_epilogue_rows_address_layer_and_token(orc):
    """One-hot rows identify (token, layer) after norm; one-hot k_pe at pair 0
    identifies the token's position after RoPE."""
    T, L, R, P = 6, 3, 512, 64
    all_kv = np.zeros((T, L, R + P), np.uint16)
    for t in range(T):
        for l in range(L):
            all_kv[t, l, (7 * t + 31 * l) % R] = bf(1.0)
            all_kv[t, l, R] = bf(1.0)
    gamma = np.full((L, R), bf(1.0), np.uint16)
    pos = np.arange(T, dtype=np.int64) * 3
    rows = orc.ctx_kv_epilogue(all_kv, gamma, 0.0, pos, None, None)
    for l in range(L):
        for t in range(T):
            k = (7 * t + 31 * l) % R
            assert rows[l, t, k] == orc.f64_to_bf16(np.array([math.sqrt(R)]))[0]
            assert np.count_nonzero(rows[l, t, :R] & 0x7FFF) == 1
            assert rows[l, t, R] == orc.f64_to_bf16(np.array([math.cos(pos[t])]))[0]
            assert rows[l, t, R + 32] == orc.f64_to_bf16(np.array([math.sin(pos[t])]))[0]


def test_epilogue_is_norm_rope_then_grouped_insert(orc):
    d = synth.context_epilogue("cpu", num_tokens=40, num_blocks=4, with_gemm=False)
    L, T = d["num_layers"], d["num_tokens"]
    all_kv = u16(d["all_kv"])
    gamma = u16(d["gamma"])
    pos = d["positions"].numpy()
    sm = d["slot_mapping"].numpy()
    caches = [c.clone().numpy() for c in d["caches"]]
    rows = orc.ctx_kv_epilogue(all_kv, gamma, d["eps"], pos, sm, caches,
                               d["scales"].numpy())
    for l in range(L):
        for t in range(T):
            assert np.array_equal(rows[l, t, :512], orc.rmsnorm_row(all_kv[t, l, :512], gamma[l], d["eps"]))
            assert np.array_equal(rows[l, t, 512:], orc.rope_row(all_kv[t, l, 512:], pos[t]))
    expect = [c.clone().numpy() for c in d["caches"]]
    orc.insert_grouped(rows[:, :, :512], rows[:, :, 512:], sm, expect, d["scales"].numpy())
    for l in range(L):
        assert np.array_equal(caches[l], expect[l])


# ------------------------------------------------------------------- gather --
@pytest.mark.parametrize("fp8", [True, False])
def test_gather_matches_torch_indexing(orc, fp8):
    g = torch.Generator().manual_seed(12)
    nb, bs, W, T = 6, 8, 576, 30
    if fp8:
        cache = synth.finite_e4m3_codes((nb, bs, W), g)
    else:
        cache = synth.random_bf16_bits((nb, bs, W), g).view(torch.int16)
    blocks = torch.randperm(nb, generator=g)[:4]
    slots = synth.block_table_slots(blocks, bs, T)
    rows = cache.view(nb * bs, W)[slots]
    if fp8:
        ref = (rows.view(torch.float8_e4m3fn).float() * torch.tensor(0.5)).to(torch.bfloat16)
        ref = u16(ref)
        ours = orc.gather(cache.numpy(), slots.numpy(), scale=0.5)
    else:
        ref = rows.numpy().view(np.uint16)
        ours = orc.gather(cache.numpy().view(np.uint16), slots.numpy())
    assert np.array_equal(ours, ref)


# --------------------------------------------------------------------- pack --
@pytest.mark.parametrize("H", GOLDEN["pack_test_matrix"]["num_heads"] + [64])
@pytest.mark.parametrize("T", [0, 1, 37])
def test_pack_bf16_matches_torch_concat(orc, T, H):
    g = torch.Generator().manual_seed(13 + H + T)
    kvb = torch.randn(T, H, 256, generator=g).to(torch.bfloat16)
    ws = torch.randn(T, 576, generator=g).to(torch.bfloat16)
    k_nope, k_pe = kvb[..., :128], ws[:, 512:]
    ref = torch.cat([k_nope, k_pe[:, None, :].expand(T, H, 64)], dim=-1)
    kn = u16(kvb)[..., :128]
    kp = u16(ws)[:, 512:]
    key, v = orc.pack(kn, kp)
    assert v is None and key.shape == (T, H, 192)
    assert np.array_equal(key, u16(ref))


@pytest.mark.parametrize("H", GOLDEN["pack_test_matrix"]["num_heads"] + [64])
@pytest.mark.parametrize("T", [0, 1, 37])
def test_pack_fp8_matches_torch_cast(orc, T, H):
    g = torch.Generator().manual_seed(17 + H + T)
    kvb = torch.randn(T, H, 256, generator=g).to(torch.bfloat16)
    ws = torch.randn(T, 576, generator=g).to(torch.bfloat16)
    k_nope, v, k_pe = kvb[..., :128], kvb[..., 128:], ws[:, 512:]
    key_ref = torch.cat([k_nope, k_pe[:, None, :].expand(T, H, 64)], dim=-1)
    key_ref = key_ref.float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    v_ref = v.float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    key, vo = orc.pack(u16(kvb)[..., :128], u16(ws)[:, 512:], u16(kvb)[..., 128:],
                       mode=orc.PACK_KEY_V_FP8)
    assert np.array_equal(key, key_ref)
    assert np.array_equal(vo, v_ref)
    if T:
        assert (key[:, :, 128:] == key[:, :1, 128:]).all()   # broadcast over heads


def test_pack_fp8_scales_divide(orc):
    g = torch.Generator().manual_seed(19)
    T, H = 5, 3
    kvb = torch.randn(T, H, 256, generator=g).to(torch.bfloat16)
    ws = torch.randn(T, 576, generator=g).to(torch.bfloat16)
    ks, vs = 0.7312, 1.37
    key, vo = orc.pack(u16(kvb)[..., :128], u16(ws)[:, 512:], u16(kvb)[..., 128:],
                       mode=orc.PACK_KEY_V_FP8, k_scale=ks, v_scale=vs)
    key_ref = torch.cat([kvb[..., :128], ws[:, None, 512:].expand(T, H, 64)], -1).float()
    key_ref = (key_ref / torch.tensor(ks)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    v_ref = (kvb[..., 128:].float() / torch.tensor(vs)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(key, key_ref) and np.array_equal(vo, v_ref)
