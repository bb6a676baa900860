"""GPU parity of the new-token epilogue against the CPU oracle.

Page: "PR #51772 完整报告", 功能与动机 and 关键源码片段 (the chunked-context pack
is fused_mla_key_concat_kv_cache_insert without the query, the cache insert
and RoPE; the op itself is named only, so both sides follow the same reading:
pack + RoPE of q_pe and k_pe + query row + insert of [kv_c | RoPE(k_pe)]).

Bars: the nope parts, V and the cache's kv_c part are casts or copies, so
bit-exact; the rotated parts follow the context epilogue's RoPE bar -- within
1 bf16 ulp of the float64 oracle (both sides round the rotation correctly
to bf16; they can differ only where the device's and the host's cos / sin
differ in their last bits and that moves a rounding);
their fp8 codes are identical wherever the GPU's bf16 rotation equals the
oracle's, else within one code.  Workloads: strided views of the model's tensors (query
[T, H, 192], kv_b_proj output [T, H, 256], latent row [T, 576]), 1 to 300
tokens and 1 to 32 heads with a padded token, both output modes and all
three cache formats (fp8 outputs with heads a multiple of 16 run the grouped
form), the full 8192-token x 64-head prefill (every token), capped grids of
both forms, a cache-only call, and special values (NaN, +-Inf, -0,
subnormals, values beyond the fp8 range; rotations that produce NaN are
compared as NaN, since the sign of a NaN made by arithmetic is not fixed).
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_paged_insert_amd import synth
from gpu_util import (DEV, announce, bf16_ulps, check_slots, fp8_codes_apart, requires_gpu,
                      run_sliced, u16, u8)

pytestmark = [pytest.mark.gpu, requires_gpu]

R, P, NOPE, VD = 512, 64, 128, 128
FMT = {"bf16": ("auto", None), "e4m3": ("fp8", "e4m3"), "e5m2": ("fp8_e5m2", "e5m2")}


def f32(bits):
    return oracle.bf16_to_f32(np.ascontiguousarray(bits)).astype(np.float64)


def assert_rope_close(got, ref, pe_bits, what):
    """Rotated values within 1 bf16 ulp of the oracle's (pe_bits: the inputs,
    named in the message of a failure)."""
    ul = bf16_ulps(got, ref)
    bad = ul > 1
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} rotated values more than 1 ulp off, "
                             f"first at {i}: gpu 0x{int(got[i]):04x} oracle 0x{int(ref[i]):04x}")
    announce(f"{what}: {np.mean(ul == 0):.6f} identical")


def assert_codes(got, ref, gpu_bf16, ref_bf16, what):
    """fp8 codes of rotated values: equal where the bf16 rotations agree, else
    within one code."""
    agree = gpu_bf16 == ref_bf16
    assert np.array_equal(got[agree], ref[agree]), what
    assert fp8_codes_apart(got, ref).max() <= 1, what


class Case:
    """Inputs on the host (torch CPU, strided views) and their device copies."""

    def __init__(self, seed, T, H, cache_fmt, num_blocks=None):
        nb = num_blocks or max(2, (T + 63) // 64 * 2)
        self.d = synth.new_tokens("cpu", seed, num_tokens=T, heads=H, num_blocks=nb,
                                  requests=min(8, max(1, T)), fp8_cache=cache_fmt != "bf16")
        self.T, self.H, self.fmt = T, H, cache_fmt
        self.dt, self.ofmt = FMT[cache_fmt]
        d = self.d
        check_slots(d["slots"], d["cache"].shape[0] * d["cache"].shape[1])
        self.g = {k: v.to(DEV) for k, v in d.items() if isinstance(v, torch.Tensor)}
        self.max_pos = d["max_pos"]
        self.cs = torch.empty(self.max_pos, 2 * P, dtype=torch.float32, device=DEV)
        import fp8_paged_insert_amd as mk
        mk.mla_rope_cos_sin_cache(self.cs, self.max_pos, P, 10000.0)

    def host_views(self):
        d = self.d
        q, kvb, kv = u16(d["q"]), u16(d["kvb"]), u16(d["kv"])
        return dict(q_nope=q[:, :, :NOPE], q_pe=q[:, :, NOPE:], k_nope=kvb[:, :, :NOPE],
                    v=kvb[:, :, NOPE:], kv_c=kv[:, :R], k_pe=kv[:, R:])

    def run_gpu(self, mk, fp8, cache=True, max_blocks=0, scales=True):
        g, T, H = self.g, self.T, self.H
        out_dt = torch.uint8 if fp8 else torch.bfloat16
        q_out = torch.empty(T, H, NOPE + P, dtype=out_dt, device=DEV)
        key = torch.empty(T, H, NOPE + P, dtype=out_dt, device=DEV)
        v_out = torch.empty(T, H, VD, dtype=torch.uint8, device=DEV) if fp8 else None
        c = g["cache"].clone() if cache else None
        q, kvb, kv = g["q"], g["kvb"], g["kv"]
        kw = {}
        if fp8:
            kw = dict(v=kvb[:, :, NOPE:], v_out=v_out, mode=mk.MLA_PACK_KEY_V_FP8)
            if scales:
                kw.update(q_scale=g["q_scale"], k_scale=g["k_scale"], v_scale=g["v_scale"])
        if cache:
            kw.update(cache=c, slot_mapping=g["slots"], kv_cache_dtype=self.dt,
                      cache_scale=g["cache_scale"] if self.fmt != "bf16" else None)
        mk.mla_new_token_epilogue(q[:, :, :NOPE], q[:, :, NOPE:], kvb[:, :, :NOPE], kv[:, :R],
                                  kv[:, R:], g["positions"], self.cs, q_out, key,
                                  max_blocks=max_blocks, **kw)
        torch.cuda.synchronize()
        return q_out, key, v_out, c

    def run_oracle(self, fp8, rows=None, scales=True):
        """The oracle over all tokens, or over the token subset `rows` (its
        cache is then a fresh copy of the initial one)."""
        d = self.d
        h = self.host_views()
        pos = d["positions"].numpy()
        slots = d["slots"].numpy()
        if rows is not None:
            h = {k: np.ascontiguousarray(v[rows]) for k, v in h.items()}
            pos, slots = pos[rows], slots[rows]
        cache = (u8(d["cache"]) if self.fmt != "bf16" else u16(d["cache"])).copy()
        sc = lambda k: float(d[k][0]) if (fp8 and scales) else 1.0

        def part(a, b):
            # token slices on host threads; their slots are distinct, so the
            # slices write disjoint cache entries
            return oracle.new_token_epilogue(
                h["q_nope"][a:b], h["q_pe"][a:b], h["k_nope"][a:b], h["kv_c"][a:b],
                h["k_pe"][a:b], pos[a:b], v=h["v"][a:b],
                mode=oracle.PACK_KEY_V_FP8 if fp8 else oracle.PACK_KEY_BF16,
                q_scale=sc("q_scale"), k_scale=sc("k_scale"), v_scale=sc("v_scale"),
                cache=cache, slots=slots[a:b],
                cache_scale=float(d["cache_scale"][0]) if self.fmt != "bf16" else 1.0,
                fp8_format=self.ofmt or "e4m3")
        parts = run_sliced(part, len(pos))
        q = np.concatenate([p[0] for p in parts])
        key = np.concatenate([p[1] for p in parts])
        v = np.concatenate([p[2] for p in parts]) if fp8 else None
        return q, key, v, cache, h, slots


def check_case(mk, case, fp8, rows=None, scales=True, max_blocks=0):
    T, H = case.T, case.H
    qg, kg, vg, cg = case.run_gpu(mk, fp8, max_blocks=max_blocks, scales=scales)
    # the bf16 run gives the GPU's own rotations, against which fp8 codes are judged
    qb, kb, _, _ = case.run_gpu(mk, False, cache=False) if fp8 else (qg, kg, None, None)
    q, key, v, cache, h, slots = case.run_oracle(fp8, rows, scales)
    sel = slice(None) if rows is None else rows
    conv = u8 if fp8 else u16
    qg_, kg_ = conv(qg)[sel], conv(kg)[sel]
    qb_, kb_ = u16(qb)[sel], u16(kb)[sel]
    # nope parts and V: casts / copies, bit-exact
    assert np.array_equal(qg_[..., :NOPE], q[..., :NOPE]), "query nope part"
    assert np.array_equal(kg_[..., :NOPE], key[..., :NOPE]), "key nope part"
    if fp8:
        assert np.array_equal(u8(vg)[sel], v), "V"
    # rotated parts, against the bf16 oracle
    qref, kref, _ = (case.run_oracle(False, rows)[:3]) if fp8 else (q, key, None)
    assert_rope_close(qb_[..., NOPE:], qref[..., NOPE:], h["q_pe"], "query rope")
    kpe_b = np.broadcast_to(h["k_pe"][:, None, :], kref[..., NOPE:].shape)
    assert_rope_close(kb_[..., NOPE:], kref[..., NOPE:], kpe_b, "key rope")
    if fp8:
        assert_codes(qg_[..., NOPE:], q[..., NOPE:], qb_[..., NOPE:], qref[..., NOPE:], "query codes")
        assert_codes(kg_[..., NOPE:], key[..., NOPE:], kb_[..., NOPE:], kref[..., NOPE:], "key codes")
    # cache: untouched entries unchanged, touched ones per part
    conv_c = u16 if case.fmt == "bf16" else u8
    init = conv_c(case.d["cache"]).reshape(-1, R + P)
    got = conv_c(cg).reshape(-1, R + P)
    ref = cache.reshape(-1, R + P)
    all_slots = case.d["slots"].numpy()
    touched = np.zeros(got.shape[0], bool)
    touched[all_slots[all_slots >= 0]] = True
    assert np.array_equal(got[~touched], init[~touched]), "stray cache writes"
    ok = slots >= 0
    gs, rs = got[slots[ok]], ref[slots[ok]]
    assert np.array_equal(gs[:, :R], rs[:, :R]), "cache kv_c part"
    kgpu = kb_[ok][:, 0, NOPE:]        # the GPU's rotated k_pe (bf16 run, head 0)
    if case.fmt == "bf16":
        assert_rope_close(gs[:, R:], rs[:, R:], h["k_pe"][ok], "cache rope part")
        assert np.array_equal(gs[:, R:], kgpu), "cache rope part differs from the key's"
    else:
        assert_codes(gs[:, R:], rs[:, R:], kgpu, kref[ok][:, 0, NOPE:], "cache rope codes")


CASES = [  # (seed, T, H, cache format, fp8 outputs)
    (31, 1, 1, "bf16", False),
    (32, 37, 3, "bf16", False),
    (33, 37, 3, "e4m3", False),
    (34, 37, 4, "e5m2", False),
    (35, 37, 3, "bf16", True),
    (36, 130, 4, "e4m3", True),
    (37, 130, 4, "e5m2", True),
    (38, 300, 16, "e4m3", True),
    (39, 300, 16, "bf16", False),
    # fp8 outputs with heads a multiple of 16 take the grouped form (16 heads
    # per wavefront); 77 tokens leave the last cache wavefront 1 row of 4
    (42, 77, 32, "e5m2", True),
    (43, 45, 16, "bf16", True),
]


@pytest.mark.parametrize("seed,T,H,fmt,fp8", CASES)
def test_matches_oracle(mk, seed, T, H, fmt, fp8):
    announce("new-token epilogue", seed, T, H, fmt, fp8)
    check_case(mk, Case(seed, T, H, fmt), fp8)


def test_no_scales_is_a_plain_cast(mk):
    announce("new-token epilogue without q/k/v scales")
    check_case(mk, Case(40, 64, 4, "e4m3"), True, scales=False)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("fp8", [False, True])
def test_full_prefill(mk, fp8):
    """8192 new tokens x 64 heads into a [512, 64, 576] cache, e4m3fn cache
    and (fp8) e4m3fn query / key / V: every token against the oracle (token
    slices on host threads), and the whole cache outside the written slots
    untouched."""
    announce("new-token epilogue full size", fp8)
    check_case(mk, Case(8, 8192, 64, "e4m3", num_blocks=512), fp8)


@pytest.mark.parametrize("H", [8, 16])
def test_capped_grid_and_cache_only(mk, H):
    """A capped grid gives the same bytes as the default one (8 heads: one
    task per 16-lane row; 16 heads: the grouped form), and num_heads = 0
    runs only the cache insert."""
    announce("new-token epilogue capped grid / cache only", H)
    case = Case(41, 201, H, "e4m3")
    a = case.run_gpu(mk, True)
    b = case.run_gpu(mk, True, max_blocks=7)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    # num_heads = 0: only the cache insert runs
    g = case.g
    c = g["cache"].clone()
    empty = torch.empty(case.T, 0, NOPE + P, dtype=torch.uint8, device=DEV)
    kvb0 = g["kvb"][:, :0]
    q0 = g["q"][:, :0]
    mk.mla_new_token_epilogue(q0[:, :, :NOPE], q0[:, :, NOPE:], kvb0[:, :, :NOPE],
                              g["kv"][:, :R], g["kv"][:, R:], g["positions"], case.cs, empty,
                              empty.clone(), v=kvb0[:, :, NOPE:],
                              v_out=torch.empty(case.T, 0, VD, dtype=torch.uint8, device=DEV),
                              mode=mk.MLA_PACK_KEY_V_FP8, cache=c, slot_mapping=g["slots"],
                              kv_cache_dtype="fp8", cache_scale=g["cache_scale"])
    torch.cuda.synchronize()
    assert torch.equal(c, a[3])


@pytest.mark.parametrize("nope,vdim", [(64, 96), (256, 128)])
@pytest.mark.parametrize("fp8", [False, True])
def test_other_head_widths(mk, nope, vdim, fp8):
    """nope / V widths other than 128 (the MLA shape has its own straight-line
    path): 64 / 96 leaves lanes of each 16-lane row idle, 256 gives each lane
    two nope chunks.  The nope parts and V are casts (bit-exact against the
    oracle); the rotated parts are judged as in the other cases."""
    announce("new-token epilogue widths", nope, vdim, fp8)
    g = synth.gen(60 + nope + vdim)
    T, H = 37, 3
    qn, qp = synth.bf16_normal((T, H, nope), g), synth.bf16_normal((T, H, P), g)
    kn, v = synth.bf16_normal((T, H, nope), g), synth.bf16_normal((T, H, vdim), g)
    kv = synth.bf16_normal((T, R + P), g)
    pos = torch.randint(0, 4096, (T,), generator=g)
    cs = torch.empty(4096, 2 * P, dtype=torch.float32, device=DEV)
    mk.mla_rope_cos_sin_cache(cs, 4096, P, 10000.0)
    kvd = kv.to(DEV)

    def run(fp8_out):
        odt = torch.uint8 if fp8_out else torch.bfloat16
        qo = torch.empty(T, H, nope + P, dtype=odt, device=DEV)
        ko = torch.empty(T, H, nope + P, dtype=odt, device=DEV)
        vo = torch.empty(T, H, vdim, dtype=torch.uint8, device=DEV) if fp8_out else None
        kw = dict(v=v.to(DEV), v_out=vo, mode=mk.MLA_PACK_KEY_V_FP8) if fp8_out else {}
        mk.mla_new_token_epilogue(qn.to(DEV), qp.to(DEV), kn.to(DEV), kvd[:, :R], kvd[:, R:],
                                  pos.to(DEV), cs, qo, ko, **kw)
        torch.cuda.synchronize()
        return qo, ko, vo

    h = [u16(x) for x in (qn, qp, kn, kv[:, :R], kv[:, R:], v)]
    qb, kb, _ = run(False)
    qref, kref, _ = oracle.new_token_epilogue(h[0], h[1], h[2], h[3], h[4], pos.numpy())
    assert_rope_close(u16(qb)[..., nope:], qref[..., nope:], h[1], "query rope")
    kpe_b = np.broadcast_to(h[4][:, None, :], kref[..., nope:].shape)
    assert_rope_close(u16(kb)[..., nope:], kref[..., nope:], kpe_b, "key rope")
    if not fp8:
        assert np.array_equal(u16(qb)[..., :nope], qref[..., :nope]), "query nope part"
        assert np.array_equal(u16(kb)[..., :nope], kref[..., :nope]), "key nope part"
        return
    qg, kg, vg = run(True)
    q8, k8, v8 = oracle.new_token_epilogue(h[0], h[1], h[2], h[3], h[4], pos.numpy(), v=h[5],
                                           mode=oracle.PACK_KEY_V_FP8)
    assert np.array_equal(u8(qg)[..., :nope], q8[..., :nope]), "query nope codes"
    assert np.array_equal(u8(kg)[..., :nope], k8[..., :nope]), "key nope codes"
    assert np.array_equal(u8(vg), v8), "V codes"
    assert_codes(u8(qg)[..., nope:], q8[..., nope:], u16(qb)[..., nope:], qref[..., nope:],
                 "query rope codes")
    assert_codes(u8(kg)[..., nope:], k8[..., nope:], u16(kb)[..., nope:], kref[..., nope:],
                 "key rope codes")


def is_bf16_nan(b):
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)


def check_rope_special(got, ref, what):
    """Rotations with special inputs: NaN exactly where the oracle's is NaN
    (the sign of a NaN made by arithmetic is not fixed), every other value
    within 1 bf16 ulp."""
    rn = is_bf16_nan(ref)
    assert np.array_equal(rn, is_bf16_nan(got)), f"{what}: NaN positions differ"
    ul = bf16_ulps(np.where(rn, 0, got), np.where(rn, 0, ref))
    assert ul.max() <= 1, f"{what}: up to {ul.max()} ulp"
    return rn


def check_codes_special(got, ref, gpu_bf16, ref_bf16, rn, what):
    assert np.all((got[rn] & 0x7F) == 0x7F) and np.all((ref[rn] & 0x7F) == 0x7F), what
    agree = (gpu_bf16 == ref_bf16) & ~rn
    assert np.array_equal(got[agree], ref[agree]), what
    assert fp8_codes_apart(np.where(rn, 0, got), np.where(rn, 0, ref)).max() <= 1, what


@pytest.mark.parametrize("fp8", [False, True])
def test_special_values(mk, fp8):
    """NaN (both signs), +-Inf, -0, a bf16 subnormal and +-1.7e38 planted in
    q_nope, k_nope, V and kv_c (casts and copies: bit-exact, saturating at
    the fp8 bound), and NaN / +-Inf in q_pe and k_pe, at position 0 (sin = 0,
    so the partner of an infinite value becomes NaN) and elsewhere; 16 heads,
    so the fp8 outputs take the grouped form."""
    announce("new-token epilogue special values", fp8)
    case = Case(70, 40, 16, "e4m3")
    d = case.d
    pats = torch.tensor([0x7FC0, 0xFFC0, 0x7F80, 0xFF80, 0x8000, 0x0005, 0x7F00, 0xFF00],
                        dtype=torch.int32).to(torch.int16)
    q, kvb, kv = (d[k].view(torch.int16) for k in ("q", "kvb", "kv"))
    q[0, 0, 0:8] = pats
    q[3, 15, 120:128] = pats
    kvb[1, 1, 0:8] = pats              # k_nope
    kvb[2, 7, 128:136] = pats          # V
    kv[2, 0:8] = pats                  # kv_c
    nan, inf, ninf = 0x7FC0, 0x7F80, 0xFF80 - 0x10000  # bit patterns as int16 values
    q[0, 2, NOPE + 3] = nan
    q[0, 2, NOPE + 40] = inf
    q[6, 3, NOPE + 10] = ninf
    kv[0, R + 40] = inf                 # position 0: its partner k_pe[8] -> NaN
    kv[7, R + 2] = nan
    kv[9, R + 50] = ninf
    d["positions"][0] = 0
    case.g = {k: v.to(DEV) for k, v in d.items() if isinstance(v, torch.Tensor)}

    qg, kg, vg, cg = case.run_gpu(mk, fp8)
    qb, kb, _, _ = case.run_gpu(mk, False, cache=False)
    q_o, key_o, v_o, cache_o, h, slots = case.run_oracle(fp8)
    qref, kref, _ = case.run_oracle(False)[:3]
    conv = u8 if fp8 else u16
    assert np.array_equal(conv(qg)[..., :NOPE], q_o[..., :NOPE]), "query nope part"
    assert np.array_equal(conv(kg)[..., :NOPE], key_o[..., :NOPE]), "key nope part"
    if fp8:
        assert np.array_equal(u8(vg), v_o), "V"
    qrn = check_rope_special(u16(qb)[..., NOPE:], qref[..., NOPE:], "query rope")
    krn = check_rope_special(u16(kb)[..., NOPE:], kref[..., NOPE:], "key rope")
    assert qrn[0, 2].sum() >= 2 and krn[0, :, 8].all() and krn[7].any()
    if fp8:
        check_codes_special(u8(qg)[..., NOPE:], q_o[..., NOPE:], u16(qb)[..., NOPE:],
                            qref[..., NOPE:], qrn, "query rope codes")
        check_codes_special(u8(kg)[..., NOPE:], key_o[..., NOPE:], u16(kb)[..., NOPE:],
                            kref[..., NOPE:], krn, "key rope codes")
    got = u8(cg).reshape(-1, R + P)
    ref = cache_o.reshape(-1, R + P)
    ok = slots >= 0
    gs, rs = got[slots[ok]], ref[slots[ok]]
    assert np.array_equal(gs[:, :R], rs[:, :R]), "cache kv_c part"
    check_codes_special(gs[:, R:], rs[:, R:], u16(kb)[ok][:, 0, NOPE:], kref[ok][:, 0, NOPE:],
                        krn[ok][:, 0], "cache rope codes")
    announce(f"special values: {int(qrn.sum())} query and {int(krn.sum())} key NaN rotations")
