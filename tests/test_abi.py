"""CPU checks of the C ABI: the library loads, exports every symbol the header
declares, parses cache dtypes, and rejects bad arguments on the host before
anything is enqueued (no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_kv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_exports(mk):
    assert declared_functions() == sorted(mk.EXPORTS)


def test_library_exports_every_declared_symbol(mk):
    h = ctypes.CDLL(mk.LIB_PATH)
    for name in declared_functions():
        assert hasattr(h, name), name


def test_version(mk):
    assert "gfx950" in mk.version()



def test_missing_library_fails_loudly(monkeypatch):
    """Without the built HIP library every call raises: there is no CPU or
    fallback path behind the binding."""
    import fp8_paged_insert_amd._binding as B
    monkeypatch.setattr(B, "LIB_PATH", os.path.join(ROOT, "_no_such_dir", "libmla_kv.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        B.version()
    with pytest.raises(RuntimeError, match="not built"):
        B.lib()


def test_product_package_does_not_use_the_oracle():
    """The package (binding, build script, input generators) never imports
    or loads anything under oracle/."""
    pkg = os.path.join(ROOT, "fp8_paged_insert_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "mla_oracle" not in text and "liborc" not in text, f


@pytest.mark.parametrize("s,code", [("auto", 0), ("bfloat16", 1), ("fp8", 2), ("fp8_e4m3", 2),
                                    ("fp8_e5m2", 3)])
def test_parse_dtype_accepts_whitelist(mk, s, code):
    assert mk.parse_kv_cache_dtype(s) == code


def test_parse_dtype_rejects(mk):
    with pytest.raises(mk.MlaError) as e:
        mk.parse_kv_cache_dtype("int8")
    assert e.value.status == mk.MLA_ERR_INVALID_ARGUMENT


# Raw C calls with host-side argument errors.  Dummy non-NULL addresses are
# never dereferenced: validation fails first.
P16 = 0x10000  # 16-byte aligned dummy address
P_ODD = 0x10008


def insert_call(mk, **kw):
    a = dict(kv_c=P16, kv_ls=512, kv_ts=2560, k_pe=P16, pe_ls=64, pe_ts=320, ptrs=P16,
             scales=P16, slots=P16, sls=0, L=5, T=4, R=512, P=64, bs=64, bstride=64 * 576,
             estride=576, dt=mk.MLA_KV_FP8_E4M3)
    a.update(kw)
    return mk.lib().mla_kv_insert_grouped(
        a["kv_c"], a["kv_ls"], a["kv_ts"], a["k_pe"], a["pe_ls"], a["pe_ts"], a["ptrs"],
        a["scales"], a["slots"], a["sls"], a["L"], a["T"], a["R"], a["P"], a["bs"],
        a["bstride"], a["estride"], a["dt"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(dt=3, scales=None), 1, "needs kv_scales"),
    (dict(dt=9), 1, "unknown KV cache dtype"),
    (dict(scales=None), 1, "needs kv_scales"),
    (dict(dt=0), 1, "takes no kv_scales"),
    (dict(dt=1), 1, "takes no kv_scales"),
    (dict(T=-1), 1, "negative"),
    (dict(bs=0), 1, "positive"),
    (dict(estride=500), 1, "smaller than the entry width"),
    (dict(bstride=100), 1, "overlap"),
    (dict(ptrs=None), 1, "must not be NULL"),
    (dict(slots=None), 1, "must not be NULL"),
    (dict(kv_c=None), 1, "must not be NULL"),
    (dict(kv_c=P_ODD), 3, "multiples of 16 bytes"),
    (dict(kv_ts=2564), 3, "multiples of 16 bytes"),
    (dict(estride=584, bstride=64 * 584), 3, "multiples of 16 bytes"),
    (dict(R=520, estride=592, bstride=64 * 592), 2, "multiples of 16"),
])
def test_insert_rejects_bad_arguments(mk, kw, status, msg):
    assert insert_call(mk, **kw) == status
    assert msg in mk.last_error()


def test_insert_zero_tokens_or_layers_is_a_noop(mk):
    assert insert_call(mk, T=0) == mk.MLA_OK
    assert insert_call(mk, L=0) == mk.MLA_OK
    assert insert_call(mk, T=0, kv_c=None, k_pe=None, ptrs=None, slots=None) == mk.MLA_OK


def epilogue_call(mk, **kw):
    a = dict(all_kv=P16, kls=576, kts=2880, gamma=P16, eps=1e-6, pos=P16, cs=P16, max_pos=4096,
             ptrs=P16, scales=P16, slots=P16, sls=4096, L=5, T=4096, R=512, P=64, bs=64,
             bstride=64 * 576, estride=576, dt=mk.MLA_KV_FP8_E4M3, dbg=None)
    a.update(kw)
    return mk.lib().mla_ctx_kv_epilogue(
        a["all_kv"], a["kls"], a["kts"], a["gamma"], a["eps"], a["pos"], a["cs"], a["max_pos"],
        a["ptrs"], a["scales"], a["slots"], a["sls"], a["L"], a["T"], a["R"], a["P"], a["bs"],
        a["bstride"], a["estride"], a["dt"], a["dbg"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(dt=3, scales=None), 1, "needs kv_scales"),
    (dict(scales=None), 1, "needs kv_scales"),
    (dict(R=256, estride=320, bstride=64 * 320), 2, "kv_lora_rank 512"),
    (dict(gamma=None), 1, "NULL"),
    (dict(max_pos=0), 1, "max_pos"),
    (dict(eps=-1.0), 1, "eps"),
    (dict(kts=2881), 3, "multiples of 16 bytes"),
    (dict(dbg=P_ODD), 3, "multiples of 16 bytes"),
])
def test_epilogue_rejects_bad_arguments(mk, kw, status, msg):
    assert epilogue_call(mk, **kw) == status
    assert msg in mk.last_error()


def pack_call(mk, **kw):
    a = dict(kn=P16, kn_ts=16384, kn_hs=256, kpe=P16, kpe_ts=576, v=P16, v_ts=16384,
             v_hs=256, T=8192, H=64, nope=128, rope=64, vdim=128, mode=mk.MLA_PACK_KEY_V_FP8,
             src=mk.MLA_KV_BF16, ks=None, vs=None, key=P16, vo=P16, maxb=0)
    a.update(kw)
    return mk.lib().mla_ctx_kv_pack(
        a["kn"], a["kn_ts"], a["kn_hs"], a["kpe"], a["kpe_ts"], a["v"], a["v_ts"], a["v_hs"],
        a["T"], a["H"], a["nope"], a["rope"], a["vdim"], a["mode"], a["src"], a["ks"], a["vs"],
        a["key"], a["vo"], a["maxb"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(mode=7), 1, "unknown mode"),
    (dict(mode=0), 1, "takes no v"),
    (dict(T=-1), 1, "negative"),
    (dict(maxb=-1), 1, "negative"),
    (dict(key=None), 1, "NULL"),
    (dict(nope=120), 2, "multiples of 16"),
    (dict(kn_hs=257), 3, "multiples of 16 bytes"),
    (dict(vo=P_ODD), 3, "multiples of 16 bytes"),
    (dict(src=2), 1, "src_dtype"),
    (dict(src=0), 1, "src_dtype"),
    (dict(mode=2, kpe_ts=577), 3, "multiples of 16 bytes"),
    (dict(mode=1, kpe_ts=580), 3, "multiples of 16 bytes"),
])
def test_pack_rejects_bad_arguments(mk, kw, status, msg):
    assert pack_call(mk, **kw) == status
    assert msg in mk.last_error()


def test_pack_zero_tokens_is_a_noop(mk):
    assert pack_call(mk, T=0) == mk.MLA_OK
    assert pack_call(mk, H=0) == mk.MLA_OK
    assert pack_call(mk, T=0, mode=mk.MLA_PACK_KEY_V_FP8_KPE_RAW, src=mk.MLA_KV_FP16) == mk.MLA_OK



def gather_call(mk, **kw):
    a = dict(cache=P16, dt=mk.MLA_KV_FP8_E4M3, scale=P16, bs=64, bstride=64 * 576,
             estride=576, slots=P16, T=8192, width=576, odt=mk.MLA_KV_BF16, out=P16, maxb=0)
    a.update(kw)
    return mk.lib().mla_ctx_latent_gather(
        a["cache"], a["dt"], a["scale"], a["bs"], a["bstride"], a["estride"], a["slots"],
        a["T"], a["width"], a["odt"], a["out"], a["maxb"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(scale=None), 1, "needs cache_scale"),
    (dict(dt=1), 1, "takes no cache_scale"),
    (dict(dt=3, scale=None), 1, "needs cache_scale"),
    (dict(dt=3, odt=2, scale=None), 1, "must equal cache_dtype"),
    (dict(dt=2, odt=3, scale=None), 1, "must equal cache_dtype"),
    (dict(width=600), 1, "exceeds entry_stride"),
    (dict(width=40), 2, "multiple of 16"),
    (dict(out=None), 1, "NULL"),
    (dict(out=P_ODD), 3, "multiples of 16 bytes"),
    (dict(odt=0), 1, "out_dtype"),
    (dict(odt=2), 1, "does not dequantise"),
    (dict(odt=2, scale=None, dt=1), 1, "needs an fp8 cache"),
])
def test_gather_rejects_bad_arguments(mk, kw, status, msg):
    assert gather_call(mk, **kw) == status
    assert msg in mk.last_error()


P_GATHER_OUT = 1 << 44   # a fake, 16-byte aligned address far from P16's ranges


def pack_gather_call(mk, pack=None, gather=None):
    a = dict(kn=P16, kn_ts=16384, kn_hs=256, kpe=P16 + 1024, kpe_ts=576, v=P16 + 256,
             v_ts=16384, v_hs=256, T=8192, H=64, nope=128, rope=64, vdim=128,
             mode=mk.MLA_PACK_KEY_V_FP8, src=mk.MLA_KV_BF16, ks=None, vs=None,
             key=P16 + (1 << 32), vo=P16 + (1 << 33))
    a.update(pack or {})
    g = dict(cache=P16, dt=mk.MLA_KV_FP8_E4M3, scale=P16, bs=64, bstride=64 * 576,
             estride=576, slots=P16, T=8192, width=576, odt=mk.MLA_KV_BF16, out=P_GATHER_OUT)
    g.update(gather or {})
    return mk.lib().mla_ctx_kv_pack_gather(
        a["kn"], a["kn_ts"], a["kn_hs"], a["kpe"], a["kpe_ts"], a["v"], a["v_ts"], a["v_hs"],
        a["T"], a["H"], a["nope"], a["rope"], a["vdim"], a["mode"], a["src"], a["ks"], a["vs"],
        a["key"], a["vo"], g["cache"], g["dt"], g["scale"], g["bs"], g["bstride"], g["estride"],
        g["slots"], g["T"], g["width"], g["odt"], g["out"], a.get("maxb", 0), None)


@pytest.mark.parametrize("pack,gather,status,msg", [
    (dict(mode=7), None, 1, "unknown mode"),
    (dict(nope=120), None, 2, "multiples of 16"),
    (None, dict(scale=None), 1, "needs cache_scale"),
    (None, dict(width=40), 2, "multiple of 16"),
    (None, dict(out=P16 + (1 << 32) + 4096), 1, "overlaps"),    # inside key_out
    (None, dict(out=P16 + 512), 1, "overlaps"),                  # inside the kv_b_proj rows
    (dict(mode=2, kpe_ts=576), None, 2, "joint launch"),         # verbatim fp8 k_pe
    (dict(src=4), None, 2, "joint launch"),                       # fp16 sources
    (dict(maxb=-1), None, 1, "negative"),
])
def test_pack_gather_rejects_bad_arguments(mk, pack, gather, status, msg):
    assert pack_gather_call(mk, pack, gather) == status
    assert msg in mk.last_error()


def test_pack_gather_both_parts_empty_is_a_noop(mk):
    assert pack_gather_call(mk, dict(T=0), dict(T=0)) == mk.MLA_OK


def test_stream_copy_rejects(mk):
    lib = mk.lib()
    assert lib.mla_stream_copy(P16, P16 + (1 << 20), -16, None) == mk.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_stream_copy(P16, P16 + (1 << 20), 0, None) == mk.MLA_OK
    assert lib.mla_stream_copy(P_ODD, P16 + (1 << 20), 64, None) == mk.MLA_ERR_MISALIGNED
    assert lib.mla_stream_copy(P16, P16 + (1 << 20), 40, None) == mk.MLA_ERR_MISALIGNED
    assert lib.mla_stream_copy(P16, P16 + 32, 64, None) == mk.MLA_ERR_INVALID_ARGUMENT
    assert "overlap" in mk.last_error()


def test_stream_mix_rejects(mk):
    lib = mk.lib()
    far = P16 + (1 << 32)
    assert lib.mla_stream_mix(P16, far, 64, 0, None) == mk.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_stream_mix(P16, far, 64, 5, None) == mk.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_stream_mix(P16, far, 0, 2, None) == mk.MLA_OK
    assert lib.mla_stream_mix(P_ODD, far, 64, 2, None) == mk.MLA_ERR_MISALIGNED
    assert lib.mla_stream_mix(P16, far, 40, 2, None) == mk.MLA_ERR_MISALIGNED
    # src spans 2 x 64 bytes from P16 - 96: it reaches into dst
    assert lib.mla_stream_mix(P16, P16 - 96, 64, 2, None) == mk.MLA_ERR_INVALID_ARGUMENT
    assert "overlap" in mk.last_error()


def test_mfma_rate_rejects(mk):
    lib = mk.lib()
    assert lib.mla_mfma_rate(0, P16, 1 << 20, None) == mk.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_mfma_rate((1 << 20) + 1, P16, 1 << 20, None) == mk.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_mfma_rate(15, P16, 1 << 20, None) == mk.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_mfma_rate(16, None, 1 << 20, None) == mk.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_mfma_rate(16, P16, 15, None) == mk.MLA_ERR_INVALID_ARGUMENT
    assert "needed" in mk.last_error()


def test_transpose_rejects(mk):
    lib = mk.lib()
    far = P16 + (1 << 32)
    assert lib.mla_transpose_bf16(P16, -8, 8, 8, far, 8, None) == mk.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_transpose_bf16(P16, 0, 8, 8, far, 8, None) == mk.MLA_OK
    assert lib.mla_transpose_bf16(P16, 12, 8, 8, far, 12, None) == mk.MLA_ERR_UNSUPPORTED
    assert lib.mla_transpose_bf16(P16, 16, 16, 8, far, 16, None) == mk.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_transpose_bf16(P_ODD, 16, 16, 16, far, 16, None) == mk.MLA_ERR_MISALIGNED
    assert lib.mla_transpose_bf16(P16, 16, 16, 16, P16 + 64, 16, None) == mk.MLA_ERR_INVALID_ARGUMENT
    assert "overlap" in mk.last_error()


def test_rope_table_rejects(mk):
    assert mk.lib().mla_rope_cos_sin_cache(P16, 10, 63, 10000.0, None) == mk.MLA_ERR_INVALID_ARGUMENT
    assert mk.lib().mla_rope_cos_sin_cache(P16, 10, 64, -1.0, None) == mk.MLA_ERR_INVALID_ARGUMENT
    assert mk.lib().mla_rope_cos_sin_cache(None, 0, 64, 10000.0, None) == mk.MLA_OK


def merge_call(mk, **kw):
    a = dict(out=P16, ots=8192, ohs=128, lse=P16, lhs=16384, lts=1, part=P16 + 0x100000,
             pts=8192, phs=128, plse=P16, plhs=16384, plts=1, T=16384, H=64, D=128,
             mode=mk.MLA_MERGE_ACCUMULATE)
    a.update(kw)
    return mk.lib().mla_ctx_merge_chunk(
        a["out"], a["ots"], a["ohs"], a["lse"], a["lhs"], a["lts"], a["part"], a["pts"], a["phs"],
        a["plse"], a["plhs"], a["plts"], a["T"], a["H"], a["D"], a["mode"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(mode=5), 1, "unknown mode"),
    (dict(T=-1), 1, "negative"),
    (dict(lse=None), 1, "NULL"),
    (dict(plse=None), 1, "NULL part_lse"),
    (dict(part=None), 1, "NULL part"),
    (dict(D=100), 2, "multiple of 8"),
    (dict(ohs=127), 3, "16-byte aligned"),
    (dict(part=P_ODD), 3, "16-byte aligned"),
    (dict(part=P16), 1, "continuation chunk"),
    (dict(plse=P16 + 2), 3, "4-byte aligned"),
])
def test_merge_rejects_bad_arguments(mk, kw, status, msg):
    assert merge_call(mk, **kw) == status
    assert msg in mk.last_error()


def test_merge_and_neutralize_zero_sizes_are_noops(mk):
    assert merge_call(mk, T=0) == mk.MLA_OK
    assert merge_call(mk, H=0, part=None) == mk.MLA_OK
    assert mk.lib().mla_ctx_neutralize_partials(P16, 8192, 128, P16, 16384, 1, None, 0, 64, 128,
                                                None) == mk.MLA_OK
    assert mk.lib().mla_ctx_neutralize_partials(P16, 8192, 128, P16, 16384, 1, None, 5, 64, 128,
                                                None) == mk.MLA_ERR_INVALID_ARGUMENT


def new_token_call(mk, **kw):
    a = dict(qn=P16, qn_ts=64 * 192, qn_hs=192, qp=P16, qp_ts=64 * 192, qp_hs=192, kn=P16,
             kn_ts=16384, kn_hs=256, v=P16, v_ts=16384, v_hs=256, kvc=P16, kvc_ts=576, kpe=P16,
             kpe_ts=576, pos=P16, cs=P16, maxpos=16384, T=8192, H=64, nope=128, rope=64,
             vdim=128, R=512, mode=mk.MLA_PACK_KEY_V_FP8, qs=None, ks=None, vs=None, qo=P16,
             ko=P16, vo=P16, cache=P16, dt=mk.MLA_KV_FP8_E4M3, cscale=P16, slots=P16, bs=64,
             bstride=64 * 576, estride=576, maxb=0)
    a.update(kw)
    return mk.lib().mla_new_token_epilogue(
        a["qn"], a["qn_ts"], a["qn_hs"], a["qp"], a["qp_ts"], a["qp_hs"], a["kn"], a["kn_ts"],
        a["kn_hs"], a["v"], a["v_ts"], a["v_hs"], a["kvc"], a["kvc_ts"], a["kpe"], a["kpe_ts"],
        a["pos"], a["cs"], a["maxpos"], a["T"], a["H"], a["nope"], a["rope"], a["vdim"], a["R"],
        a["mode"], a["qs"], a["ks"], a["vs"], a["qo"], a["ko"], a["vo"], a["cache"], a["dt"],
        a["cscale"], a["slots"], a["bs"], a["bstride"], a["estride"], a["maxb"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(mode=2), 1, "KEY_BF16 or KEY_V_FP8"),
    (dict(mode=0), 1, "takes no v"),
    (dict(T=-1), 1, "negative"),
    (dict(maxb=-1), 1, "negative"),
    (dict(cscale=None), 1, "needs kv_scales"),
    (dict(dt=1), 1, "takes no kv_scales"),
    (dict(dt=9), 1, "unknown KV cache dtype"),
    (dict(slots=None), 1, "needs slot_mapping"),
    (dict(bs=0), 1, "positive"),
    (dict(estride=560), 1, "wider than entry_stride"),
    (dict(cache=None), 1, "without a cache"),
    (dict(rope=48), 2, "rope must be 64"),
    (dict(rope=32), 2, "rope must be 64"),
    (dict(nope=120), 2, "multiples of 16"),
    (dict(pos=None), 1, "positions"),
    (dict(maxpos=0), 1, "max_pos"),
    (dict(qo=None), 1, "NULL input or output"),
    (dict(vo=None), 1, "NULL input or output"),
    (dict(kvc=None), 1, "NULL kv_c"),
    (dict(qp_hs=193), 3, "multiples of 16 bytes"),
    (dict(kpe=P_ODD), 3, "multiples of 16 bytes"),
    (dict(dt=1, cscale=None, estride=580), 3, "multiples of 16 bytes"),
])
def test_new_token_rejects_bad_arguments(mk, kw, status, msg):
    assert new_token_call(mk, **kw) == status
    assert msg in mk.last_error()


def test_new_token_zero_tokens_is_a_noop(mk):
    assert new_token_call(mk, T=0) == mk.MLA_OK
    assert new_token_call(mk, T=0, mode=mk.MLA_PACK_KEY_BF16, v=None, vo=None) == mk.MLA_OK
    assert new_token_call(mk, T=0, cache=None, cscale=None, slots=None) == mk.MLA_OK


def test_sizes_beyond_one_launch_are_refused_before_launching(mk):
    """Every entry point indexes with 32-bit work-item counters; sizes past
    that are rejected on the host with UNSUPPORTED (nothing is launched)."""
    big = 1 << 31
    assert insert_call(mk, T=big) == mk.MLA_ERR_UNSUPPORTED
    assert "exceed one launch" in mk.last_error()
    assert pack_call(mk, T=1 << 27) == mk.MLA_ERR_UNSUPPORTED
    assert "split the chunk" in mk.last_error()
    assert gather_call(mk, T=big // 36 + 1) == mk.MLA_ERR_UNSUPPORTED
    assert "too many tokens" in mk.last_error()
    assert merge_call(mk, T=1 << 25) == mk.MLA_ERR_UNSUPPORTED
    assert "too many rows" in mk.last_error()
    assert new_token_call(mk, T=1 << 21) == mk.MLA_ERR_UNSUPPORTED
    assert "split the batch" in mk.last_error()
    assert mk.lib().mla_ctx_kv_proj(P16, 7168, big, 7168, P16, 2880, P16, 2880,
                                    None) == mk.MLA_ERR_UNSUPPORTED
    assert "beyond 2^31" in mk.last_error()
    # the projection's tile copies use 32-bit byte offsets: a 256-row tile of X
    # spanning 2 GiB (a row stride of about 4.2M elements, or K that large) is
    # refused (W's 192-row tiles span less, since X's stride is at least K)
    span = (1 << 30) // 255
    assert mk.lib().mla_ctx_kv_proj(P16, span + 64, 4, 64, P16, 16, P16, 16,
                                    None) == mk.MLA_ERR_UNSUPPORTED
    assert "2 GiB" in mk.last_error()
    big_k = (1 << 30) // 256 // 64 * 64 + 64
    assert mk.lib().mla_ctx_kv_proj(P16, big_k, 4, big_k, P16, 16, P16, 16,
                                    None) == mk.MLA_ERR_UNSUPPORTED
    assert "2 GiB" in mk.last_error()
    # just inside the limits the same calls pass validation (T = 0 variants are no-ops)
    assert pack_call(mk, T=0) == mk.MLA_OK


def test_proj_binding_refuses_a_strided_weight(mk):
    """The ABI takes W dense ([N, K], row stride K); a wider storage viewed as
    [N, K] is refused by the binding instead of being read with the wrong stride."""
    import torch
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    w = torch.zeros(32, 128, dtype=torch.bfloat16)[:, :64]
    y = torch.zeros(4, 32, dtype=torch.bfloat16)
    with pytest.raises(RuntimeError, match="row stride K"):
        mk.mla_ctx_kv_proj(x, w, y)
