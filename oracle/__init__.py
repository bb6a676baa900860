"""CPU oracle for the MLA latent-KV insert / epilogue / gather / pack path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product library
(``fp8_paged_insert_amd``) never imports it, and this package never imports the
product library: the two share nothing but the seeded input generators.

The arithmetic lives in ``mla_oracle.c`` (plain serial C, built with gcc
``-O2 -fno-fast-math -ffp-contract=off``); this module only marshals numpy
arrays into it.  bf16 arrays are ``numpy.uint16`` bit patterns, fp8 arrays are
``numpy.uint8`` codes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB = os.path.join(_HERE, "libmla_oracle.so")

CACHE_BF16 = 0
CACHE_FP8_E4M3 = 1
CACHE_FP8_E5M2 = 2
PACK_KEY_BF16 = 0
PACK_KEY_V_FP8 = 1
PACK_KEY_V_FP8_KPE_RAW = 2
SRC_BF16 = 0
SRC_FP16 = 1
GATHER_BF16 = 0
GATHER_FP8_RAW = 1
MERGE_INIT_COPY = 0
MERGE_INIT_WRITTEN = 1
MERGE_ACCUMULATE = 2

OK = 0
EINVAL = -1
EDUPSLOT = -2


class OracleError(RuntimeError):
    pass


def build(force: bool = True) -> str:
    """Compile the oracle shared library with gcc; returns its path."""
    if not force and os.path.exists(_LIB):
        srcs = (_SRC, os.path.splitext(_SRC)[0] + ".h")
        if all(os.path.getmtime(x) <= os.path.getmtime(_LIB) for x in srcs):
            return _LIB
    tmp = _LIB + ".tmp"
    cmd = [
        "gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off",
        "-Wall", "-Wextra", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_f32 = ctypes.c_float
_f64 = ctypes.c_double
_int = ctypes.c_int


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    sig = {
        "orc_bf16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "orc_f64_to_bf16": (ctypes.c_uint16, [_f64]),
        "orc_e4m3_decode": (_f64, [ctypes.c_uint8]),
        "orc_e4m3_encode": (ctypes.c_uint8, [_f64]),
        "orc_quantize": (ctypes.c_uint8, [ctypes.c_uint16, _f32]),
        "orc_dequantize": (ctypes.c_uint16, [ctypes.c_uint8, _f32]),
        "orc_f64_to_bf16_n": (None, [_vp, _i64, _vp]),
        "orc_e4m3_encode_f32_n": (None, [_vp, _i64, _vp]),
        "orc_e4m3_decode_n": (None, [_vp, _i64, _vp]),
        "orc_quantize_n": (None, [_vp, _i64, _f32, _vp]),
        "orc_dequantize_n": (None, [_vp, _i64, _f32, _vp]),
        "orc_insert_single": (_int, [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64,
                                     _vp, _i64, _i64, _i64, _int, _f32]),
        "orc_insert_grouped": (_int, [_vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp,
                                      _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                      _i64, _i64, _int]),
        "orc_gemm_rows": (_int, [_vp, _i64, _vp, _i64, _i64, _i64, _i64, _vp,
                                 _i64, _vp]),
        "orc_rmsnorm_row": (_int, [_vp, _i64, _vp, _f32, _vp]),
        "orc_rope_row": (_int, [_vp, _i64, _i64, _f64, _vp]),
        "orc_ctx_kv_epilogue": (_int, [_vp, _i64, _i64, _vp, _f32, _vp, _f64,
                                       _i64, _i64, _i64, _i64, _vp, _vp, _vp,
                                       _i64, _i64, _i64, _i64, _int, _vp]),
        "orc_gather": (_int, [_vp, _int, _f32, _i64, _i64, _i64, _vp, _i64, _i64,
                              _int, _vp]),
        "orc_pack": (_int, [_vp, _i64, _i64, _vp, _i64, _vp, _i64, _i64, _i64,
                            _i64, _i64, _i64, _i64, _int, _int, _f32, _f32, _vp, _vp]),
        "orc_f16_to_f32_n": (None, [_vp, _i64, _vp]),
        "orc_new_token_epilogue": (_int, [_vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64,
                                          _vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _f64,
                                          _i64, _i64, _i64, _i64, _i64, _i64, _int,
                                          _f32, _f32, _f32, _vp, _vp, _vp,
                                          _vp, _vp, _i64, _i64, _i64, _int, _f32]),
        "orc_merge_chunk": (_int, [_vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _vp,
                                   _i64, _i64, _i64, _i64, _i64, _int]),
        "orc_neutralize_partials": (_int, [_vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64,
                                           _i64]),
        "orc_transpose_u16": (_int, [_vp, _i64, _i64, _i64, _vp, _i64]),
        "orc_e5m2_decode": (_f64, [ctypes.c_uint8]),
        "orc_e5m2_encode": (ctypes.c_uint8, [_f64]),
        "orc_e5m2_encode_f32_n": (None, [_vp, _i64, _vp]),
        "orc_e5m2_decode_n": (None, [_vp, _i64, _vp]),
        "orc_quantize_e5m2_n": (None, [_vp, _i64, _f32, _vp]),
        "orc_dequantize_e5m2_n": (None, [_vp, _i64, _f32, _vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _check(rc: int, what: str):
    if rc != OK:
        raise OracleError(f"{what}: oracle rejected the input (code {rc})")


def _need(a, dtype, name):
    if not isinstance(a, np.ndarray) or a.dtype != dtype:
        raise TypeError(f"{name} must be a numpy {np.dtype(dtype).name} array")


# ---------------------------------------------------------------- formats --
def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact)."""
    _need(bits, np.uint16, "bits")
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f64_to_bf16(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    _load().orc_f64_to_bf16_n(_ptr(x), x.size, _ptr(out))
    return out


def e4m3_encode(x) -> np.ndarray:
    """Saturating round-to-nearest-even float32 -> e4m3fn codes."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint8)
    _load().orc_e4m3_encode_f32_n(_ptr(x), x.size, _ptr(out))
    return out


def e4m3_encode_scalar(x: float) -> int:
    return int(_load().orc_e4m3_encode(float(x)))


def e4m3_decode(codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().orc_e4m3_decode_n(_ptr(c), c.size, _ptr(out))
    return out


def quantize(x_bf16: np.ndarray, scale: float) -> np.ndarray:
    x = np.ascontiguousarray(x_bf16)
    _need(x, np.uint16, "x_bf16")
    out = np.empty(x.shape, np.uint8)
    _load().orc_quantize_n(_ptr(x), x.size, float(scale), _ptr(out))
    return out


def dequantize(codes: np.ndarray, scale: float) -> np.ndarray:
    c = np.ascontiguousarray(codes)
    _need(c, np.uint8, "codes")
    out = np.empty(c.shape, np.uint16)
    _load().orc_dequantize_n(_ptr(c), c.size, float(scale), _ptr(out))
    return out


def e5m2_encode(x) -> np.ndarray:
    """Saturating round-to-nearest-even float32 -> e5m2 codes."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint8)
    _load().orc_e5m2_encode_f32_n(_ptr(x), x.size, _ptr(out))
    return out


def e5m2_decode(codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().orc_e5m2_decode_n(_ptr(c), c.size, _ptr(out))
    return out


def quantize_e5m2(x_bf16: np.ndarray, scale: float) -> np.ndarray:
    x = np.ascontiguousarray(x_bf16)
    _need(x, np.uint16, "x_bf16")
    out = np.empty(x.shape, np.uint8)
    _load().orc_quantize_e5m2_n(_ptr(x), x.size, float(scale), _ptr(out))
    return out


def dequantize_e5m2(codes: np.ndarray, scale: float) -> np.ndarray:
    c = np.ascontiguousarray(codes)
    _need(c, np.uint8, "codes")
    out = np.empty(c.shape, np.uint16)
    _load().orc_dequantize_e5m2_n(_ptr(c), c.size, float(scale), _ptr(out))
    return out


# ----------------------------------------------------------------- insert --
def _cache_dtype_code(cache: np.ndarray, fp8_format="e4m3") -> int:
    """uint16 arrays are bf16 caches; uint8 arrays hold fp8 codes of the
    given format ("e4m3" = e4m3fn, "e5m2")."""
    if cache.dtype == np.uint16:
        return CACHE_BF16
    if cache.dtype == np.uint8:
        if fp8_format == "e4m3":
            return CACHE_FP8_E4M3
        if fp8_format == "e5m2":
            return CACHE_FP8_E5M2
        raise ValueError(f"unknown fp8 format {fp8_format!r}")
    raise TypeError("cache must be uint16 (bf16) or uint8 (fp8 codes)")


def insert_single(kv_c, k_pe, slots, cache, scale=1.0, fp8_format="e4m3"):
    """In-place single-layer concat-and-cache.

    kv_c [T, R] uint16, k_pe [T, P] uint16 (row strides taken from the arrays),
    slots [T] int64, cache [num_blocks, block_size, E] (uint16 or uint8,
    strides taken from the array).
    """
    _need(kv_c, np.uint16, "kv_c")
    _need(k_pe, np.uint16, "k_pe")
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    it_c = kv_c.itemsize
    it = cache.itemsize
    rc = _load().orc_insert_single(
        _ptr(kv_c), kv_c.strides[0] // it_c, _ptr(k_pe), k_pe.strides[0] // it_c,
        _ptr(slots), slots.shape[0], kv_c.shape[1], k_pe.shape[1],
        _ptr(cache), cache.shape[1], cache.strides[0] // it, cache.strides[1] // it,
        _cache_dtype_code(cache, fp8_format), float(scale))
    _check(rc, "insert_single")


def insert_grouped(kv_c, k_pe, slot_mapping, caches, scales=None, fp8_format="e4m3"):
    """In-place grouped insert.

    kv_c [L, T, R] and k_pe [L, T, P] uint16 views with any strides;
    slot_mapping [L, T] int64 (layer stride 0 = shared mapping);
    caches: list of L arrays [num_blocks, block_size, E] with one layout;
    scales: float32 [L] for fp8 caches, None for bf16.
    """
    _need(kv_c, np.uint16, "kv_c")
    _need(k_pe, np.uint16, "k_pe")
    _need(slot_mapping, np.int64, "slot_mapping")
    L, T, R = kv_c.shape
    P = k_pe.shape[2]
    c0 = caches[0]
    it = c0.itemsize
    for c in caches:
        if c.dtype != c0.dtype or c.strides != c0.strides or c.shape[1] != c0.shape[1]:
            raise ValueError("caches must share dtype and layout")
    dt = _cache_dtype_code(c0, fp8_format)
    ptr_arr = (ctypes.c_void_p * max(L, 1))(*[c.ctypes.data for c in caches])
    sc = None
    if dt != CACHE_BF16:
        sc = np.ascontiguousarray(scales, dtype=np.float32)
    rc = _load().orc_insert_grouped(
        _ptr(kv_c), kv_c.strides[0] // 2, kv_c.strides[1] // 2,
        _ptr(k_pe), k_pe.strides[0] // 2, k_pe.strides[1] // 2,
        ctypes.cast(ptr_arr, ctypes.c_void_p), _ptr(sc),
        _ptr(slot_mapping), slot_mapping.strides[0] // 8,
        L, T, R, P, c0.shape[1], c0.strides[0] // it, c0.strides[1] // it, dt)
    _check(rc, "insert_grouped")


# ------------------------------------------- projection / norm / rope / epi --
def gemm_rows(x, w_kn, rows=None) -> np.ndarray:
    """Y[rows] = X[rows] . W with W addressed as the [K, N] matrix (any strides)."""
    _need(x, np.uint16, "x")
    _need(w_kn, np.uint16, "w_kn")
    T, K = x.shape
    K2, N = w_kn.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    if x.strides[1] != 2:
        raise ValueError("x rows must be contiguous")
    rows = np.arange(T, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    out = np.empty((rows.shape[0], N), np.uint16)
    rc = _load().orc_gemm_rows(_ptr(x), x.strides[0] // 2, _ptr(w_kn),
                               w_kn.strides[0] // 2, w_kn.strides[1] // 2, K, N,
                               _ptr(rows), rows.shape[0], _ptr(out))
    _check(rc, "gemm_rows")
    return out


def rmsnorm_row(x, gamma, eps) -> np.ndarray:
    x = np.ascontiguousarray(x, np.uint16)
    gamma = np.ascontiguousarray(gamma, np.uint16)
    out = np.empty_like(x)
    _check(_load().orc_rmsnorm_row(_ptr(x), x.size, _ptr(gamma), float(eps), _ptr(out)),
           "rmsnorm_row")
    return out


def rope_row(x, pos, base=10000.0) -> np.ndarray:
    x = np.ascontiguousarray(x, np.uint16)
    out = np.empty_like(x)
    _check(_load().orc_rope_row(_ptr(x), x.size, int(pos), float(base), _ptr(out)),
           "rope_row")
    return out


def ctx_kv_epilogue(all_kv, gamma, eps, positions, slot_mapping, caches,
                    scales=None, rope_base=10000.0, kv_lora_rank=512, fp8_format="e4m3"):
    """Norm + RoPE of every (layer, token) row, then the grouped insert.

    all_kv: [T, L, R+P] uint16 view (any strides); gamma [L, R] uint16;
    positions [T] int64; slot_mapping [L, T] int64 (layer stride 0 allowed);
    caches: list of L cache arrays, or None to compute the rows only.
    Returns the bf16 rows [L, T, R+P] that were inserted.
    """
    _need(all_kv, np.uint16, "all_kv")
    T, L, W = all_kv.shape
    R = kv_lora_rank
    P = W - R
    gamma = np.ascontiguousarray(gamma, np.uint16)
    positions = np.ascontiguousarray(positions, np.int64)
    rows = np.empty((L, T, W), np.uint16)
    ptrs = None
    dt = CACHE_BF16
    sc = None
    bs = bstride = estride = 1
    sls = 0
    if caches is not None:
        c0 = caches[0]
        it = c0.itemsize
        dt = _cache_dtype_code(c0, fp8_format)
        ptr_arr = (ctypes.c_void_p * max(L, 1))(*[c.ctypes.data for c in caches])
        ptrs = ctypes.cast(ptr_arr, ctypes.c_void_p)
        bs, bstride, estride = c0.shape[1], c0.strides[0] // it, c0.strides[1] // it
        _need(slot_mapping, np.int64, "slot_mapping")
        sls = slot_mapping.strides[0] // 8
        if dt != CACHE_BF16:
            sc = np.ascontiguousarray(scales, dtype=np.float32)
    rc = _load().orc_ctx_kv_epilogue(
        _ptr(all_kv), all_kv.strides[1] // 2, all_kv.strides[0] // 2, _ptr(gamma),
        float(eps), _ptr(positions), float(rope_base), L, T, R, P, ptrs, _ptr(sc),
        None if caches is None else _ptr(slot_mapping), sls, bs, bstride, estride,
        dt, _ptr(rows))
    _check(rc, "ctx_kv_epilogue")
    return rows


# --------------------------------------------------------- gather / pack --
def gather(cache, src_slots, scale=1.0, width=None, raw=False, fp8_format="e4m3") -> np.ndarray:
    """Contiguous [T, width] rows read through src_slots: bf16 (dequantised for
    an fp8 cache) or, with raw=True (fp8 caches only), the codes as they are."""
    dt = _cache_dtype_code(cache, fp8_format)
    it = cache.itemsize
    src_slots = np.ascontiguousarray(src_slots, np.int64)
    width = cache.shape[2] if width is None else width
    out = np.empty((src_slots.shape[0], width), np.uint8 if raw else np.uint16)
    rc = _load().orc_gather(_ptr(cache), dt, float(scale), cache.shape[1],
                            cache.strides[0] // it, cache.strides[1] // it,
                            _ptr(src_slots), src_slots.shape[0], width,
                            GATHER_FP8_RAW if raw else GATHER_BF16, _ptr(out))
    _check(rc, "gather")
    return out


def f16_to_f32(bits: np.ndarray) -> np.ndarray:
    """IEEE fp16 bit patterns -> float32 values (exact), via the oracle."""
    _need(bits, np.uint16, "bits")
    c = np.ascontiguousarray(bits)
    out = np.empty(c.shape, np.float32)
    _load().orc_f16_to_f32_n(_ptr(c), c.size, _ptr(out))
    return out


def pack(k_nope, k_pe, v=None, mode=PACK_KEY_BF16, k_scale=1.0, v_scale=1.0, fp16=False):
    """Full key [T, H, nope+rope] (+ fp8 V [T, H, vdim]) from strided inputs.

    k_nope [T, H, nope] uint16 view (last dim contiguous); k_pe [T, rope]
    uint16 view, or uint8 e4m3fn codes in PACK_KEY_V_FP8_KPE_RAW mode (last
    dim contiguous); v [T, H, vdim] uint16 view or None.  fp16=True reads the
    16-bit inputs as IEEE fp16 instead of bf16.
    """
    _need(k_nope, np.uint16, "k_nope")
    raw = mode == PACK_KEY_V_FP8_KPE_RAW
    _need(k_pe, np.uint8 if raw else np.uint16, "k_pe")
    T, H, nope = k_nope.shape
    rope = k_pe.shape[-1]
    esz = k_pe.itemsize
    if (k_nope.size and k_nope.strides[2] != 2) or (k_pe.size and k_pe.strides[-1] != esz):
        raise ValueError("innermost dimensions must be contiguous")
    kpe_ts = k_pe.strides[0] // esz
    if mode == PACK_KEY_BF16:
        key = np.empty((T, H, nope + rope), np.uint16)
        vout = None
        vd, vts, vhs = 0, 0, 0
    else:
        _need(v, np.uint16, "v")
        if v.size and v.strides[2] != 2:
            raise ValueError("v innermost dimension must be contiguous")
        vd = v.shape[2]
        vts, vhs = v.strides[0] // 2, v.strides[1] // 2
        key = np.empty((T, H, nope + rope), np.uint8)
        vout = np.empty((T, H, vd), np.uint8)
    rc = _load().orc_pack(_ptr(k_nope), k_nope.strides[0] // 2, k_nope.strides[1] // 2,
                          _ptr(k_pe), kpe_ts, _ptr(v), vts, vhs, T, H, nope, rope, vd,
                          mode, SRC_FP16 if fp16 else SRC_BF16, float(k_scale),
                          float(v_scale), _ptr(key), _ptr(vout))
    _check(rc, "pack")
    return key, vout


# ------------------------------------------------------ new-token epilogue --
def new_token_epilogue(q_nope, q_pe, k_nope, kv_c, k_pe, positions, v=None, mode=PACK_KEY_BF16,
                       q_scale=1.0, k_scale=1.0, v_scale=1.0, cache=None, slots=None,
                       cache_scale=1.0, fp8_format="e4m3", rope_base=10000.0):
    """RoPE of q_pe and k_pe, the query row, the chunked-context pack of the
    key (and V), and the insert of [kv_c | rotated k_pe] into `cache` (in place).

    q_nope [T, H, nope], q_pe [T, H, rope], k_nope [T, H, nope], v [T, H, vdim]
    uint16 views with contiguous last dims; kv_c [T, R], k_pe [T, rope] uint16
    views; positions [T] int64; cache [num_blocks, block_size, E] or None,
    slots [T] int64.  Returns (q_out, key, v_out) as the pack does.
    """
    for a, n in ((q_nope, "q_nope"), (q_pe, "q_pe"), (k_nope, "k_nope"), (kv_c, "kv_c"),
                 (k_pe, "k_pe")):
        _need(a, np.uint16, n)
        if a.size and a.strides[-1] != 2:
            raise ValueError(f"{n}: innermost dimension must be contiguous")
    T, H, nope = q_nope.shape
    rope = q_pe.shape[2]
    R = kv_c.shape[1]
    positions = np.ascontiguousarray(positions, np.int64)
    fp8 = mode != PACK_KEY_BF16
    q_out = np.empty((T, H, nope + rope), np.uint8 if fp8 else np.uint16)
    key = np.empty((T, H, nope + rope), np.uint8 if fp8 else np.uint16)
    vout, vd, vts, vhs = None, 0, 0, 0
    if fp8:
        _need(v, np.uint16, "v")
        vd = v.shape[2]
        vts, vhs = v.strides[0] // 2, v.strides[1] // 2
        vout = np.empty((T, H, vd), np.uint8)
    bs = bst = est = 0
    cdt = CACHE_BF16
    if cache is not None:
        slots = np.ascontiguousarray(slots, np.int64)
        it = cache.itemsize
        bs, bst, est = cache.shape[1], cache.strides[0] // it, cache.strides[1] // it
        cdt = _cache_dtype_code(cache, fp8_format)
    rc = _load().orc_new_token_epilogue(
        _ptr(q_nope), q_nope.strides[0] // 2, q_nope.strides[1] // 2,
        _ptr(q_pe), q_pe.strides[0] // 2, q_pe.strides[1] // 2,
        _ptr(k_nope), k_nope.strides[0] // 2, k_nope.strides[1] // 2,
        _ptr(v), vts, vhs, _ptr(kv_c), kv_c.strides[0] // 2, _ptr(k_pe), k_pe.strides[0] // 2,
        _ptr(positions), float(rope_base), T, H, nope, rope, vd, R, mode,
        float(q_scale), float(k_scale), float(v_scale), _ptr(q_out), _ptr(key), _ptr(vout),
        _ptr(cache), _ptr(slots), bs, bst, est, cdt, float(cache_scale))
    _check(rc, "new_token_epilogue")
    return q_out, key, vout


# ------------------------------------------------------------ chunk merge --
def merge_chunk(out, lse, part, part_lse, mode=MERGE_ACCUMULATE):
    """In-place merge of one chunk's partial into the accumulator.

    out / part: [T, H, D] uint16 (bf16 bits) views with contiguous rows;
    lse / part_lse: [H, T] float32 views (any strides).  Returns out, lse.
    """
    _need(out, np.uint16, "out")
    _need(part, np.uint16, "part")
    _need(lse, np.float32, "lse")
    _need(part_lse, np.float32, "part_lse")
    T, H, D = out.shape
    if part.shape != out.shape or lse.shape != (H, T) or part_lse.shape != (H, T):
        raise ValueError("shape mismatch")
    rc = _load().orc_merge_chunk(
        _ptr(out), out.strides[0] // 2, out.strides[1] // 2,
        _ptr(lse), lse.strides[0] // 4, lse.strides[1] // 4,
        _ptr(part), part.strides[0] // 2, part.strides[1] // 2,
        _ptr(part_lse), part_lse.strides[0] // 4, part_lse.strides[1] // 4, T, H, D, mode)
    _check(rc, "merge_chunk")
    return out, lse


def neutralize_partials(out, lse, no_context):
    """out[t] = 0 and lse[:, t] = -inf wherever no_context[t] is nonzero (in place)."""
    _need(out, np.uint16, "out")
    _need(lse, np.float32, "lse")
    T, H, D = out.shape
    m = np.ascontiguousarray(no_context, dtype=np.uint8)
    rc = _load().orc_neutralize_partials(
        _ptr(out), out.strides[0] // 2, out.strides[1] // 2,
        _ptr(lse), lse.strides[0] // 4, lse.strides[1] // 4, _ptr(m), T, H, D)
    _check(rc, "neutralize_partials")
    return out, lse


# ------------------------------------------------------ weight preparation --
def transpose(src: np.ndarray) -> np.ndarray:
    """[rows, cols] 16-bit bit patterns (rows may be strided) -> the
    contiguous [cols, rows] transpose."""
    _need(src, np.uint16, "src")
    rows, cols = src.shape
    if cols and src.strides[1] != 2:
        raise ValueError("src rows must be contiguous")
    out = np.empty((cols, rows), np.uint16)
    _check(_load().orc_transpose_u16(_ptr(src), rows, cols, src.strides[0] // 2, _ptr(out), rows),
           "transpose")
    return out
