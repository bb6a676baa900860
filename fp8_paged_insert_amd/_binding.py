"""ctypes binding of libmla_kv.so: argument marshalling only.

Every function here has the name and meaning of the C entry point declared in
``include/mla_kv.h``; it checks what raw pointers cannot express (tensor
dtype, device, contiguity, element counts), turns tensors into pointers,
strides and sizes, and calls the library on the current HIP stream of the
tensors' device.  No step of the computation runs here.  If the library is
not built, every call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmla_kv.so")

MLA_OK = 0
MLA_ERR_INVALID_ARGUMENT = 1
MLA_ERR_UNSUPPORTED = 2
MLA_ERR_MISALIGNED = 3
MLA_ERR_DEVICE = 4

MLA_KV_AUTO = 0
MLA_KV_BF16 = 1
MLA_KV_FP8_E4M3 = 2
MLA_KV_FP8_E5M2 = 3
MLA_KV_FP16 = 4

MLA_PACK_KEY_BF16 = 0
MLA_PACK_KEY_V_FP8 = 1
MLA_PACK_KEY_V_FP8_KPE_RAW = 2

MLA_MERGE_INIT_COPY = 0
MLA_MERGE_INIT_WRITTEN = 1
MLA_MERGE_ACCUMULATE = 2

# Every symbol include/mla_kv.h declares.
EXPORTS = (
    "mla_last_error", "mla_version", "mla_parse_kv_cache_dtype", "mla_set_launch_events",
    "mla_kv_insert_grouped", "mla_rope_cos_sin_cache", "mla_ctx_kv_epilogue",
    "mla_ctx_kv_proj", "mla_ctx_latent_gather", "mla_ctx_kv_pack", "mla_ctx_kv_pack_gather",
    "mla_ctx_merge_chunk", "mla_ctx_neutralize_partials", "mla_new_token_epilogue",
    "mla_stream_copy", "mla_stream_mix", "mla_transpose_bf16", "mla_mfma_rate",
)


class MlaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_i64, _i32, _vp, _f32, _f64 = (ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                               ctypes.c_float, ctypes.c_double)

_SIGS = {
    "mla_last_error": (ctypes.c_char_p, []),
    "mla_version": (ctypes.c_char_p, []),
    "mla_parse_kv_cache_dtype": (_i32, [ctypes.c_char_p, ctypes.POINTER(_i32)]),
    "mla_set_launch_events": (_i32, [_vp, _vp]),
    "mla_kv_insert_grouped": (_i32, [_vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _vp, _i64,
                                     _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i32, _vp]),
    "mla_rope_cos_sin_cache": (_i32, [_vp, _i64, _i64, _f64, _vp]),
    "mla_ctx_kv_epilogue": (_i32, [_vp, _i64, _i64, _vp, _f32, _vp, _vp, _i64, _vp, _vp, _vp,
                                   _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i32, _vp,
                                   _vp]),
    "mla_ctx_kv_proj": (_i32, [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp]),
    "mla_ctx_latent_gather": (_i32, [_vp, _i32, _vp, _i64, _i64, _i64, _vp, _i64, _i64, _i32,
                                     _vp, _i64, _vp]),
    "mla_ctx_kv_pack": (_i32, [_vp, _i64, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _i64,
                               _i64, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _i64, _vp]),
    "mla_ctx_kv_pack_gather": (_i32, [_vp, _i64, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i64,
                                      _i64, _i64, _i64, _i32, _i32, _vp, _vp, _vp, _vp,
                                      _vp, _i32, _vp, _i64, _i64, _i64, _vp, _i64, _i64, _i32,
                                      _vp, _i64, _vp]),
    "mla_stream_copy": (_i32, [_vp, _vp, _i64, _vp]),
    "mla_mfma_rate": (_i32, [_i64, _vp, _i64, _vp]),
    "mla_stream_mix": (_i32, [_vp, _vp, _i64, _i32, _vp]),
    "mla_transpose_bf16": (_i32, [_vp, _i64, _i64, _i64, _vp, _i64, _vp]),
    "mla_ctx_merge_chunk": (_i32, [_vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _vp,
                                   _i64, _i64, _i64, _i64, _i64, _i32, _vp]),
    "mla_ctx_neutralize_partials": (_i32, [_vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64,
                                           _i64, _vp]),
    "mla_new_token_epilogue": (_i32, [_vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _vp,
                                      _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _i64, _i64,
                                      _i64, _i64, _i64, _i64, _i64, _i32, _vp, _vp, _vp, _vp,
                                      _vp, _vp, _vp, _i32, _vp, _vp, _i64, _i64, _i64, _i64,
                                      _vp]),
}

_lib = None


def lib():
    """Load libmla_kv.so (torch is imported first so both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m fp8_paged_insert_amd.build` "
            "(or __graft_entry__.build()) first -- there is no fallback path")
    h = ctypes.CDLL(LIB_PATH, mode=ctypes.RTLD_GLOBAL)
    for name, (res, args) in _SIGS.items():
        fn = getattr(h, name)
        fn.restype = res
        fn.argtypes = args
    _lib = h
    return h


def last_error() -> str:
    return lib().mla_last_error().decode()


def version() -> str:
    return lib().mla_version().decode()


def _check(status: int, fn: str):
    if status != MLA_OK:
        raise MlaError(status, f"{fn} failed (status {status}): {last_error()}")


def parse_kv_cache_dtype(s: str) -> int:
    out = _i32(-1)
    _check(lib().mla_parse_kv_cache_dtype(s.encode(), ctypes.byref(out)),
           "mla_parse_kv_cache_dtype")
    return out.value


def set_launch_events(start=None, stop=None):
    """Arm timing events for the next kernel this thread launches through the
    library: torch.cuda.Event objects (already recorded once, so that their
    HIP events exist) or raw hipEvent_t handles; None, None disarms."""
    h0 = getattr(start, "cuda_event", start)
    h1 = getattr(stop, "cuda_event", stop)
    _check(lib().mla_set_launch_events(h0 or None, h1 or None), "mla_set_launch_events")


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_get_device = getattr(torch._C, "_cuda_getDevice", None)


def _stream(t: torch.Tensor):
    """torch's current HIP stream on the tensor's device (a hipStream_t).  The
    library launches on the calling thread's current device, so the tensors
    must live there (select it with torch.cuda.device / set_device).  Device
    indices are compared as integers: t.device builds a Python object on
    every access, which a small-batch call would pay several times."""
    idx = t.get_device()
    if idx < 0 or not t.is_cuda:
        raise RuntimeError(f"tensor on {t.device}, expected a GPU tensor")
    cur = _get_device() if _get_device is not None else torch.cuda.current_device()
    if idx != cur:
        raise RuntimeError(f"tensors on {t.device} but the current device is cuda:{cur}; "
                           f"call under torch.cuda.device({idx})")
    if _raw_stream is not None:
        return _raw_stream(cur)
    return torch.cuda.current_stream(cur).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t, dtypes, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise RuntimeError(f"{name} must have dtype {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")


def _same_device(t, ref, name, ref_name):
    if t.get_device() != ref.get_device() or t.is_cuda != ref.is_cuda:
        raise RuntimeError(f"{name} is not on the same CUDA device as {ref_name} "
                           f"({t.device} vs {ref.device})")


def _check_scales(scales, n, ref, name="kv_scales"):
    _need(scales, (torch.float32,), name)
    if scales.numel() != n:
        raise RuntimeError(f"{name} must hold one scale per layer: expected {n}, got {scales.numel()}")
    _same_device(scales, ref, name, "kv_c")
    if not scales.is_contiguous():
        raise RuntimeError(f"{name} must be contiguous")


_dtype_codes = {}


def _cache_dtype_code(kv_cache_dtype) -> int:
    """Dtype string -> code through the library's parser (memoised)."""
    if isinstance(kv_cache_dtype, str):
        code = _dtype_codes.get(kv_cache_dtype)
        if code is None:
            code = parse_kv_cache_dtype(kv_cache_dtype)
            _dtype_codes[kv_cache_dtype] = code
        return code
    return int(kv_cache_dtype)


def cache_ptr_table(caches, device=None) -> torch.Tensor:
    """int64 device tensor of per-layer cache base addresses."""
    device = device or caches[0].device
    return torch.tensor([c.data_ptr() for c in caches], dtype=torch.int64).to(device)


# tensor dtypes that may hold each fp8 cache format's codes
_FP8_TENSOR_DTYPES = {MLA_KV_FP8_E4M3: (torch.uint8, torch.float8_e4m3fn),
                      MLA_KV_FP8_E5M2: (torch.uint8, torch.float8_e5m2)}


def _is_fp8(dt) -> bool:
    return dt in _FP8_TENSOR_DTYPES


def _resolve_caches(kv_caches, L, dt, width, block_size, block_stride, entry_stride, ref):
    """Accept either an int64 device table of base addresses (the raw C form;
    layout and dtype are then the caller's promise) or the list of per-layer
    cache tensors, whose dtype and layout are checked against the arguments
    before their table is built."""
    if isinstance(kv_caches, torch.Tensor):
        _need(kv_caches, (torch.int64,), "kv_cache_ptrs")
        if kv_caches.numel() != L:
            raise RuntimeError(f"kv_cache_ptrs must hold {L} addresses")
        _same_device(kv_caches, ref, "kv_cache_ptrs", "kv_c")
        return kv_caches
    caches = list(kv_caches)
    if len(caches) != L:
        raise RuntimeError(f"expected {L} caches, got {len(caches)}")
    want = _FP8_TENSOR_DTYPES.get(dt, (torch.bfloat16,))
    c0 = caches[0]
    for i, c in enumerate(caches):
        _need(c, want, f"cache {i} (for kv_cache_dtype code {dt})")
        _same_device(c, ref, f"cache {i}", "kv_c")
        if c.dim() != 3 or c.stride() != c0.stride() or c.shape != c0.shape:
            raise RuntimeError("all caches must be [num_blocks, block_size, entry] with one layout")
    if c0.shape[1] != block_size or c0.stride(0) != block_stride or c0.stride(1) != entry_stride:
        raise RuntimeError(
            f"block_size / block_stride / entry_stride ({block_size}, {block_stride}, "
            f"{entry_stride}) disagree with the cache layout "
            f"({c0.shape[1]}, {c0.stride(0)}, {c0.stride(1)})")
    if c0.stride(2) != 1 or c0.shape[2] < width:
        raise RuntimeError(f"cache entries must hold {width} contiguous elements")
    return cache_ptr_table(caches, ref.device)


def _slots_2d(slot_mapping, L, T):
    """[T] (shared) or [L, T] int64 -> (tensor, layer stride)."""
    _need(slot_mapping, (torch.int64,), "slot_mapping")
    if slot_mapping.dim() == 1:
        if slot_mapping.shape[0] != T:
            raise RuntimeError(f"slot_mapping has {slot_mapping.shape[0]} entries, expected {T}")
        if slot_mapping.stride(0) != 1:
            raise RuntimeError("slot_mapping must be contiguous along tokens")
        return slot_mapping, 0
    if tuple(slot_mapping.shape) != (L, T):
        raise RuntimeError(f"slot_mapping shape {tuple(slot_mapping.shape)}, expected ({L}, {T})")
    if T > 1 and slot_mapping.stride(1) != 1:
        raise RuntimeError("slot_mapping must be contiguous along tokens")
    return slot_mapping, slot_mapping.stride(0) if L > 1 else 0


# ---------------------------------------------------------------------------
def _insert_args(kv_c, k_pe, kv_cache_ptrs, slot_mapping, block_size, block_stride,
                 entry_stride, kv_scales, kv_cache_dtype):
    """Check and marshal the grouped-insert arguments; returns the C argument
    tuple and the device pointer table it refers to."""
    _need(kv_c, (torch.bfloat16,), "kv_c")
    _need(k_pe, (torch.bfloat16,), "k_pe")
    if kv_c.dim() != 3 or k_pe.dim() != 3:
        raise RuntimeError("kv_c and k_pe must be [num_layers, num_tokens, dim] views")
    L, T, R = kv_c.shape
    Lp, Tp, P = k_pe.shape
    if (Lp, Tp) != (L, T):
        raise RuntimeError("kv_c and k_pe disagree on layers/tokens")
    skv, spe = kv_c.stride(), k_pe.stride()
    if (R > 1 and skv[2] != 1) or (P > 1 and spe[2] != 1):
        raise RuntimeError("kv_c / k_pe innermost dimension must be contiguous")
    _same_device(k_pe, kv_c, "k_pe", "kv_c")
    sm, sls = _slots_2d(slot_mapping, L, T)
    _same_device(sm, kv_c, "slot_mapping", "kv_c")
    dt = _cache_dtype_code(kv_cache_dtype)
    kv_cache_ptrs = _resolve_caches(kv_cache_ptrs, L, dt, R + P, block_size, block_stride,
                                    entry_stride, kv_c)
    if _is_fp8(dt):
        if kv_scales is None:
            raise RuntimeError("an fp8 cache needs kv_scales (one fp32 scale per layer)")
        _check_scales(kv_scales, L, kv_c)
    elif kv_scales is not None:
        raise RuntimeError("a bf16 cache takes no kv_scales")
    args = (_ptr(kv_c), skv[0], skv[1], _ptr(k_pe), spe[0],
            spe[1], _ptr(kv_cache_ptrs), _ptr(kv_scales), _ptr(sm), sls, L, T, R, P,
            int(block_size), int(block_stride), int(entry_stride), dt, _stream(kv_c))
    return args, kv_cache_ptrs


def mla_kv_insert_grouped(kv_c, k_pe, kv_cache_ptrs, slot_mapping, block_size,
                          block_stride, entry_stride, kv_scales=None,
                          kv_cache_dtype="auto"):
    """Grouped insert of [kv_c | k_pe] rows of every layer into its paged cache.

    kv_c [L, T, R] / k_pe [L, T, P] bf16 views (innermost dim contiguous);
    kv_cache_ptrs: int64 [L] device table of cache bases, or the list of L
    cache tensors (then checked against the dtype and layout arguments);
    slot_mapping int64 [L, T] (layer stride 0 allowed) or [T] shared;
    block/entry strides in cache elements; kv_scales fp32 [L] for fp8 caches,
    None otherwise.
    """
    args, _ = _insert_args(kv_c, k_pe, kv_cache_ptrs, slot_mapping, block_size, block_stride,
                           entry_stride, kv_scales, kv_cache_dtype)
    _check(lib().mla_kv_insert_grouped(*args), "mla_kv_insert_grouped")


class PreparedInsert:
    """mla_kv_insert_grouped with its arguments checked once.  Calling the
    object enqueues the same insert again on the current stream of the
    tensors' device: their contents may change between calls, their storage
    and layout may not.  Meant for decode loops inserting a few tokens per
    step, where the per-call checks would cost more than the kernel."""

    def __init__(self, kv_c, k_pe, kv_cache_ptrs, slot_mapping, block_size, block_stride,
                 entry_stride, kv_scales=None, kv_cache_dtype="auto"):
        args, table = _insert_args(kv_c, k_pe, kv_cache_ptrs, slot_mapping, block_size,
                                   block_stride, entry_stride, kv_scales, kv_cache_dtype)
        self._keep = (kv_c, k_pe, table, slot_mapping, kv_scales)  # keep storage alive
        self._args = list(args)
        self._index = kv_c.device.index if kv_c.device.index is not None else \
            torch.cuda.current_device()
        self._fn = lib().mla_kv_insert_grouped

    def __call__(self):
        cur = _get_device() if _get_device is not None else torch.cuda.current_device()
        if cur != self._index:
            raise RuntimeError(f"prepared on cuda:{self._index} but the current device is "
                               f"cuda:{cur}")
        self._args[-1] = (_raw_stream(self._index) if _raw_stream is not None else
                          torch.cuda.current_stream(self._index).cuda_stream)
        st = self._fn(*self._args)
        if st != MLA_OK:
            _check(st, "mla_kv_insert_grouped")


def prepare_insert_grouped(*args, **kwargs) -> PreparedInsert:
    return PreparedInsert(*args, **kwargs)


def mla_rope_cos_sin_cache(out, max_pos, rope_dim, base=10000.0):
    """Fill the fp32 [max_pos, 2 * rope_dim] rotary table (cos hi | sin hi |
    cos lo | sin lo of each position's angles) on the device."""
    _need(out, (torch.float32,), "out")
    if not out.is_contiguous() or out.numel() != max_pos * 2 * rope_dim:
        raise RuntimeError("out must be a contiguous fp32 [max_pos, 2 * rope_dim] tensor")
    _check(lib().mla_rope_cos_sin_cache(_ptr(out), int(max_pos), int(rope_dim), float(base),
                                        _stream(out)), "mla_rope_cos_sin_cache")


def mla_ctx_kv_epilogue(all_kv, gamma, eps, positions, cos_sin, kv_cache_ptrs, slot_mapping,
                        block_size, block_stride, entry_stride, kv_scales=None,
                        kv_cache_dtype="auto", kv_lora_rank=512, dbg_rows=None):
    """RMSNorm + RoPE + quantise + grouped insert for all_kv [T, L, R+P] (bf16 view)."""
    _need(all_kv, (torch.bfloat16,), "all_kv")
    _need(gamma, (torch.bfloat16,), "gamma")
    _need(positions, (torch.int64,), "positions")
    _need(cos_sin, (torch.float32,), "cos_sin")
    if all_kv.dim() != 3 or all_kv.stride(2) != 1:
        raise RuntimeError("all_kv must be a [T, L, width] view with contiguous rows")
    T, L, W = all_kv.shape
    R = int(kv_lora_rank)
    P = W - R
    if tuple(gamma.shape) != (L, R) or not gamma.is_contiguous():
        raise RuntimeError(f"gamma must be contiguous [{L}, {R}]")
    if positions.numel() != T or not positions.is_contiguous():
        raise RuntimeError(f"positions must be contiguous [{T}]")
    if cos_sin.dim() != 2 or cos_sin.shape[1] != 2 * P or not cos_sin.is_contiguous():
        raise RuntimeError(f"cos_sin must be a contiguous fp32 [max_pos, {2 * P}] table")
    for t, n in ((gamma, "gamma"), (positions, "positions"), (cos_sin, "cos_sin")):
        _same_device(t, all_kv, n, "all_kv")
    sm, sls = _slots_2d(slot_mapping, L, T)
    _same_device(sm, all_kv, "slot_mapping", "all_kv")
    dt = _cache_dtype_code(kv_cache_dtype)
    kv_cache_ptrs = _resolve_caches(kv_cache_ptrs, L, dt, W, block_size, block_stride,
                                    entry_stride, all_kv)
    if _is_fp8(dt):
        if kv_scales is None:
            raise RuntimeError("an fp8 cache needs kv_scales (one fp32 scale per layer)")
        _check_scales(kv_scales, L, all_kv)
    elif kv_scales is not None:
        raise RuntimeError("a bf16 cache takes no kv_scales")
    if dbg_rows is not None:
        _need(dbg_rows, (torch.bfloat16,), "dbg_rows")
        if tuple(dbg_rows.shape) != (L, T, W) or not dbg_rows.is_contiguous():
            raise RuntimeError(f"dbg_rows must be contiguous [{L}, {T}, {W}]")
    st = lib().mla_ctx_kv_epilogue(
        _ptr(all_kv), all_kv.stride(1), all_kv.stride(0), _ptr(gamma), float(eps),
        _ptr(positions), _ptr(cos_sin), cos_sin.shape[0], _ptr(kv_cache_ptrs), _ptr(kv_scales),
        _ptr(sm), sls, L, T, R, P, int(block_size), int(block_stride), int(entry_stride), dt,
        _ptr(dbg_rows), _stream(all_kv))
    _check(st, "mla_ctx_kv_epilogue")


def mla_ctx_kv_proj(x, w_nk, y):
    """y[T, N] = x[T, K] . w_nk[N, K]^T (bf16 in/out, fp32 accumulation)."""
    for t, n in ((x, "x"), (w_nk, "w_nk"), (y, "y")):
        _need(t, (torch.bfloat16,), n)
        if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
            raise RuntimeError(f"{n} must be a 2-D row-major matrix")
    T, K = x.shape
    N = w_nk.shape[0]
    if w_nk.shape[1] != K or tuple(y.shape) != (T, N):
        raise RuntimeError("shape mismatch: x [T, K], w_nk [N, K], y [T, N]")
    if N > 1 and w_nk.stride(0) != K:
        raise RuntimeError("w_nk must be a dense [N, K] weight (row stride K)")
    _same_device(w_nk, x, "w_nk", "x")
    _same_device(y, x, "y", "x")
    _check(lib().mla_ctx_kv_proj(_ptr(x), x.stride(0), T, K, _ptr(w_nk), N, _ptr(y),
                                 y.stride(0), _stream(x)), "mla_ctx_kv_proj")


def _gather_args(cache, src_slots, out, cache_scale, kv_cache_dtype):
    """Checked argument list of the gather (without max_blocks and stream)."""
    _need(src_slots, (torch.int64,), "src_slots")
    raw = out.dtype != torch.bfloat16
    dt = _cache_dtype_code(kv_cache_dtype)
    if _is_fp8(dt):
        _need(cache, _FP8_TENSOR_DTYPES[dt], "cache")
        _need(out, (torch.bfloat16,) + _FP8_TENSOR_DTYPES[dt], "out")
        if raw:
            if cache_scale is not None:
                raise RuntimeError("the raw fp8 gather does not dequantise; pass no cache_scale")
        else:
            if cache_scale is None:
                raise RuntimeError("an fp8 cache needs cache_scale")
            _check_scales(cache_scale, 1, cache, "cache_scale")
    else:
        _need(cache, (torch.bfloat16,), "cache")
        _need(out, (torch.bfloat16, torch.uint8), "out")
        if raw:
            raise RuntimeError("a raw fp8 gather needs an fp8 cache")
        if cache_scale is not None:
            raise RuntimeError("a bf16 cache takes no cache_scale")
    if cache.dim() != 3 or cache.stride(2) != 1:
        raise RuntimeError("cache must be a [num_blocks, block_size, entry] view")
    T = src_slots.numel()
    if out.dim() != 2 or out.shape[0] != T or not out.is_contiguous():
        raise RuntimeError(f"out must be contiguous [{T}, width]")
    if not src_slots.is_contiguous():
        raise RuntimeError("src_slots must be contiguous")
    _same_device(src_slots, cache, "src_slots", "cache")
    _same_device(out, cache, "out", "cache")
    return (_ptr(cache), dt, _ptr(cache_scale), cache.shape[1], cache.stride(0),
            cache.stride(1), _ptr(src_slots), T, out.shape[1], dt if raw else MLA_KV_BF16,
            _ptr(out))


def mla_transpose_bf16(src, dst):
    """dst[c, r] = src[r, c]: src bf16 [rows, cols] with contiguous rows,
    dst bf16 [cols, rows] with contiguous rows (weight preparation for
    mla_ctx_kv_proj: the [K, N] matrix -> its [N, K] storage)."""
    _need(src, (torch.bfloat16,), "src")
    _need(dst, (torch.bfloat16,), "dst")
    if src.dim() != 2 or dst.dim() != 2 or tuple(dst.shape) != (src.shape[1], src.shape[0]):
        raise RuntimeError("src [rows, cols] and dst [cols, rows] expected")
    for t, n in ((src, "src"), (dst, "dst")):
        if t.shape[1] > 1 and t.stride(1) != 1:
            raise RuntimeError(f"{n} must have contiguous rows")
    _same_device(dst, src, "dst", "src")
    _check(lib().mla_transpose_bf16(_ptr(src), src.shape[0], src.shape[1], src.stride(0),
                                    _ptr(dst), dst.stride(0), _stream(src)), "mla_transpose_bf16")


def mla_ctx_latent_gather(cache, src_slots, out, cache_scale=None, kv_cache_dtype="fp8",
                          max_blocks=0):
    """out[j, :] = cache row of src_slots[j]; cache [num_blocks, block_size, E].

    A bf16 `out` receives bf16 rows (dequantised with cache_scale for an fp8
    cache); a uint8 (or same-format float8) `out` receives an fp8 cache's
    codes as they are (no cache_scale).
    """
    args = _gather_args(cache, src_slots, out, cache_scale, kv_cache_dtype)
    _check(lib().mla_ctx_latent_gather(*args, int(max_blocks), _stream(cache)),
           "mla_ctx_latent_gather")


_SRC_DTYPES = {torch.bfloat16: MLA_KV_BF16, torch.float16: MLA_KV_FP16}
_FP8_VIEWS = (torch.uint8, torch.float8_e4m3fn)


def _pack_args(k_nope, k_pe, key_out, v, v_out, mode, k_scale, v_scale):
    """Checked argument list of the pack (without max_blocks and stream)."""
    _need(k_nope, tuple(_SRC_DTYPES), "k_nope")
    src = _SRC_DTYPES[k_nope.dtype]
    if k_pe.dim() == 3:  # [T, 1, rope]
        k_pe = k_pe.reshape(k_pe.shape[0], k_pe.shape[-1])
    kpe_raw = k_pe.dtype in _FP8_VIEWS
    if mode == MLA_PACK_KEY_V_FP8 and kpe_raw:
        mode = MLA_PACK_KEY_V_FP8_KPE_RAW
    if mode == MLA_PACK_KEY_V_FP8_KPE_RAW:
        _need(k_pe, _FP8_VIEWS, "k_pe")
    else:
        _need(k_pe, (k_nope.dtype,), "k_pe")
    T, H, nope = k_nope.shape
    rope = k_pe.shape[1]
    if (nope > 1 and k_nope.stride(2) != 1) or (rope > 1 and k_pe.stride(1) != 1):
        raise RuntimeError("k_nope / k_pe innermost dimension must be contiguous")
    if k_pe.shape[0] != T:
        raise RuntimeError("k_pe must have one row per token")
    _same_device(k_pe, k_nope, "k_pe", "k_nope")
    _same_device(key_out, k_nope, "key_out", "k_nope")
    if not key_out.is_contiguous() or tuple(key_out.shape) != (T, H, nope + rope):
        raise RuntimeError(f"key_out must be contiguous [{T}, {H}, {nope + rope}]")
    vd = vts = vhs = 0
    if mode == MLA_PACK_KEY_BF16:
        _need(key_out, (k_nope.dtype,), "key_out")
        if v is not None or v_out is not None or k_scale is not None or v_scale is not None:
            raise RuntimeError("the 16-bit key mode takes no v, v_out or scales")
    elif mode in (MLA_PACK_KEY_V_FP8, MLA_PACK_KEY_V_FP8_KPE_RAW):
        _need(key_out, _FP8_VIEWS, "key_out")
        _need(v, (k_nope.dtype,), "v")
        _need(v_out, _FP8_VIEWS, "v_out")
        if tuple(v.shape[:2]) != (T, H) or (v.shape[2] > 1 and v.stride(2) != 1):
            raise RuntimeError("v must be a [T, H, vdim] view with contiguous rows")
        vd, vts, vhs = v.shape[2], v.stride(0), v.stride(1)
        if not v_out.is_contiguous() or tuple(v_out.shape) != (T, H, vd):
            raise RuntimeError(f"v_out must be contiguous [{T}, {H}, {vd}]")
        _same_device(v, k_nope, "v", "k_nope")
        _same_device(v_out, k_nope, "v_out", "k_nope")
        for sc, n in ((k_scale, "k_scale"), (v_scale, "v_scale")):
            if sc is not None:
                _check_scales(sc, 1, k_nope, n)
    else:
        raise RuntimeError(f"unknown pack mode {mode}")
    return (_ptr(k_nope), k_nope.stride(0), k_nope.stride(1), _ptr(k_pe), k_pe.stride(0),
            _ptr(v), vts, vhs, T, H, nope, rope, vd, int(mode), src, _ptr(k_scale),
            _ptr(v_scale), _ptr(key_out), _ptr(v_out))


def mla_ctx_kv_pack(k_nope, k_pe, key_out, v=None, v_out=None, mode=MLA_PACK_KEY_BF16,
                    k_scale=None, v_scale=None, max_blocks=0):
    """Contiguous full key [T, H, nope+rope] (+ fp8 V) from strided k_nope / k_pe / v.

    k_nope and v are bf16 or fp16.  k_pe has k_nope's dtype, or -- in the fp8
    modes -- holds fp8 codes (uint8 / float8_e4m3fn, e.g. a view of a raw fp8
    gather), which are copied into the key as they are.
    """
    args = _pack_args(k_nope, k_pe, key_out, v, v_out, mode, k_scale, v_scale)
    _check(lib().mla_ctx_kv_pack(*args, int(max_blocks), _stream(k_nope)), "mla_ctx_kv_pack")


def mla_ctx_kv_pack_gather(k_nope, k_pe, key_out, cache, src_slots, gather_out, v=None,
                           v_out=None, mode=MLA_PACK_KEY_BF16, k_scale=None, v_scale=None,
                           cache_scale=None, kv_cache_dtype="fp8", max_blocks=0):
    """One launch: the pack of one chunk (arguments as mla_ctx_kv_pack;
    max_blocks caps its part of the grid) and the latent gather of the next
    (as mla_ctx_latent_gather, into gather_out, which must not overlap the
    pack's tensors)."""
    pa = _pack_args(k_nope, k_pe, key_out, v, v_out, mode, k_scale, v_scale)
    ga = _gather_args(cache, src_slots, gather_out, cache_scale, kv_cache_dtype)
    _same_device(cache, k_nope, "cache", "k_nope")
    _check(lib().mla_ctx_kv_pack_gather(*pa, *ga, int(max_blocks), _stream(k_nope)),
           "mla_ctx_kv_pack_gather")


# ------------------------------------------------------ new-token epilogue --
def mla_new_token_epilogue(q_nope, q_pe, k_nope, kv_c, k_pe, positions, cos_sin, q_out, key_out,
                           v=None, v_out=None, mode=MLA_PACK_KEY_BF16, q_scale=None,
                           k_scale=None, v_scale=None, cache=None, slot_mapping=None,
                           kv_cache_dtype="auto", cache_scale=None, max_blocks=0):
    """RoPE of q_pe / k_pe, the query row [q_nope | RoPE(q_pe)], the full key
    [k_nope | RoPE(k_pe)] (+ fp8 V), and the insert of [kv_c | RoPE(k_pe)]
    into one layer's paged cache [num_blocks, block_size, >= R + rope].

    q_nope / q_pe / k_nope / v: bf16 [T, H, d] views with contiguous rows;
    kv_c / k_pe: bf16 [T, d] views; positions int64 [T]; cos_sin fp32
    [max_pos, 2 * rope] (mla_rope_cos_sin_cache).  q_out / key_out [T, H, nope+rope]
    and v_out [T, H, vdim] contiguous: bf16 in KEY_BF16 mode, fp8 e4m3fn
    (uint8 or float8_e4m3fn) in KEY_V_FP8 mode.  cache=None skips the insert.
    """
    for t_, n in ((q_nope, "q_nope"), (q_pe, "q_pe"), (k_nope, "k_nope"), (kv_c, "kv_c"),
                  (k_pe, "k_pe")):
        _need(t_, (torch.bfloat16,), n)
        if t_.shape[-1] > 1 and t_.stride(-1) != 1:
            raise RuntimeError(f"{n} innermost dimension must be contiguous")
        _same_device(t_, q_nope, n, "q_nope")
    if k_pe.dim() == 3:  # [T, 1, rope]
        k_pe = k_pe.reshape(k_pe.shape[0], k_pe.shape[-1])
    T, H, nope = q_nope.shape
    rope = q_pe.shape[2]
    if tuple(q_pe.shape[:2]) != (T, H) or tuple(k_nope.shape) != (T, H, nope):
        raise RuntimeError("q_pe / k_nope must be [T, H, d] like q_nope")
    if kv_c.dim() != 2 or kv_c.shape[0] != T or tuple(k_pe.shape) != (T, rope):
        raise RuntimeError("kv_c must be [T, R] and k_pe [T, rope]")
    R = kv_c.shape[1]
    _need(positions, (torch.int64,), "positions")
    if positions.numel() != T or not positions.is_contiguous():
        raise RuntimeError("positions must be a contiguous int64 [T] tensor")
    _need(cos_sin, (torch.float32,), "cos_sin")
    if cos_sin.dim() != 2 or cos_sin.shape[1] != 2 * rope or not cos_sin.is_contiguous():
        raise RuntimeError(f"cos_sin must be a contiguous fp32 [max_pos, {2 * rope}] table")
    for t_, n in ((positions, "positions"), (cos_sin, "cos_sin"), (q_out, "q_out"),
                  (key_out, "key_out")):
        _same_device(t_, q_nope, n, "q_nope")
    for t_, n in ((q_out, "q_out"), (key_out, "key_out")):
        if not t_.is_contiguous() or tuple(t_.shape) != (T, H, nope + rope):
            raise RuntimeError(f"{n} must be contiguous [{T}, {H}, {nope + rope}]")
    vd = vts = vhs = 0
    if mode == MLA_PACK_KEY_BF16:
        _need(q_out, (torch.bfloat16,), "q_out")
        _need(key_out, (torch.bfloat16,), "key_out")
        if any(x is not None for x in (v, v_out, q_scale, k_scale, v_scale)):
            raise RuntimeError("the bf16 mode takes no v, v_out or query/key/V scales")
    elif mode == MLA_PACK_KEY_V_FP8:
        _need(q_out, _FP8_VIEWS, "q_out")
        _need(key_out, _FP8_VIEWS, "key_out")
        _need(v, (torch.bfloat16,), "v")
        _need(v_out, _FP8_VIEWS, "v_out")
        if tuple(v.shape[:2]) != (T, H) or (v.shape[2] > 1 and v.stride(2) != 1):
            raise RuntimeError("v must be a [T, H, vdim] view with contiguous rows")
        vd, vts, vhs = v.shape[2], v.stride(0), v.stride(1)
        if not v_out.is_contiguous() or tuple(v_out.shape) != (T, H, vd):
            raise RuntimeError(f"v_out must be contiguous [{T}, {H}, {vd}]")
        _same_device(v, q_nope, "v", "q_nope")
        _same_device(v_out, q_nope, "v_out", "q_nope")
        for sc, n in ((q_scale, "q_scale"), (k_scale, "k_scale"), (v_scale, "v_scale")):
            if sc is not None:
                _check_scales(sc, 1, q_nope, n)
    else:
        raise RuntimeError(f"unknown new-token mode {mode}")
    dt = _cache_dtype_code(kv_cache_dtype)
    bs = bst = est = 0
    if cache is not None:
        _need(cache, _FP8_TENSOR_DTYPES.get(dt, (torch.bfloat16,)), "cache")
        if cache.dim() != 3 or cache.shape[2] < R + rope or cache.stride(2) != 1:
            raise RuntimeError(f"cache must be [num_blocks, block_size, >= {R + rope}] with "
                               "contiguous entries")
        _same_device(cache, q_nope, "cache", "q_nope")
        _need(slot_mapping, (torch.int64,), "slot_mapping")
        if slot_mapping.numel() != T or not slot_mapping.is_contiguous():
            raise RuntimeError("slot_mapping must be a contiguous int64 [T] tensor")
        _same_device(slot_mapping, q_nope, "slot_mapping", "q_nope")
        if _is_fp8(dt):
            if cache_scale is None:
                raise RuntimeError("an fp8 cache requires cache_scale")
            _check_scales(cache_scale, 1, q_nope, "cache_scale")
        elif cache_scale is not None:
            raise RuntimeError("a bf16 cache does not use cache_scale")
        bs, bst, est = cache.shape[1], cache.stride(0), cache.stride(1)
    elif slot_mapping is not None or cache_scale is not None:
        raise RuntimeError("slot_mapping / cache_scale given without a cache")
    st = lib().mla_new_token_epilogue(
        _ptr(q_nope), q_nope.stride(0), q_nope.stride(1), _ptr(q_pe), q_pe.stride(0),
        q_pe.stride(1), _ptr(k_nope), k_nope.stride(0), k_nope.stride(1), _ptr(v), vts, vhs,
        _ptr(kv_c), kv_c.stride(0), _ptr(k_pe), k_pe.stride(0), _ptr(positions), _ptr(cos_sin),
        cos_sin.shape[0], T, H, nope, rope, vd, R, int(mode), _ptr(q_scale), _ptr(k_scale),
        _ptr(v_scale), _ptr(q_out), _ptr(key_out), _ptr(v_out), _ptr(cache), dt,
        _ptr(cache_scale), _ptr(slot_mapping), bs, bst, est, int(max_blocks), _stream(q_nope))
    _check(st, "mla_new_token_epilogue")


# ------------------------------------------------------------ chunk merge --
def _check_partial(o, lse, T, H, D, name, lname, ref):
    _need(o, (torch.bfloat16,), name)
    _need(lse, (torch.float32,), lname)
    if o.dim() != 3 or tuple(o.shape) != (T, H, D) or (D > 1 and o.stride(2) != 1):
        raise RuntimeError(f"{name} must be a [{T}, {H}, {D}] view with contiguous rows")
    if lse.dim() != 2 or tuple(lse.shape) != (H, T):
        raise RuntimeError(f"{lname} must be a [{H}, {T}] view (heads, tokens)")
    _same_device(o, ref, name, "out")
    _same_device(lse, ref, lname, "out")


def mla_ctx_merge_chunk(out, lse, part, part_lse, mode=MLA_MERGE_ACCUMULATE):
    """Fold one chunk's partial (part [T, H, D] bf16, part_lse [H, T] fp32) into
    the accumulator (out, lse), in place.  In MLA_MERGE_INIT_WRITTEN mode the
    chunk's output is already in `out`; pass part=None (or out)."""
    if out.dim() != 3:
        raise RuntimeError("out must be [num_tokens, num_heads, head_dim]")
    T, H, D = out.shape
    _check_partial(out, lse, T, H, D, "out", "lse", out)
    if mode == MLA_MERGE_INIT_WRITTEN and part is None:
        part = out
    _check_partial(part, part_lse, T, H, D, "part", "part_lse", out)
    st = lib().mla_ctx_merge_chunk(
        _ptr(out), out.stride(0), out.stride(1), _ptr(lse), lse.stride(0), lse.stride(1),
        None if mode == MLA_MERGE_INIT_WRITTEN else _ptr(part), part.stride(0), part.stride(1),
        _ptr(part_lse), part_lse.stride(0), part_lse.stride(1), T, H, D, int(mode), _stream(out))
    _check(st, "mla_ctx_merge_chunk")


def mla_ctx_neutralize_partials(out, lse, no_context):
    """out[t] = 0 and lse[:, t] = -inf wherever no_context[t] (bool/uint8 [T]) is set."""
    if out.dim() != 3:
        raise RuntimeError("out must be [num_tokens, num_heads, head_dim]")
    T, H, D = out.shape
    _check_partial(out, lse, T, H, D, "out", "lse", out)
    _need(no_context, (torch.uint8, torch.bool), "no_context")
    if no_context.numel() != T or not no_context.is_contiguous():
        raise RuntimeError(f"no_context must be a contiguous [{T}] mask")
    _same_device(no_context, out, "no_context", "out")
    st = lib().mla_ctx_neutralize_partials(
        _ptr(out), out.stride(0), out.stride(1), _ptr(lse), lse.stride(0), lse.stride(1),
        _ptr(no_context), T, H, D, _stream(out))
    _check(st, "mla_ctx_neutralize_partials")


# ------------------------------------------------------------ measurement --
def mla_stream_copy(dst, src):
    """dst <- src (same number of bytes, contiguous, 16-byte multiples), with
    the library's streaming launch shape: a measurement aid."""
    if not (dst.is_contiguous() and src.is_contiguous()):
        raise RuntimeError("dst and src must be contiguous")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise RuntimeError("dst and src must have the same size in bytes")
    _same_device(dst, src, "dst", "src")
    _check(lib().mla_stream_copy(_ptr(dst), _ptr(src), nbytes, _stream(src)), "mla_stream_copy")


def mla_stream_mix(dst, src, reads_per_write):
    """dst chunk i <- XOR of src chunks r i .. r i + r - 1 (16-byte chunks,
    r = reads_per_write; src holds r times dst's bytes), with the library's
    streaming launch shape: a measurement aid."""
    if not (dst.is_contiguous() and src.is_contiguous()):
        raise RuntimeError("dst and src must be contiguous")
    nbytes = dst.numel() * dst.element_size()
    if src.numel() * src.element_size() != nbytes * reads_per_write:
        raise RuntimeError("src must hold reads_per_write times the bytes of dst")
    _same_device(dst, src, "dst", "src")
    _check(lib().mla_stream_mix(_ptr(dst), _ptr(src), nbytes, int(reads_per_write),
                                _stream(src)), "mla_stream_mix")


def mla_mfma_rate(clocks, iters):
    """Runs the library's MFMA issue-rate kernel (one workgroup of 4
    wavefronts per CU, iters x 12 v_mfma_f32_32x32x16_bf16 per wavefront)
    and leaves in clocks (int64 device tensor, 16 words per CU) each
    wavefront's shader-clock and 100 MHz real-time readings at start and end:
    a measurement aid."""
    if clocks.dtype != torch.int64 or not clocks.is_contiguous() or not clocks.is_cuda:
        raise RuntimeError("clocks must be a contiguous int64 device tensor")
    _check(lib().mla_mfma_rate(int(iters), _ptr(clocks), clocks.numel(), _stream(clocks)),
           "mla_mfma_rate")
