"""MI355X (gfx950) grouped MLA latent-KV insert, context-KV epilogue,
chunked-context gather / pack and the merge of chunk attention partials.

The computation lives in ``libmla_kv.so`` (hand-written HIP, built by
``python -m fp8_paged_insert_amd.build``); this package only marshals torch
tensors into its C ABI (``include/mla_kv.h``).  Importing the package does
not load the library; the first call does, and raises if it is not built.
"""
from ._binding import (  # noqa: F401
    EXPORTS,
    MLA_ERR_DEVICE,
    MLA_ERR_INVALID_ARGUMENT,
    MLA_ERR_MISALIGNED,
    MLA_ERR_UNSUPPORTED,
    MLA_KV_AUTO,
    MLA_KV_BF16,
    MLA_KV_FP8_E4M3,
    MLA_KV_FP8_E5M2,
    MLA_KV_FP16,
    MLA_OK,
    MLA_PACK_KEY_BF16,
    MLA_PACK_KEY_V_FP8,
    MLA_PACK_KEY_V_FP8_KPE_RAW,
    MLA_MERGE_INIT_COPY,
    MLA_MERGE_INIT_WRITTEN,
    MLA_MERGE_ACCUMULATE,
    LIB_PATH,
    MlaError,
    cache_ptr_table,
    last_error,
    lib,
    mla_ctx_kv_epilogue,
    mla_ctx_kv_pack,
    mla_ctx_kv_pack_gather,
    mla_ctx_kv_proj,
    mla_ctx_latent_gather,
    mla_ctx_merge_chunk,
    mla_ctx_neutralize_partials,
    mla_new_token_epilogue,
    mla_kv_insert_grouped,
    mla_rope_cos_sin_cache,
    mla_stream_copy,
    mla_transpose_bf16,
    parse_kv_cache_dtype,
    prepare_insert_grouped,
    PreparedInsert,
    set_launch_events,
    version,
)
