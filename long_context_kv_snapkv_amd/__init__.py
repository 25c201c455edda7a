"""SnapKV prefill-time KV-cache compression for AMD Instinct MI355X (gfx950).

The computation lives in libsnapkv.so (C ABI in include/snapkv.h, kernels in
csrc/); this package is its Python binding. Build the library with
``python -m long_context_kv_snapkv_amd.build``.
"""

from .snapkv import (  # noqa: F401
    LIB_PATH,
    SNAPKV_CACHE_COMPRESSED,
    SNAPKV_CACHE_PACKED,
    SNAPKV_ERR_HIP,
    SNAPKV_ERR_INVALID_ARGUMENT,
    SNAPKV_ERR_UNSUPPORTED,
    SNAPKV_ERR_WORKSPACE,
    SNAPKV_NUM_STAGES,
    SNAPKV_OK,
    SNAPKV_POOL_AVG,
    SNAPKV_POOL_MAX,
    SNAPKV_STATIC_SCRATCH_BYTES,
    SnapKVError,
    SnapKVLibraryMissing,
    compress,
    header_functions,
    load_library,
    new_workspace,
    pool_mode_code,
    snapkv_compress,
    snapkv_compress_fp8,
    snapkv_compress_from_lse,
    snapkv_compress_int4,
    snapkv_compress_static,
    snapkv_compress_with_scores,
    snapkv_decode_attention,
    snapkv_decode_kernels,
    prepare_decode,
    DecodeStep,
    snapkv_decode_workspace_size,
    snapkv_last_error,
    snapkv_prefill_attention,
    snapkv_gather_selects,
    snapkv_select_kernels,
    snapkv_score_kernels,
    snapkv_stage_name,
    snapkv_status_string,
    snapkv_window_scores,
    snapkv_workspace_size,
)
