"""fp64 CPU oracle of SnapKV prefill-time KV-cache compression.

Test infrastructure: imported only by the test suite, the smoke check and the
CPU-baseline leg of the benchmark. The GPU library never imports or calls it.

Every function is pinned by the CPU test suite against closed forms, library
special cases, invariants and brute force (see tests/test_oracle_*.py); no
function here is "parity unpinned".
"""

from .snapkv_oracle import (  # noqa: F401
    POOL_AVG,
    POOL_MAX,
    OracleError,
    OracleResult,
    assemble_indices,
    bf16_bits_to_f64,
    causal_window_probs,
    compress,
    pool_code,
    pool_scores,
    prompt_scores,
    select_prefix,
    validate,
    window_lse,
    window_vote,
    window_vote_from_lse,
)
from .decode import attend, decode_compressed, decode_packed  # noqa: F401
from .prefill import causal_attention, prefill_attention, window_rows  # noqa: F401
from .kv_quant import (  # noqa: F401
    Fp8Result,
    Int4Result,
    e4m3_decode,
    e4m3_encode,
    quantize_cache_fp8,
    quantize_rows_fp8,
    compress_int4,
    dequantize_int4,
    pack_int4,
    quantize_cache,
    quantize_rows_int4,
    unpack_int4,
)
