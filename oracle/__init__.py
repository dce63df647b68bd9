"""fp64 CPU oracle for paged grouped-query attention (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (``fp8_kv_amd``) never
does, and this package imports nothing from it.
"""
from .oracle import (  # noqa: F401
    ORACLE_ERR_ARG,
    ORACLE_ERR_PAGE,
    ORACLE_ERR_TABLE,
    MASK_BAD_K,
    MASK_BAD_P,
    PAGE4_EMPTY,
    PAGE4_LONG,
    PAGE4_MAX_LIVE,
    PAGE4_OVERFLOW,
    PAGE4_PAGE,
    PAGE4_PARTIAL,
    PAGE4_SEQ,
    PAGE4_TAIL,
    OracleError,
    build,
    e4m3_table,
    e4m3_value,
    f16_decode,
    load,
    num_threads,
    paged_gqa,
    qsa_page4_table,
    topk_topp_mask,
    topk_select,
)
