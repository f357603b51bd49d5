"""Paged-KV decode attention (one or several query tokens per sequence) and
KV append on MI355X (gfx950).

The computation lives in the HIP library ``libpagedattn.so`` (C ABI declared
in ``include/pagedattn.h``); this package is its thin Python binding plus the
seeded workload generator used by the tests and the benchmark.
"""
from .binding import (  # noqa: F401
    CacheDesc,
    CapacityError,
    PagedAttnError,
    PoolAcct,
    acct_admit,
    acct_init,
    acct_retire,
    assign_slots,
    pool_init,
    pool_telemetry,
    prepare_assign_slots,
    release_seqs,
    rmsnorm,
    prepare_rmsnorm,
    attend,
    cache_desc,
    cache_shapes,
    decode,
    decode_append,
    decode_rope_append,
    lib,
    library_path,
    new_cache,
    new_workspace,
    prepare_attend,
    prepare_decode,
    prepare_decode_append,
    prepare_decode_rope_append,
    prepare_read_probe,
    prepare_write_kv,
    rope,
    workspace_bytes,
    write_kv,
)
