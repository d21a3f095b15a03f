"""Paged decode attention for AMD MI355X (gfx950).

The compute path is the HIP library ``libpkv.so`` behind the C ABI in
``include/pkv.h``; :mod:`paged_kv_cache_08_amd.binding` marshals arguments to
it. :mod:`paged_kv_cache_08_amd.workloads` builds seeded synthetic inputs.
"""
from .binding import (  # noqa: F401
    DecodeParams, PreparedDecode, PKV_OUT_BF16, PKV_OUT_F32, debug_split_ranges, debug_token_offsets,
    debug_token_splits, device_cu_count, last_variant, lib, magic_div_check, make_params, paged_decode_attention,
    paged_decode_attention_noalloc, paged_prefill_attention,
    paged_varlen_attention, plan_constants,
    plan_splits, read_error_word, set_timing_events, validate, version, workspace_bytes,
)

__all__ = [
    "DecodeParams", "PreparedDecode", "paged_decode_attention", "paged_decode_attention_noalloc",
    "paged_varlen_attention", "paged_prefill_attention",
    "make_params", "plan_splits", "plan_constants",
    "workspace_bytes", "validate", "last_variant", "set_timing_events", "debug_token_offsets",
    "debug_split_ranges", "debug_token_splits", "device_cu_count", "magic_div_check", "read_error_word",
    "version", "lib",
]
