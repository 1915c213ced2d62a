"""MI355X-native GQA decode attention: RoPE + KV-cache append + split-K
flash-decoding, hand-written HIP for gfx950 behind a C ABI (libkvdecode.so).

The compute entry points are imported lazily from ``_binding`` so that the
workload generators and the sizing helpers import without the native library.
"""
__all__ = ["rope_append_kv", "gqa_decode_attn", "rope_append_kv_int8", "gqa_decode_attn_int8",
           "rope_append_kv_multi", "gqa_decode_attn_multi", "gqa_decode_step", "gqa_prefill_attn",
           "workspace_size", "library_path"]


def __getattr__(name):
    if name in __all__ or name in ("Options", "get_plan", "KvdError", "read_probe",
                                   "v_cache_shape_int8", "gqa_decode_attn_noalloc",
                                   "PREFILL_PAIRS_FASTEST", "PREFILL_TILES_FASTEST",
                                   "PREFILL_XCD_RUNS", "prefill_workspace_size",
                                   "rope_append_kv_mixed", "gqa_decode_attn_mixed",
                                   "workspace_size_mixed"):
        from . import _binding
        return getattr(_binding, name)
    raise AttributeError(name)
