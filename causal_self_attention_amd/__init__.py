"""MI355X (gfx950) causal attention: flash-style forward, its VJP, the
materialized path (probabilities as an output), paged decode and the paged K/V
cache it reads (page leasing and appends).

The computation runs in the HIP kernels of ``libattn.so`` behind a C ABI
(``include/attn.h``); this package is a thin ctypes binding with the same
names.  torch is used only for device memory and streams.
"""
from ._binding import (  # noqa: F401
    ATTN_ABI_VERSION,
    ATTN_DEVICE_ERROR,
    ATTN_INVALID_ARGUMENT,
    ATTN_KV_OK,
    ATTN_KV_POOL_EXHAUSTED,
    ATTN_KV_SEQUENCE_FULL,
    ATTN_KV_STACK_OVERFLOW,
    ATTN_OK,
    ATTN_PAGED_DECODE_NOALLOC_SCRATCH_BYTES,
    ATTN_UNSUPPORTED,
    ATTN_WORKSPACE_TOO_SMALL,
    AttnError,
    PagedKvCache,
    PreparedPagedDecode,
    attn_abi_version,
    attn_causal_bwd,
    attn_causal_bwd_workspace_bytes,
    attn_causal_fwd,
    attn_kv_append,
    attn_kv_append_tokens,
    attn_kv_release,
    attn_last_error,
    attn_materialized_bwd,
    attn_materialized_bwd_workspace_bytes,
    attn_materialized_fwd,
    attn_paged_decode,
    attn_paged_decode_noalloc,
    attn_paged_decode_workspace_bytes,
    attn_paged_prefill,
    lib,
    library_path,
)
from .autograd import CausalAttentionFunction, causal_attention  # noqa: F401
