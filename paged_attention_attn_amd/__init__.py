"""Exact attention forward, chunked prefill and decode over a paged KV cache on AMD Instinct MI355X (gfx950).

The kernels are hand-written HIP in ``csrc/`` behind the C ABI declared in
``include/paged_attention_attn.h``; this package is the thin Python binding
(the same names as the C entry points, argument marshalling only).
"""

from ._binding import (  # noqa: F401
    LIB_PATH,
    PagedDecodeGraph,
    attn_fwd,
    attn_fwd_f32,
    attn_fwd_fp8,
    attn_fwd_window,
    attn_status_string,
    declared_functions,
    lib,
    paged_attn_decode,
    paged_attn_decode_fp8,
    paged_attn_decode_no_alloc,
    paged_attn_decode_workspace_size,
    paged_prefill,
)
