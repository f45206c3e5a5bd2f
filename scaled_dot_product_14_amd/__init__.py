"""Fused scaled-dot-product attention for AMD MI355X (gfx950).

The compute lives in ``libsdpa14.so`` (hand-written HIP kernels behind the C ABI
declared in ``include/sdpa14.h``); this package is its thin Python binding.

    out, lse, seed, offset = sdpa_fwd(q, k, v, dropout_p, is_causal, scale)
    dq, dk, dv = sdpa_bwd(dout, q, k, v, out, lse, dropout_p, is_causal, seed, offset, scale)

Tensors are bf16 or fp16, logical [B, H, S, E], BHSE or BSHE stride order, E a
multiple of 8 up to 128.
``sdpa_fwd_ext`` / ``sdpa_bwd_ext`` add head sharding of the dropout stream, a
device-resident RNG state for captured graphs, an additive bias and its
gradient (``dbias``), a dropout keep-bit cache, an inference-only forward and
launching the backward's two kernels apart.  ``sdpa_bwd_noalloc`` is the
backward for callers that cannot allocate device memory.
"""

from ._binding import (  # noqa: F401
    EXPORTED,
    KERNEL_BWD,
    KERNEL_BWD_ROWS,
    KERNEL_FWD,
    LIB_PATH,
    SdpaError,
    describe,
    load_library,
    sdpa_bwd,
    sdpa_bwd_ext,
    sdpa_bwd_noalloc,
    sdpa_bwd_noalloc_max_rows,
    sdpa_bwd_workspace_size,
    sdpa_debug_dropout_mask,
    sdpa_fwd,
    sdpa_fwd_ext,
    sdpa_get_rng_state,
    sdpa_keep_bits_size,
    sdpa_profile_enable,
    sdpa_profile_read,
    sdpa_set_rng_state,
)
