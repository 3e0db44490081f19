"""MoE dispatch / combine on one MI355X: Python binding of libep_mi355x.so.

The binding only marshals arguments: it allocates output tensors with torch
(device memory is torch's plumbing), passes raw device pointers and torch's
current stream to the C ABI of ``include/ep_mi355x.h``, and turns status codes
into exceptions.  Every step of the path runs in the library's HIP kernels;
there is no fallback: if the library is missing, importing works but every
call raises.

    h = get_layout(Config(P, S, H, K, E, A), topk_idx)       # plan (syncs once)
    recv_x, recv_scales, recv_w, meta = dispatch(h, x, topk_weights, fp8=False,
                                                 zero_padding=True)
    y = experts(recv_x, ...)                                  # caller's work
    out = combine(h, y, topk_weights)
    h.free()
"""

from __future__ import annotations

from ._native import (  # noqa: F401
    EP_ABI_VERSION,
    Config,
    EpError,
    EventOverlap,
    Handle,
    LibraryMissing,
    STATUS_ROUTING,
    STATUS_TRUNCATED,
    Status,
    TENSORS,
    buffer_size_hint,
    combine,
    comm_stream,
    debug_copy,
    debug_e4m3_encode,
    dispatch,
    dispatch_cached,
    get_layout,
    lib,
    lib_path,
    relayout,
)
