"""ctypes binding of the C ABI in include/ep_mi355x.h (argument marshalling only)."""

from __future__ import annotations

import ctypes
import dataclasses
import enum
import os

PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libep_mi355x.so"
EP_ABI_VERSION = 4

# dispatch flags
_FP8 = 1
_ZERO_PADDING = 2
_SCALES_COL_MAJOR = 4
_SCALES_UE8M0 = 8
_SYMMETRIC_WINDOWS = 1
# ep_handle_status bits
STATUS_ROUTING = 1
STATUS_TRUNCATED = 2


class Status(enum.IntEnum):
    OK = 0
    ERR_NULL = -1
    ERR_SHAPE = -2
    ERR_ROUTING = -3
    ERR_OVERFLOW = -4
    ERR_HANDLE_MISMATCH = -5
    ERR_HIP = -6
    ERR_NOMEM = -7


# handle tensor ids -> (name, id, numpy-ish dtype name)
TENSORS = {
    "is_token_in_rank": (0, "uint8"),
    "num_tokens_per_rank": (1, "int32"),
    "num_tokens_per_expert": (2, "int32"),
    "rank_prefix_matrix": (3, "int32"),
    "num_recv_tokens": (4, "int32"),
    "num_tokens_per_expert_total": (5, "int32"),
    "expert_offset": (6, "int64"),
    "num_expanded": (7, "int64"),
    "window_row_base": (8, "int64"),
    "dst_slot": (9, "int32"),
    "send_head": (10, "int32"),
    "recv_src_idx": (11, "int32"),
    "recv_src_base": (12, "int64"),
    "dst_row": (13, "int32"),
}


class LibraryMissing(RuntimeError):
    pass


class EpError(RuntimeError):
    def __init__(self, status: int, message: str):
        try:
            name = Status(status).name
        except ValueError:
            name = str(status)
        super().__init__(f"{name}: {message}")
        self.status = status


class _Config(ctypes.Structure):
    _fields_ = [
        ("num_ranks", ctypes.c_int32),
        ("num_tokens", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("num_topk", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("expert_alignment", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("num_worst_rows", ctypes.c_int32),
    ]


class _SizeHint(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int64) for name in (
        "handle_bytes", "max_rows", "recv_x_bytes", "recv_scales_bytes", "recv_weights_bytes",
        "recv_src_meta_bytes", "combine_out_bytes", "total_bytes")]


@dataclasses.dataclass(frozen=True)
class Config:
    """P virtual ranks x S tokens, hidden H, top-K of E experts, expert_alignment A.

    num_worst_rows > 0 fixes every window at that many expanded rows (no read-back)."""

    P: int
    S: int
    H: int
    K: int
    E: int
    A: int
    symmetric_windows: bool = False
    num_worst_rows: int = 0

    def _c(self) -> _Config:
        return _Config(self.P, self.S, self.H, self.K, self.E, self.A,
                       _SYMMETRIC_WINDOWS if self.symmetric_windows else 0, self.num_worst_rows)

    @property
    def T(self) -> int:
        return self.P * self.S


_lib = None


def lib_path() -> str:
    return os.path.join(PKG, _LIB_NAME)


def lib() -> ctypes.CDLL:
    """Load libep_mi355x.so (built in-tree by build.py); raise if it is not there."""
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise LibraryMissing(f"{path} is not built; run `python -m combine_topk_idx_expert_amd.build` "
                                 "or __graft_entry__.build()")
        L = ctypes.CDLL(path)
        vp, i32, u32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_int64
        L.ep_get_layout.argtypes = [ctypes.POINTER(_Config), vp, vp, ctypes.POINTER(vp), ctypes.POINTER(i64)]
        L.ep_relayout.argtypes = [vp, vp, vp, ctypes.POINTER(i64)]
        L.ep_buffer_size_hint.argtypes = [ctypes.POINTER(_Config), u32, ctypes.POINTER(_SizeHint)]
        L.ep_buffer_size_hint.restype = i32
        L.ep_dispatch.argtypes = [vp, u32, vp, vp, vp, vp, vp, vp, vp]
        L.ep_dispatch_noalloc.argtypes = [vp, u32, vp, vp, vp, vp, vp, vp, vp]
        L.ep_dispatch_cached.argtypes = [vp, u32, vp, vp, vp, vp]
        L.ep_dispatch_prequant.argtypes = [vp, u32, vp, vp, vp, vp, vp, vp, vp, vp]
        L.ep_dispatch_prequant_cached.argtypes = [vp, u32, vp, vp, vp, vp, vp]
        L.ep_combine.argtypes = [vp, vp, vp, vp, vp, vp]
        L.ep_handle_free.argtypes = [vp]
        L.ep_handle_free.restype = None
        L.ep_handle_config.argtypes = [vp, ctypes.POINTER(_Config)]
        L.ep_handle_check.argtypes = [vp, ctypes.POINTER(_Config)]
        L.ep_handle_counts.argtypes = [vp, vp, vp, vp]
        L.ep_handle_status.argtypes = [vp, ctypes.POINTER(u32), ctypes.POINTER(i64)]
        L.ep_handle_tensor.argtypes = [vp, i32, ctypes.POINTER(vp), ctypes.POINTER(i64), ctypes.POINTER(i32)]
        for fn in ("ep_get_layout", "ep_relayout", "ep_dispatch", "ep_dispatch_noalloc", "ep_dispatch_cached",
                   "ep_dispatch_prequant",
                   "ep_dispatch_prequant_cached", "ep_combine",
                   "ep_handle_config", "ep_handle_check", "ep_handle_counts", "ep_handle_status",
                   "ep_handle_tensor"):
            getattr(L, fn).restype = i32
        L.ep_debug_e4m3_encode.argtypes = [vp, vp, i64, vp]
        L.ep_debug_e4m3_encode.restype = i32
        L.ep_debug_timing.argtypes = [vp, i64]
        L.ep_debug_timing.restype = i32
        L.ep_debug_copy.argtypes = [vp, vp, i64, vp]
        L.ep_debug_copy.restype = i32
        L.ep_last_error.argtypes = []
        L.ep_last_error.restype = ctypes.c_char_p
        L.ep_abi_version.argtypes = []
        L.ep_abi_version.restype = i32
        if L.ep_abi_version() != EP_ABI_VERSION:
            raise LibraryMissing(f"{path}: ABI version {L.ep_abi_version()} != {EP_ABI_VERSION}")
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise EpError(status, lib().ep_last_error().decode(errors="replace"))


def _stream(device) -> int:
    """torch's current stream on ``device`` as a hipStream_t.  torch's raw accessor is used
    when present: it skips building a Stream object (~0.2 against ~1.8 us per call)."""
    import torch

    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None and device.index is not None:
        return raw(device.index)
    return torch.cuda.current_stream(device).cuda_stream


def _on(device):
    """``torch.cuda.device(device)``, or nothing when it is already the current device (the
    usual case; entering the context costs ~1 us)."""
    import contextlib

    import torch

    if device.index is not None and torch.cuda.current_device() == device.index:
        return contextlib.nullcontext()
    return torch.cuda.device(device)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _require(t, dtype, shape, name, device=None):
    """Every tensor handed to the library is checked here: the C ABI takes bare
    pointers, so a wrong size or device would only show up as a memory fault."""
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the handle on {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _require_recv(h, recv_x, recv_scales, fp8: bool, scales_col_major: bool, scales_ue8m0: bool = False):
    """Caller-provided expanded outputs: [total_rows, H] payload and, for fp8, the scales."""
    import torch

    H, R = h.cfg.H, h.total_rows
    _require(recv_x, torch.uint8 if fp8 else torch.bfloat16, (R, H), "recv_x", h.device)
    if fp8:
        if recv_scales is None:
            raise ValueError("recv_scales is required for fp8 output")
        if scales_ue8m0:
            _require(recv_scales, torch.uint8, (R, H // 32), "recv_scales (UE8M0)", h.device)
        else:
            shape = (H // 128, R) if scales_col_major else (R, H // 128)
            _require(recv_scales, torch.float32, shape, "recv_scales", h.device)


class Handle:
    """Owns an ep_handle*: the layout of one routing table."""

    def __init__(self, ptr: int, cfg: Config, total_rows: int, device):
        self._ptr = ptr
        self.cfg = cfg
        self.total_rows = total_rows
        self.device = device
        self._pending = []  # completion events of async calls that read the handle

    @property
    def ptr(self) -> int:
        if not self._ptr:
            raise ValueError("handle was freed")
        return self._ptr

    def free(self) -> None:
        """Release the handle's device memory.  Work already enqueued with it may still read
        it, so the device's current stream and the handle's pending async calls are waited for
        first (also when the handle is garbage collected)."""
        if self._ptr:
            import torch

            for ev in self._pending:
                ev.synchronize()
            self._pending.clear()
            torch.cuda.current_stream(self.device).synchronize()
            lib().ep_handle_free(self._ptr)
            self._ptr = None

    def __del__(self):  # pragma: no cover - best effort
        try:
            self.free()
        except Exception:
            pass

    def check(self, cfg: Config) -> None:
        c = cfg._c()
        _check(lib().ep_handle_check(self.ptr, ctypes.byref(c)))

    def counts(self):
        """(num_expanded [P], num_recv_tokens [P], window_row_base [P+1]) as numpy int64."""
        import numpy as np

        P = self.cfg.P
        ne, nr, wb = np.zeros(P, np.int64), np.zeros(P, np.int64), np.zeros(P + 1, np.int64)
        _check(lib().ep_handle_counts(self.ptr, ne.ctypes.data, nr.ctypes.data, wb.ctypes.data))
        return ne, nr, wb

    def status(self):
        """(EP_STATUS_* flags, dropped rows) of the last layout; waits for it in fixed mode."""
        f, d = ctypes.c_uint32(), ctypes.c_int64()
        _check(lib().ep_handle_status(self.ptr, ctypes.byref(f), ctypes.byref(d)))
        return f.value, d.value

    def tensor(self, name: str):
        """A device copy (torch tensor) of one of the handle's arrays."""
        import torch

        which, dt = TENSORS[name]
        p, n, b = ctypes.c_void_p(), ctypes.c_int64(), ctypes.c_int32()
        _check(lib().ep_handle_tensor(self.ptr, which, ctypes.byref(p), ctypes.byref(n), ctypes.byref(b)))
        out = torch.empty(n.value, dtype=getattr(torch, dt), device=self.device)
        if n.value:
            _hip_memcpy_d2d(out.data_ptr(), p.value, n.value * b.value, _stream(self.device))
        return out


_hip = None


def _hip_memcpy_d2d(dst: int, src: int, nbytes: int, stream: int) -> None:
    """Stream-ordered device-to-device copy through the HIP runtime (plumbing)."""
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                        ctypes.c_void_p]
        _hip.hipMemcpyAsync.restype = ctypes.c_int
    rc = _hip.hipMemcpyAsync(dst, src, nbytes, 3, stream)  # hipMemcpyDeviceToDevice
    if rc != 0:
        raise EpError(Status.ERR_HIP, f"hipMemcpyAsync failed ({rc})")


class EventOverlap:
    """Work enqueued on the library's communication stream, not yet ordered before the
    caller's stream: the tutorial's EventOverlap (ch. 38, section 3.4).  ``wait()`` makes the
    caller's current stream wait for it and returns the call's results."""

    def __init__(self, event, result):
        self.event = event
        self._result = result

    def wait(self):
        import torch

        torch.cuda.current_stream().wait_event(self.event)
        return self._result


_comm_streams: dict = {}


def comm_stream(device):
    """The library's communication stream on ``device`` (created once, default priority)."""
    import torch

    idx = torch.device(device).index
    if idx is None:
        idx = torch.cuda.current_device()
    if idx not in _comm_streams:
        _comm_streams[idx] = torch.cuda.Stream(device=idx)
    return _comm_streams[idx]


def _overlapped(h, device, tensors, launch, previous_event):
    """Run ``launch`` on the communication stream after ``previous_event`` (default: all
    work enqueued so far on the current stream); return an EventOverlap.  The tensors the
    call reads or writes are marked as used on the communication stream, so that torch's
    allocator does not hand their memory out again before that work is done."""
    import torch

    compute = torch.cuda.current_stream(device)
    comm = comm_stream(device)
    if previous_event is None:
        previous_event = torch.cuda.Event()
        previous_event.record(compute)
    comm.wait_event(previous_event)
    with torch.cuda.stream(comm):
        result = launch()
    for t in tensors:
        if t is not None:
            t.record_stream(comm)
    done = torch.cuda.Event()
    done.record(comm)
    h._pending = [e for e in h._pending if not e.query()]
    h._pending.append(done)  # h.free() waits for it
    return EventOverlap(done, result)


def buffer_size_hint(cfg: Config, fp8: bool = False, scales_ue8m0: bool = False) -> dict:
    """ep_buffer_size_hint: device bytes the config needs (handle arena, expanded tensors at
    their largest row count, combine output, total rounded up to 2 MiB), computed on the host;
    nothing is allocated."""
    out = _SizeHint()
    _check(lib().ep_buffer_size_hint(ctypes.byref(cfg._c()), _flags(fp8, False, False, scales_ue8m0),
                                     ctypes.byref(out)))
    return {name: getattr(out, name) for name, _ in _SizeHint._fields_}


def get_layout(cfg: Config, topk_idx) -> Handle:
    """ep_get_layout: topk_idx int64 [T, K] on the device -> Handle (synchronizes once in exact
    mode; only enqueues with cfg.num_worst_rows > 0)."""
    import torch

    _require(topk_idx, torch.int64, (cfg.T, cfg.K), "topk_idx")
    c = cfg._c()
    h = ctypes.c_void_p()
    rows = ctypes.c_int64()
    with _on(topk_idx.device):
        _check(lib().ep_get_layout(ctypes.byref(c), _ptr(topk_idx), _stream(topk_idx.device), ctypes.byref(h),
                                   ctypes.byref(rows)))
    return Handle(h.value, cfg, rows.value, topk_idx.device)


def relayout(h: Handle, topk_idx) -> Handle:
    """ep_relayout: new routing for an existing handle of the same config (no allocation)."""
    import torch

    _require(topk_idx, torch.int64, (h.cfg.T, h.cfg.K), "topk_idx", h.device)
    # the new layout overwrites the handle's arrays: order it after the async calls still
    # reading them (a stream wait, no host synchronisation)
    if h._pending:
        cur = torch.cuda.current_stream(h.device)
        for ev in h._pending:
            cur.wait_event(ev)
        h._pending.clear()
    rows = ctypes.c_int64()
    with _on(topk_idx.device):
        _check(lib().ep_relayout(h.ptr, _ptr(topk_idx), _stream(topk_idx.device), ctypes.byref(rows)))
    h.total_rows = rows.value
    return h


def _flags(fp8: bool, zero_padding: bool, scales_col_major: bool = False, scales_ue8m0: bool = False) -> int:
    return ((_FP8 if fp8 else 0) | (_ZERO_PADDING if zero_padding else 0) |
            (_SCALES_COL_MAJOR if scales_col_major else 0) | (_SCALES_UE8M0 if scales_ue8m0 else 0))


def _alloc_recv(h: Handle, fp8: bool, device, scales_col_major: bool = False, scales_ue8m0: bool = False):
    import torch

    H, R = h.cfg.H, h.total_rows
    recv_x = torch.empty((R, H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=device)
    recv_scales = None
    if fp8 and scales_ue8m0:
        recv_scales = torch.empty((R, H // 32), dtype=torch.uint8, device=device)
    elif fp8:
        shape = (H // 128, R) if scales_col_major else (R, H // 128)
        recv_scales = torch.empty(shape, dtype=torch.float32, device=device)
    return recv_x, recv_scales


def _input(h: Handle, x):
    """x: bf16 [T, H], or the pre-quantised pair (E4M3 bytes uint8 [T, H], fp32 scales [T, H/128])."""
    import torch

    cfg = h.cfg
    if isinstance(x, tuple):
        codes, scales = x
        _require(codes, torch.uint8, (cfg.T, cfg.H), "x codes", h.device)
        _require(scales, torch.float32, (cfg.T, cfg.H // 128), "x scales", h.device)
        return codes, scales, codes.device
    _require(x, torch.bfloat16, (cfg.T, cfg.H), "x", h.device)
    return x, None, x.device


def dispatch(h: Handle, x, topk_weights, fp8: bool = False, zero_padding: bool = False,
             scales_col_major: bool = False, out=None, async_with_compute_stream: bool = False,
             previous_event=None, scales_ue8m0: bool = False):
    """ep_dispatch (x bf16) or ep_dispatch_prequant (x = (codes, scales), output fp8)
    -> (recv_x, recv_scales | None, recv_weights, recv_src_meta).

    scales_ue8m0: fp8 output with one UE8M0 exponent byte per 32 channels (recv_scales uint8
    [total_rows, H/32]); implies fp8.

    out: optional preallocated (recv_x, recv_scales, recv_weights, recv_src_meta).
    async_with_compute_stream: run on the library's communication stream after
    previous_event (default: the current stream's work so far) and return an EventOverlap
    whose wait() gives the tuple; one such call per handle may be in flight at a time."""
    import torch

    cfg = h.cfg
    xin, xs, device = _input(h, x)
    fp8 = fp8 or xs is not None or scales_ue8m0
    _require(topk_weights, torch.float32, (cfg.T, cfg.K), "topk_weights", h.device)
    if out is None:
        recv_x, recv_scales = _alloc_recv(h, fp8, device, scales_col_major, scales_ue8m0)
        recv_w = torch.empty(h.total_rows, dtype=torch.float32, device=device)
        recv_meta = torch.empty((h.total_rows, 2), dtype=torch.int32, device=device)
    else:
        recv_x, recv_scales, recv_w, recv_meta = out
        _require_recv(h, recv_x, recv_scales, fp8, scales_col_major, scales_ue8m0)
        _require(recv_w, torch.float32, (h.total_rows,), "recv_weights", h.device)
        _require(recv_meta, torch.int32, (h.total_rows, 2), "recv_src_meta", h.device)
    flags = _flags(fp8, zero_padding, scales_col_major, scales_ue8m0)

    def launch():
        with _on(device):
            if xs is None:
                _check(lib().ep_dispatch(h.ptr, flags, _ptr(xin), _ptr(topk_weights), _ptr(recv_x),
                                         _ptr(recv_scales), _ptr(recv_w), _ptr(recv_meta), _stream(device)))
            else:
                _check(lib().ep_dispatch_prequant(h.ptr, flags, _ptr(xin), _ptr(xs), _ptr(topk_weights),
                                                  _ptr(recv_x), _ptr(recv_scales), _ptr(recv_w), _ptr(recv_meta),
                                                  _stream(device)))
        return recv_x, recv_scales, recv_w, recv_meta

    if not async_with_compute_stream:
        return launch()
    return _overlapped(h, device, [xin, xs, topk_weights, recv_x, recv_scales, recv_w, recv_meta], launch,
                       previous_event)


def dispatch_cached(h: Handle, x, fp8: bool = False, zero_padding: bool = False, scales_col_major: bool = False,
                    out=None, async_with_compute_stream: bool = False, previous_event=None,
                    scales_ue8m0: bool = False):
    """ep_dispatch_cached / ep_dispatch_prequant_cached -> (recv_x, recv_scales | None);
    out: optional (recv_x, recv_scales); async_with_compute_stream and scales_ue8m0 as in
    dispatch."""
    import torch

    xin, xs, device = _input(h, x)
    fp8 = fp8 or xs is not None or scales_ue8m0
    if out is None:
        recv_x, recv_scales = _alloc_recv(h, fp8, device, scales_col_major, scales_ue8m0)
    else:
        recv_x, recv_scales = out
        _require_recv(h, recv_x, recv_scales, fp8, scales_col_major, scales_ue8m0)
    flags = _flags(fp8, zero_padding, scales_col_major, scales_ue8m0)

    def launch():
        with _on(device):
            if xs is None:
                _check(lib().ep_dispatch_cached(h.ptr, flags, _ptr(xin), _ptr(recv_x), _ptr(recv_scales),
                                                _stream(device)))
            else:
                _check(lib().ep_dispatch_prequant_cached(h.ptr, flags, _ptr(xin), _ptr(xs), _ptr(recv_x),
                                                         _ptr(recv_scales), _stream(device)))
        return recv_x, recv_scales

    if not async_with_compute_stream:
        return launch()
    return _overlapped(h, device, [xin, xs, recv_x, recv_scales], launch, previous_event)


def combine(h: Handle, y, topk_weights=None, bias=None, out=None, async_with_compute_stream: bool = False,
            previous_event=None):
    """ep_combine: y bf16 [total_rows, H] (+ optional bias bf16 [T, H]) -> out bf16 [T, H];
    async_with_compute_stream as in dispatch (wait() gives out)."""
    import torch

    cfg = h.cfg
    _require(y, torch.bfloat16, (h.total_rows, cfg.H), "y", h.device)
    if topk_weights is not None:
        _require(topk_weights, torch.float32, (cfg.T, cfg.K), "topk_weights", h.device)
    if bias is not None:
        _require(bias, torch.bfloat16, (cfg.T, cfg.H), "bias", h.device)
    if out is None:
        out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=y.device)
    else:
        _require(out, torch.bfloat16, (cfg.T, cfg.H), "out", h.device)

    def launch():
        with _on(y.device):
            _check(lib().ep_combine(h.ptr, _ptr(y), _ptr(topk_weights), _ptr(bias), _ptr(out), _stream(y.device)))
        return out

    if not async_with_compute_stream:
        return launch()
    return _overlapped(h, y.device, [y, topk_weights, bias, out], launch, previous_event)


def debug_e4m3_encode(q):
    """The fp8 dispatch kernel's float -> E4M3FN conversion on a float32 device tensor."""
    import torch

    if q.dtype != torch.float32 or not q.is_cuda or not q.is_contiguous():
        raise TypeError("q must be a contiguous float32 device tensor")
    out = torch.empty(q.shape, dtype=torch.uint8, device=q.device)
    _check(lib().ep_debug_e4m3_encode(_ptr(q), _ptr(out), q.numel(), _stream(q.device)))
    return out


def debug_copy(dst, src):
    """Calibration copy (ep_debug_copy) of src into dst: same-size contiguous device tensors,
    byte size a multiple of 1024."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n or not (src.is_cuda and dst.is_cuda):
        raise ValueError("dst and src must be device tensors of the same byte size")
    if not (src.is_contiguous() and dst.is_contiguous()) or src.device != dst.device:
        raise ValueError("dst and src must be contiguous and on one device")
    _check(lib().ep_debug_copy(_ptr(dst), _ptr(src), n, _stream(src.device)))
    return dst
