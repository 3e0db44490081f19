"""CPU oracle of the MoE dispatch/combine path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The library under
``combine_topk_idx_expert_amd`` never does, and nothing here imports it.

The arithmetic lives in ``oracle.c`` (plain single-threaded C, built with gcc
with FMA contraction off); this module only loads it with ctypes and marshals
numpy arrays.  See the header of ``oracle.c`` for the definitions it follows.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
against closed forms, brute force, library routines (numpy stable argsort,
torch float8/bfloat16 casts) and the values the pages print.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_HDR = os.path.join(_HERE, "oracle.h")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"]

OK, ERR_SHAPE, ERR_ROUTING = 0, -2, -3


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < max(
            os.path.getmtime(_SRC), os.path.getmtime(_HDR)):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", *CFLAGS, "-I", _HERE, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        # EP_ORACLE_LIB: load another build of oracle.c instead (the planted-mistake
        # builds of tests/test_oracle_mutants.py); nothing else sets it
        override = os.environ.get("EP_ORACLE_LIB")
        if override:
            path = override
        else:
            path = _LIB_PATH
            if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < max(
                    os.path.getmtime(_SRC), os.path.getmtime(_HDR)):
                build(force=True)
        L = ctypes.CDLL(path)
        P_ = ctypes.c_void_p
        i32, i64 = ctypes.c_int, ctypes.c_int64
        L.oracle_layout.argtypes = [i32] * 6 + [P_] * 14
        L.oracle_layout.restype = i32
        L.oracle_dispatch.argtypes = [i32] * 8 + [P_] * 7 + [i64, i64] + [P_] * 4
        L.oracle_dispatch.restype = i32
        L.oracle_dispatch_fixed.argtypes = [i32] * 8 + [P_] * 4 + [i64] + [P_] * 2 + [i64, i64] + [P_] * 5
        L.oracle_dispatch_fixed.restype = i32
        L.oracle_combine.argtypes = [i32] * 5 + [P_] * 5 + [i64, i64, P_]
        L.oracle_combine.restype = i32
        L.oracle_combine_fixed.argtypes = [i32] * 5 + [P_] * 2 + [i64] + [P_] * 2 + [i64, i64, P_]
        L.oracle_combine_fixed.restype = i32
        L.oracle_dispatch_general.argtypes = [i32] * 9 + [i64] + [P_] * 9 + [i64, i64] + [P_] * 5
        L.oracle_dispatch_general.restype = i32
        L.oracle_combine_general.argtypes = [i32] * 5 + [i64] + [P_] * 6 + [i64, i64, P_]
        L.oracle_combine_general.restype = i32
        L.oracle_combine_identity_bias.argtypes = [i32] * 3 + [P_] * 4 + [i64, i64, P_]
        L.oracle_combine_identity_bias.restype = i32
        L.oracle_combine_identity.argtypes = [i32] * 3 + [P_] * 3 + [i64, i64, P_]
        L.oracle_combine_identity.restype = i32
        L.oracle_quantize_row.argtypes = [P_, i32, P_, P_]
        L.oracle_quantize_row.restype = None
        L.oracle_quantize_row_ue8m0.argtypes = [P_, i32, P_, P_]
        L.oracle_quantize_row_ue8m0.restype = None
        L.oracle_quantize_rows.argtypes = [P_, i32, i64, i64, P_, P_]
        L.oracle_quantize_rows_ue8m0.argtypes = [P_, i32, i64, i64, P_, P_]
        L.oracle_quantize_rows_ue8m0.restype = None
        L.oracle_quantize_rows.restype = None
        for fn in ("oracle_e4m3_encode_array", "oracle_e4m3_decode_array", "oracle_bf16_round_array"):
            getattr(L, fn).argtypes = [P_, i64, P_]
            getattr(L, fn).restype = None
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_bf16_round.argtypes = [ctypes.c_float]
        L.oracle_bf16_round.restype = ctypes.c_uint16
        _lib = L
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


class OracleError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"oracle status {status}")
        self.status = status


@dataclass
class Layout:
    P: int
    S: int
    E: int
    K: int
    A: int
    symmetric: bool
    topk_idx: np.ndarray
    is_token_in_rank: np.ndarray  # [T, P] u8
    num_tokens_per_rank: np.ndarray  # [P, P] i32
    num_tokens_per_expert: np.ndarray  # [P, E] i32
    rank_prefix_matrix: np.ndarray  # [P, P] i32
    num_recv_tokens: np.ndarray  # [P] i32
    num_tokens_per_expert_total: np.ndarray  # [E] i32
    expert_offset: np.ndarray  # [P, E_l + 1] i64
    num_expanded: np.ndarray  # [P] i64
    window_row_base: np.ndarray  # [P + 1] i64
    dst_slot: np.ndarray  # [T, K] i32
    send_head: np.ndarray  # [T, P] i32
    recv_src_idx: np.ndarray  # [sum num_recv] i32
    recv_src_base: np.ndarray  # [P + 1] i64

    @property
    def T(self) -> int:
        return self.P * self.S

    @property
    def total_rows(self) -> int:
        return int(self.window_row_base[-1])


def layout(P: int, S: int, E: int, K: int, A: int, topk_idx: np.ndarray, symmetric: bool = False) -> Layout:
    T = P * S
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int64).reshape(T, K)
    if E % P != 0 or E < 1:
        raise OracleError(ERR_SHAPE)
    El = E // P
    out = dict(
        is_token_in_rank=np.zeros((T, P), np.uint8),
        num_tokens_per_rank=np.zeros((P, P), np.int32),
        num_tokens_per_expert=np.zeros((P, E), np.int32),
        rank_prefix_matrix=np.zeros((P, P), np.int32),
        num_recv_tokens=np.zeros(P, np.int32),
        num_tokens_per_expert_total=np.zeros(E, np.int32),
        expert_offset=np.zeros((P, El + 1), np.int64),
        num_expanded=np.zeros(P, np.int64),
        window_row_base=np.zeros(P + 1, np.int64),
        dst_slot=np.zeros((T, K), np.int32),
        send_head=np.zeros((T, P), np.int32),
        recv_src_idx=np.zeros(max(1, T * min(K, P)), np.int32),
        recv_src_base=np.zeros(P + 1, np.int64),
    )
    st = lib().oracle_layout(
        P, S, E, K, A, int(symmetric), _p(topk_idx),
        *[_p(out[k]) for k in ("is_token_in_rank", "num_tokens_per_rank", "num_tokens_per_expert",
                               "rank_prefix_matrix", "num_recv_tokens", "num_tokens_per_expert_total",
                               "expert_offset", "num_expanded", "window_row_base", "dst_slot",
                               "send_head", "recv_src_idx", "recv_src_base")])
    if st != OK:
        raise OracleError(st)
    out["recv_src_idx"] = out["recv_src_idx"][: int(out["recv_src_base"][-1])].copy()
    return Layout(P=P, S=S, E=E, K=K, A=A, symmetric=symmetric, topk_idx=topk_idx, **out)


def dispatch(lay: Layout, H: int, x: np.ndarray, topk_weights: np.ndarray | None, fp8: bool,
             zero_padding: bool, row_begin: int = 0, row_end: int | None = None,
             with_meta: bool = True, fill: int = 0):
    """Expanded rows [row_begin, row_end) -> (recv_x, recv_scales, recv_weights, recv_src_meta).

    Rows the method leaves untouched keep ``fill`` (payload) / zeros (metadata).
    Passing ``x=None`` computes the row metadata only (recv_x and recv_scales are None)."""
    if row_end is None:
        row_end = lay.total_rows
    n = row_end - row_begin
    payload = x is not None
    x = np.zeros((0,), np.uint16) if x is None else np.ascontiguousarray(x, dtype=np.uint16).reshape(lay.T, H)
    recv_x = np.full((n, H), fill, np.uint8 if fp8 else np.uint16) if payload else None
    recv_scales = np.zeros((n, H // 128), np.float32) if (fp8 and payload) else None
    recv_w = np.zeros(n, np.float32) if with_meta else None
    recv_meta = np.zeros((n, 2), np.int32) if with_meta else None
    w = None if topk_weights is None else np.ascontiguousarray(topk_weights, dtype=np.float32)
    assert w is not None or not with_meta, "row metadata needs topk_weights"
    st = lib().oracle_dispatch(
        lay.P, lay.S, lay.E, lay.K, H, lay.A, int(fp8), int(zero_padding), _p(lay.topk_idx),
        _p(lay.dst_slot), _p(lay.num_tokens_per_expert_total), _p(lay.expert_offset),
        _p(lay.window_row_base), _p(x), _p(w), row_begin, row_end, _p(recv_x), _p(recv_scales),
        _p(recv_w), _p(recv_meta))
    if st != OK:
        raise OracleError(st)
    return recv_x, recv_scales, recv_w, recv_meta


def dispatch_fixed(lay: Layout, H: int, capacity: int, x: np.ndarray | None,
                   topk_weights: np.ndarray | None, fp8: bool, zero_padding: bool, row_begin: int = 0,
                   row_end: int | None = None, with_meta: bool = True, fill: int = 0):
    """Fixed output length of ``capacity`` rows per window (``oracle_dispatch_fixed``):
    rows [row_begin, row_end) of the P * capacity output ->
    (recv_x, recv_scales, recv_weights, recv_src_meta, dropped_rows)."""
    if row_end is None:
        row_end = lay.P * capacity
    n = row_end - row_begin
    payload = x is not None
    x = np.zeros((0,), np.uint16) if x is None else np.ascontiguousarray(x, dtype=np.uint16).reshape(lay.T, H)
    recv_x = np.full((n, H), fill, np.uint8 if fp8 else np.uint16) if payload else None
    recv_scales = np.zeros((n, H // 128), np.float32) if (fp8 and payload) else None
    recv_w = np.zeros(n, np.float32) if with_meta else None
    recv_meta = np.zeros((n, 2), np.int32) if with_meta else None
    w = None if topk_weights is None else np.ascontiguousarray(topk_weights, dtype=np.float32)
    assert w is not None or not with_meta, "row metadata needs topk_weights"
    dropped = np.zeros(1, np.int64)
    st = lib().oracle_dispatch_fixed(
        lay.P, lay.S, lay.E, lay.K, H, lay.A, int(fp8), int(zero_padding), _p(lay.topk_idx),
        _p(lay.dst_slot), _p(lay.num_tokens_per_expert_total), _p(lay.expert_offset), capacity,
        _p(x), _p(w), row_begin, row_end, _p(recv_x), _p(recv_scales), _p(recv_w), _p(recv_meta),
        _p(dropped))
    if st != OK:
        raise OracleError(st)
    return recv_x, recv_scales, recv_w, recv_meta, int(dropped[0])


def dispatch_general(lay: Layout, H: int, *, fp8: bool, zero_padding: bool, topk_weights=None,
                     x: np.ndarray | None = None, x_codes: np.ndarray | None = None,
                     x_scales: np.ndarray | None = None, capacity: int = 0, scales_col_major: bool = False,
                     scales_ue8m0: bool = False, row_begin: int = 0, row_end: int | None = None,
                     with_meta: bool = True, fill: int = 0):
    """``oracle_dispatch_general``: exact (capacity 0) or fixed windows, row- or column-major
    scales, fused quantisation of x or pre-quantised (x_codes, x_scales).
    -> (recv_x, recv_scales, recv_weights, recv_src_meta, dropped_rows); recv_scales is
    [n, H/128] fp32, or [H/128, n] when scales_col_major, or UE8M0 bytes [n, H/32] (uint8)
    when scales_ue8m0."""
    assert not (scales_ue8m0 and scales_col_major)
    total = lay.P * capacity if capacity > 0 else lay.total_rows
    if row_end is None:
        row_end = total
    n = row_end - row_begin
    payload = x is not None or x_codes is not None
    x = np.zeros((0,), np.uint16) if x is None else np.ascontiguousarray(x, dtype=np.uint16).reshape(lay.T, H)
    xc = None if x_codes is None else np.ascontiguousarray(x_codes, dtype=np.uint8).reshape(lay.T, H)
    xs = None if x_scales is None else np.ascontiguousarray(x_scales, dtype=np.float32).reshape(lay.T, H // 128)
    recv_x = np.full((n, H), fill, np.uint8 if fp8 else np.uint16) if payload else None
    recv_scales = None
    if fp8 and payload and scales_ue8m0:  # exponent bytes start as `fill`, like the codes
        recv_scales = np.full((n, H // 32), fill, np.uint8)
    elif fp8 and payload:
        recv_scales = np.zeros((H // 128, n) if scales_col_major else (n, H // 128), np.float32)
    recv_w = np.zeros(n, np.float32) if with_meta else None
    recv_meta = np.zeros((n, 2), np.int32) if with_meta else None
    w = None if topk_weights is None else np.ascontiguousarray(topk_weights, dtype=np.float32)
    assert w is not None or not with_meta, "row metadata needs topk_weights"
    dropped = np.zeros(1, np.int64)
    st = lib().oracle_dispatch_general(
        lay.P, lay.S, lay.E, lay.K, H, lay.A, int(fp8), int(zero_padding),
        2 if scales_ue8m0 else int(scales_col_major), capacity,
        _p(lay.topk_idx), _p(lay.dst_slot), _p(lay.num_tokens_per_expert_total), _p(lay.expert_offset),
        _p(lay.window_row_base), _p(x), _p(xc), _p(xs), _p(w), row_begin, row_end, _p(recv_x),
        _p(recv_scales), _p(recv_w), _p(recv_meta), _p(dropped))
    if st != OK:
        raise OracleError(st)
    return recv_x, recv_scales, recv_w, recv_meta, int(dropped[0])


def combine_general(lay: Layout, H: int, y: np.ndarray, topk_weights: np.ndarray | None,
                    bias: np.ndarray | None = None, capacity: int = 0, tok_begin: int = 0,
                    tok_end: int | None = None) -> np.ndarray:
    """``oracle_combine_general``: exact or fixed windows, optional bf16 bias [T, H]."""
    if tok_end is None:
        tok_end = lay.T
    y = np.ascontiguousarray(y, dtype=np.uint16)
    out = np.zeros((tok_end - tok_begin, H), np.uint16)
    w = None if topk_weights is None else np.ascontiguousarray(topk_weights, dtype=np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.uint16).reshape(lay.T, H)
    st = lib().oracle_combine_general(lay.P, lay.S, lay.E, lay.K, H, capacity, _p(lay.topk_idx),
                                      _p(lay.dst_slot), _p(lay.window_row_base), _p(y), _p(w), _p(b),
                                      tok_begin, tok_end, _p(out))
    if st != OK:
        raise OracleError(st)
    return out


def combine_fixed(lay: Layout, H: int, capacity: int, y: np.ndarray, topk_weights: np.ndarray | None,
                  tok_begin: int = 0, tok_end: int | None = None) -> np.ndarray:
    """Combine over fixed-length windows (``oracle_combine_fixed``): y is [P * capacity, H]."""
    if tok_end is None:
        tok_end = lay.T
    y = np.ascontiguousarray(y, dtype=np.uint16)
    assert y.size >= lay.P * capacity * H
    out = np.zeros((tok_end - tok_begin, H), np.uint16)
    w = None if topk_weights is None else np.ascontiguousarray(topk_weights, dtype=np.float32)
    st = lib().oracle_combine_fixed(lay.P, lay.S, lay.E, lay.K, H, _p(lay.topk_idx), _p(lay.dst_slot),
                                    capacity, _p(y), _p(w), tok_begin, tok_end, _p(out))
    if st != OK:
        raise OracleError(st)
    return out


def combine(lay: Layout, H: int, y: np.ndarray, topk_weights: np.ndarray | None,
            tok_begin: int = 0, tok_end: int | None = None) -> np.ndarray:
    if tok_end is None:
        tok_end = lay.T
    y = np.ascontiguousarray(y, dtype=np.uint16)
    assert y.size >= lay.total_rows * H
    out = np.zeros((tok_end - tok_begin, H), np.uint16)
    w = None if topk_weights is None else np.ascontiguousarray(topk_weights, dtype=np.float32)
    st = lib().oracle_combine(lay.P, lay.S, lay.E, lay.K, H, _p(lay.topk_idx), _p(lay.dst_slot),
                              _p(lay.window_row_base), _p(y), _p(w), tok_begin, tok_end, _p(out))
    if st != OK:
        raise OracleError(st)
    return out


def combine_identity(K: int, H: int, fp8: bool, topk_idx: np.ndarray, x: np.ndarray,
                     topk_weights: np.ndarray | None, tok_begin: int, tok_end: int,
                     bias: np.ndarray | None = None) -> np.ndarray:
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int64)
    x = np.ascontiguousarray(x, dtype=np.uint16)
    out = np.zeros((tok_end - tok_begin, H), np.uint16)
    w = None if topk_weights is None else np.ascontiguousarray(topk_weights, dtype=np.float32)
    if bias is None:
        st = lib().oracle_combine_identity(K, H, int(fp8), _p(topk_idx), _p(x), _p(w), tok_begin, tok_end,
                                           _p(out))
    else:
        b = np.ascontiguousarray(bias, dtype=np.uint16)
        st = lib().oracle_combine_identity_bias(K, H, int(fp8), _p(topk_idx), _p(x), _p(w), _p(b), tok_begin,
                                                tok_end, _p(out))
    if st != OK:
        raise OracleError(st)
    return out


def quantize_row(x_row: np.ndarray):
    x_row = np.ascontiguousarray(x_row, dtype=np.uint16)
    H = x_row.size
    codes = np.zeros(H, np.uint8)
    scales = np.zeros(H // 128, np.float32)
    lib().oracle_quantize_row(_p(x_row), H, _p(codes), _p(scales))
    return codes, scales


def quantize_row_ue8m0(x_row: np.ndarray):
    """``oracle_quantize_row_ue8m0``: -> (codes [H] u8, exponent bytes [H/32] u8)."""
    x_row = np.ascontiguousarray(x_row, dtype=np.uint16)
    H = x_row.size
    codes = np.zeros(H, np.uint8)
    exps = np.zeros(H // 32, np.uint8)
    lib().oracle_quantize_row_ue8m0(_p(x_row), H, _p(codes), _p(exps))
    return codes, exps


def quantize_rows(x: np.ndarray, H: int, row_begin: int = 0, row_end: int | None = None):
    """``oracle_quantize_row`` on rows [row_begin, row_end) of x [T, H] -> (codes, scales)."""
    x = np.ascontiguousarray(x, dtype=np.uint16).reshape(-1, H)
    if row_end is None:
        row_end = x.shape[0]
    n = row_end - row_begin
    codes = np.zeros((n, H), np.uint8)
    scales = np.zeros((n, H // 128), np.float32)
    lib().oracle_quantize_rows(_p(x), H, row_begin, row_end, _p(codes), _p(scales))
    return codes, scales


def quantize_rows_ue8m0(x: np.ndarray, H: int, row_begin: int = 0, row_end: int | None = None):
    """``oracle_quantize_row_ue8m0`` on rows [row_begin, row_end) of x -> (codes, exponent bytes)."""
    x = np.ascontiguousarray(x, dtype=np.uint16).reshape(-1, H)
    if row_end is None:
        row_end = x.shape[0]
    n = row_end - row_begin
    codes = np.zeros((n, H), np.uint8)
    exps = np.zeros((n, H // 32), np.uint8)
    lib().oracle_quantize_rows_ue8m0(_p(x), H, row_begin, row_end, _p(codes), _p(exps))
    return codes, exps


def e4m3_encode(q: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.float32)
    out = np.zeros(q.shape, np.uint8)
    lib().oracle_e4m3_encode_array(_p(q), q.size, _p(out))
    return out


def e4m3_decode(c: np.ndarray) -> np.ndarray:
    c = np.ascontiguousarray(c, dtype=np.uint8)
    out = np.zeros(c.shape, np.float32)
    lib().oracle_e4m3_decode_array(_p(c), c.size, _p(out))
    return out


def bf16_round(f: np.ndarray) -> np.ndarray:
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.zeros(f.shape, np.uint16)
    lib().oracle_bf16_round_array(_p(f), f.size, _p(out))
    return out
