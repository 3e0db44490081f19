"""The C-ABI library loads and exports what include/ep_mi355x.h declares; host-side
validation rejects bad configs with the documented status codes before any device
work.  CPU only: nothing here launches a kernel."""

import ctypes
import os
import re

import pytest

import combine_topk_idx_expert_amd as ep
from combine_topk_idx_expert_amd._native import _Config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ep_mi355x.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ep_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ep.lib_path()):
        import combine_topk_idx_expert_amd.build as b

        b.build()
    return ep.lib()


def test_header_declares_the_five_entry_points():
    names = declared_functions()
    for fn in ("ep_get_layout", "ep_dispatch", "ep_dispatch_cached", "ep_combine", "ep_handle_free"):
        assert fn in names


def test_library_exports_every_declared_symbol(L):
    missing = [fn for fn in declared_functions() if not hasattr(L, fn)]
    assert not missing, missing
    assert L.ep_abi_version() == ep.EP_ABI_VERSION


def test_library_has_gfx950_code_object():
    data = open(ep.lib_path(), "rb").read()
    assert b"gfx950" in data


def _layout_status(L, cfg: _Config, topk_ptr=1):
    h = ctypes.c_void_p(123)
    rows = ctypes.c_int64(-1)
    st = L.ep_get_layout(ctypes.byref(cfg), ctypes.c_void_p(topk_ptr), None, ctypes.byref(h), ctypes.byref(rows))
    return st, h.value


GOOD = dict(num_ranks=8, num_tokens=4096, hidden=7168, num_topk=8, num_experts=256, expert_alignment=128, flags=0,
            num_worst_rows=0)


@pytest.mark.parametrize("change,status", [
    (dict(num_ranks=0), ep.Status.ERR_SHAPE),
    (dict(num_ranks=2000, num_experts=4000), ep.Status.ERR_SHAPE),
    (dict(num_tokens=-1), ep.Status.ERR_SHAPE),
    (dict(hidden=7170), ep.Status.ERR_SHAPE),
    (dict(hidden=0), ep.Status.ERR_SHAPE),
    (dict(num_topk=0), ep.Status.ERR_SHAPE),
    (dict(num_topk=33), ep.Status.ERR_SHAPE),
    (dict(num_experts=250), ep.Status.ERR_SHAPE),
    (dict(num_experts=4), ep.Status.ERR_SHAPE),
    (dict(num_experts=8192), ep.Status.ERR_SHAPE),
    (dict(expert_alignment=0), ep.Status.ERR_SHAPE),
    (dict(flags=8), ep.Status.ERR_SHAPE),
    (dict(num_ranks=8, num_tokens=1 << 28), ep.Status.ERR_OVERFLOW),       # T*K >= 2^31
    (dict(num_ranks=1024, num_experts=1024, num_topk=1, num_tokens=1 << 21), ep.Status.ERR_OVERFLOW),  # T*P
    (dict(num_tokens=(1 << 31) // 64 - 100, num_topk=8), ep.Status.ERR_OVERFLOW),
    (dict(num_worst_rows=-1), ep.Status.ERR_SHAPE),
    (dict(num_worst_rows=4096, flags=1), ep.Status.ERR_SHAPE),       # fixed windows are not symmetric ones
    (dict(num_worst_rows=(1 << 31) // 8), ep.Status.ERR_OVERFLOW),    # P * W >= 2^31
])
def test_validation_errors(L, change, status):
    cfg = _Config(**{**GOOD, **change})
    st, h = _layout_status(L, cfg)
    assert st == status, (st, L.ep_last_error())
    assert h is None  # *out is cleared on error
    assert L.ep_last_error()


def test_null_arguments(L):
    cfg = _Config(**GOOD)
    st, _ = _layout_status(L, cfg, topk_ptr=0)
    assert st == ep.Status.ERR_NULL
    assert L.ep_get_layout(None, None, None, ctypes.byref(ctypes.c_void_p()), None) == ep.Status.ERR_NULL
    assert L.ep_get_layout(ctypes.byref(cfg), ctypes.c_void_p(1), None, None, None) == ep.Status.ERR_NULL
    for call in (lambda: L.ep_dispatch(None, 0, None, None, None, None, None, None, None),
                 lambda: L.ep_dispatch_cached(None, 0, None, None, None, None),
                 lambda: L.ep_combine(None, None, None, None, None, None),
                 lambda: L.ep_dispatch_prequant(None, 0, None, None, None, None, None, None, None, None),
                 lambda: L.ep_dispatch_prequant_cached(None, 0, None, None, None, None, None),
                 lambda: L.ep_relayout(None, None, None, None),
                 lambda: L.ep_handle_counts(None, None, None, None),
                 lambda: L.ep_handle_status(None, ctypes.byref(ctypes.c_uint32()), None),
                 lambda: L.ep_handle_status(None, None, None)):
        assert call() == ep.Status.ERR_NULL
    L.ep_handle_free(None)  # no-op


def test_python_binding_rejects_host_tensors():
    import torch

    cfg = ep.Config(P=2, S=4, H=64, K=2, E=4, A=1)
    with pytest.raises(ValueError):
        ep.get_layout(cfg, torch.zeros((8, 2), dtype=torch.int64))
    with pytest.raises((TypeError, ValueError)):
        ep.get_layout(cfg, torch.zeros((8, 2), dtype=torch.int32))
    with pytest.raises(TypeError):
        ep.get_layout(cfg, [[0, 1]] * 8)


def test_c_program_links_against_the_library():
    """tests/c_abi/roundtrip (built by __graft_entry__.build()) drives the C ABI from C++
    alone; on the CPU check that it resolves the library and the oracle."""
    import subprocess

    exe = os.path.join(ROOT, "tests", "c_abi", "roundtrip")
    if not os.path.exists(exe):
        import importlib.util

        spec = importlib.util.spec_from_file_location("c_abi_build", os.path.join(ROOT, "tests", "c_abi", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    out = subprocess.run(["ldd", exe], capture_output=True, text=True, check=True).stdout
    for lib in ("libep_mi355x.so", "liboracle.so"):
        line = next(ln for ln in out.splitlines() if lib in ln)
        assert "not found" not in line, line


def test_buffer_size_hint_needs_no_gpu(L):
    """ep_buffer_size_hint on the host: row bounds from the closed forms, bytes per tensor,
    the total a multiple of 2 MiB; validation as for ep_get_layout."""
    P, S, H, K, E, A = 8, 4096, 7168, 8, 256, 128
    T = P * S
    hb = ep.buffer_size_hint(ep.Config(P, S, H, K, E, A))
    assert hb["max_rows"] == T * K + E * (A - 1)
    assert hb["recv_x_bytes"] == hb["max_rows"] * H * 2 and hb["recv_scales_bytes"] == 0
    assert hb["recv_weights_bytes"] == hb["max_rows"] * 4 and hb["recv_src_meta_bytes"] == hb["max_rows"] * 8
    assert hb["combine_out_bytes"] == T * H * 2
    # the handle holds at least its [T, P] send_head, [T, K] dst_slot / dst_row and [T, P] is_token_in_rank
    assert hb["handle_bytes"] >= T * P * 4 + 2 * T * K * 4 + T * P
    parts = sum(v for k, v in hb.items() if k.endswith("_bytes") and k != "total_bytes")
    assert hb["total_bytes"] % (2 << 20) == 0 and parts <= hb["total_bytes"] < parts + (2 << 20)
    h8 = ep.buffer_size_hint(ep.Config(P, S, H, K, E, A), fp8=True)
    assert h8["recv_x_bytes"] == hb["max_rows"] * H and h8["recv_scales_bytes"] == hb["max_rows"] * (H // 32)
    assert ep.buffer_size_hint(ep.Config(P, S, H, K, E, A), scales_ue8m0=True)["recv_scales_bytes"] == \
        h8["recv_scales_bytes"]
    hf = ep.buffer_size_hint(ep.Config(P, S, H, K, E, A, num_worst_rows=35840))
    assert hf["max_rows"] == P * 35840
    hs = ep.buffer_size_hint(ep.Config(P, S, H, K, E, A, symmetric_windows=True))
    assert hs["max_rows"] == P * (T * K + (E // P) * (A - 1))
    with pytest.raises(ep.EpError):
        ep.buffer_size_hint(ep.Config(P, S, H, K, E + 1, A))
    with pytest.raises(ep.EpError):
        ep.buffer_size_hint(ep.Config(P, S, 136, K, E, A), fp8=True)


def test_debug_timing_needs_the_timing_build(L):
    """ep_debug_timing reads the device timing slots only in a library built with
    EP_DEVICE_TIMING=1; the ordinary build refuses with EP_ERR_SHAPE and says why, before any
    HIP call."""
    import numpy as np

    slots = np.zeros(8, np.uint64)
    assert L.ep_debug_timing(slots.ctypes.data, 8) == -2  # EP_ERR_SHAPE
    assert b"EP_DEVICE_TIMING" in L.ep_last_error()
    assert not slots.any()
