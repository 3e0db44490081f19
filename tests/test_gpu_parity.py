"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bar (from the method's statement of correctness): layout arrays, indices and
dispatched payload (bf16 copies, E4M3 codes and fp32 scales) bit-exact; combine
within 1 bf16 ulp of the oracle.  The kernels use the oracle's arithmetic order
(non-fused multiply then add, slots in order), so combine is also checked for
bit-exact equality, which is stronger than the bar.

Small and medium shapes (several chunks, ragged tails, edge cases) are compared
element by element.  Full-size workloads compare the whole layout, all row
metadata and, for payload, every token (bf16 and fp8 rows against the oracle's
per-token encoding) and sampled or full combine outputs.
"""

import sys

import numpy as np
import pytest
import torch

import combine_topk_idx_expert_amd as ep
import oracle
import synth
from synth import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

LAYOUT_TENSORS = ["is_token_in_rank", "num_tokens_per_rank", "num_tokens_per_expert", "rank_prefix_matrix",
                  "num_recv_tokens", "num_tokens_per_expert_total", "expert_offset", "num_expanded",
                  "window_row_base", "dst_slot", "send_head", "recv_src_idx", "recv_src_base"]


def say(*a):
    print("[gpu-parity]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def dev_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def layout_both(w, topk, symmetric=False):
    say("layout", w.name, "symmetric" if symmetric else "packed")
    lay = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk, symmetric)
    h = ep.get_layout(ep.Config(w.P, w.S, w.H, w.K, w.E, w.A, symmetric), torch.from_numpy(topk).to(DEV))
    torch.cuda.synchronize()
    return lay, h


def check_layout(lay, h):
    assert h.total_rows == lay.total_rows
    for name in LAYOUT_TENSORS:
        got = h.tensor(name).cpu().numpy()
        exp = getattr(lay, name).reshape(-1)
        np.testing.assert_array_equal(got, exp.astype(got.dtype), err_msg=name)
    El = lay.E // lay.P
    rank = np.where(lay.topk_idx >= 0, lay.topk_idx // El, 0)
    exp_row = np.where(lay.dst_slot >= 0, lay.window_row_base[rank] + lay.dst_slot, -1)
    np.testing.assert_array_equal(h.tensor("dst_row").cpu().numpy(), exp_row.reshape(-1))
    ne, nr, wb = h.counts()
    np.testing.assert_array_equal(ne, lay.num_expanded)
    np.testing.assert_array_equal(nr, lay.num_recv_tokens)
    np.testing.assert_array_equal(wb, lay.window_row_base)


def routing_with_holes(w, seed=0):
    """Workload routing plus unused (-1) slots and duplicate experts inside tokens."""
    topk = synth.gen_routing(w).copy()
    rng = np.random.default_rng(seed)
    T = w.T
    if T and w.K > 1:
        topk[rng.random(T) < 0.1, w.K - 1] = -1
        dup = rng.random(T) < 0.05
        topk[dup, 1] = topk[dup, 0]
        topk[rng.random(T) < 0.02] = -1  # tokens routed nowhere
    return topk


# --------------------------------------------------------------------------
# small and medium shapes, element-wise
# --------------------------------------------------------------------------

D = synth.CONFIGS
SMALL = [
    D["tiny-p4-s64-e16-k2-h512"],
    synth.scaled(D["dsv3-bf16-p8-s4096-e256-k8-h7168"], S=300),                 # ragged last chunk
    synth.scaled(D["ep128-zipf-p128-s1024-e256-k6-h7168"], S=70, H=1024),      # empty experts, P=128
    synth.scaled(D["ep32-group-fwdbwd-p32-s8192-e256-k8-h4096"], S=130),
    wl.Workload("p1-s100-e8-k3", 1, 100, 8, 3, 256, 4, True, "uniform", seed=3),
    wl.Workload("el1-p16-s64-e16-k4", 16, 64, 16, 4, 128, 1, True, "uniform", seed=4),
    wl.Workload("k1-p4-s65-e32-k1", 4, 65, 32, 1, 136, 8, True, "uniform", seed=5),  # H not a multiple of 64
    wl.Workload("s1-p8-s1-e64-k8", 8, 1, 64, 8, 512, 16, True, "uniform", seed=6),
    wl.Workload("big-e-p64-s33-e1024-k16", 64, 33, 1024, 16, 256, 32, True, "uniform", seed=7),
    wl.Workload("k32-p2-s70-e64-k32", 2, 70, 64, 32, 128, 3, True, "uniform", seed=8),
    wl.Workload("h8-p4-s40-e16-k3", 4, 40, 16, 3, 8, 4, True, "uniform", seed=9),  # smallest hidden: one chunk a row
    wl.Workload("h24-p3-s50-e24-k12", 3, 50, 24, 12, 24, 2, True, "uniform", seed=10),  # K > 8: register combine, 3 chunks
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
@pytest.mark.parametrize("holes", [False, True], ids=["plain", "holes"])
def test_layout_small(w, holes):
    topk = routing_with_holes(w, 11) if holes else synth.gen_routing(w)
    lay, h = layout_both(w, topk)
    check_layout(lay, h)
    h.free()


# Shapes of at most 16 chunks of 64 tokens, whose layout runs as one workgroup, and one of
# 17 chunks just past that limit (four kernels).
# Decode-sized batches.  The one-workgroup layout runs for at most 16 chunks whose fullest
# chunk holds at most 256 slots (tokens x top-k); the others take the four-kernel path.
SMALL_BATCH = [
    wl.Workload("sb-p4-s64-e16-k2", 4, 64, 16, 2, 512, 16, True, "uniform", seed=31),       # 4 chunks, one WG
    wl.Workload("sb-p16-s64-e64-k4", 16, 64, 64, 4, 256, 8, True, "uniform", seed=37),      # 16 chunks, one WG
    wl.Workload("sb-p8-s100-e256-k2", 8, 100, 256, 2, 1024, 128, True, "uniform", seed=38),  # 16 ragged, one WG
    wl.Workload("sb-p16-s64-e64-k6", 16, 64, 64, 6, 256, 8, True, "uniform", seed=32),      # 16 chunks, 4 kernels
    wl.Workload("sb-p8-s100-e256-k8", 8, 100, 256, 8, 1024, 128, True, "uniform", seed=33),  # 16 ragged, 4 kernels
    wl.Workload("sb-p1-s1-e8-k3", 1, 1, 8, 3, 128, 4, True, "uniform", seed=34),            # 1 token
    wl.Workload("sb-p2-s7-e512-k4", 2, 7, 512, 4, 256, 3, True, "uniform", seed=35),         # many experts
    wl.Workload("sb-p17-s64-e34-k3", 17, 64, 34, 3, 256, 2, True, "uniform", seed=36),      # 17 chunks
]


@pytest.mark.parametrize("w", SMALL_BATCH, ids=lambda w: w.name)
@pytest.mark.parametrize("mode", ["exact", "fixed", "symmetric"])
def test_small_batch_layout(w, mode):
    """Decode-sized batches: every handle array against the oracle with holes, duplicate
    experts and tokens routed nowhere (fixed windows: also an out-of-range id, reported as a
    status, and a window that truncates), then dispatch and combine against the oracle."""
    topk = routing_with_holes(w, 41)
    if mode == "fixed":
        topk = topk.copy()
        topk[0, 0] = w.E + 3  # out of range: counted as unused, reported as a status
    lay = oracle.layout(w.P, w.S, w.E, w.K, w.A, np.where(topk >= w.E, -1, topk), mode == "symmetric")
    x = synth.gen_bf16_rows(w.seed, wl.STREAM_X, w.T, w.H)
    wt = synth.gen_weights(w)
    xd, wd = dev_bf16(x), torch.from_numpy(wt).to(DEV)
    if mode == "fixed":
        W = max(1, int(np.median(lay.num_expanded)))  # some windows truncate
        h = ep.get_layout(ep.Config(w.P, w.S, w.H, w.K, w.E, w.A, num_worst_rows=W), torch.from_numpy(topk).to(DEV))
        torch.cuda.synchronize()
        check_fixed_layout(lay, h, W)
        flags, dropped = h.status()
        exp_drop = int(np.maximum(lay.num_expanded - W, 0).sum())
        assert flags & ep.STATUS_ROUTING and dropped == exp_drop
        assert bool(flags & ep.STATUS_TRUNCATED) == (exp_drop > 0)
        rx, _, rw, rm = ep.dispatch(h, xd, wd, zero_padding=True)
        torch.cuda.synchronize()
        ox, _, ow, om, _ = oracle.dispatch_general(lay, w.H, fp8=False, zero_padding=True, topk_weights=wt, x=x,
                                                   capacity=W)
        np.testing.assert_array_equal(host_u16(rx), ox)
        np.testing.assert_array_equal(rm.cpu().numpy(), om)
        out = ep.combine(h, rx, wd)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host_u16(out), oracle.combine_general(lay, w.H, ox, wt, capacity=W))
    else:
        h = ep.get_layout(ep.Config(w.P, w.S, w.H, w.K, w.E, w.A, mode == "symmetric"), torch.from_numpy(topk).to(DEV))
        torch.cuda.synchronize()
        check_layout(lay, h)
        rx, _, rw, rm = ep.dispatch(h, xd, wd, zero_padding=True)
        torch.cuda.synchronize()
        ox, _, ow, om = oracle.dispatch(lay, w.H, x, wt, False, True)
        got = host_u16(rx)
        in_win = np.zeros(len(om), bool)  # symmetric windows leave the rows past num_expanded alone
        for d_ in range(w.P):
            in_win[lay.window_row_base[d_]:lay.window_row_base[d_] + lay.num_expanded[d_]] = True
        np.testing.assert_array_equal(got[in_win], ox[in_win])
        np.testing.assert_array_equal(rm.cpu().numpy()[in_win], om[in_win])
        np.testing.assert_array_equal(rw.cpu().numpy()[in_win].view(np.uint32), ow[in_win].view(np.uint32))
        out = ep.combine(h, rx, wd)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host_u16(out), oracle.combine(lay, w.H, got, wt))
    # relayout of the same handle with another routing
    topk2 = routing_with_holes(w, 42)
    lay2 = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk2, mode == "symmetric")
    ep.relayout(h, torch.from_numpy(topk2).to(DEV))
    torch.cuda.synchronize()
    if mode == "fixed":
        check_fixed_layout(lay2, h, W)
    else:
        check_layout(lay2, h)
    h.free()


def test_small_batch_empty():
    """No tokens at all (S = 0) through the one-workgroup layout: zero counts, no rows."""
    w = wl.Workload("sb-empty", 4, 0, 16, 2, 128, 4, True, "uniform")
    lay, h = layout_both(w, np.zeros((0, 2), np.int64))
    check_layout(lay, h)
    assert h.total_rows == 0
    h.free()


def test_layout_symmetric_windows():
    w = SMALL[2]
    topk = synth.gen_routing(w)
    lay, h = layout_both(w, topk, symmetric=True)
    check_layout(lay, h)
    h.free()


def test_layout_empty_and_errors():
    w = wl.Workload("empty", 4, 0, 16, 2, 64, 4, True, "uniform")
    lay, h = layout_both(w, np.zeros((0, 2), np.int64))
    check_layout(lay, h)
    assert h.total_rows == 0
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    rx, _, rw, meta = ep.dispatch(h, x, torch.zeros((0, 2), dtype=torch.float32, device=DEV), zero_padding=True)
    out = ep.combine(h, rx)
    assert out.shape == (0, 64)
    h.free()
    w = D["tiny-p4-s64-e16-k2-h512"]
    for bad in (16, -2, 1 << 33):
        topk = synth.gen_routing(w).copy()
        topk[77, 1] = bad
        say("routing error case", bad)
        with pytest.raises(ep.EpError) as ei:
            ep.get_layout(ep.Config(w.P, w.S, w.H, w.K, w.E, w.A), torch.from_numpy(topk).to(DEV))
        assert ei.value.status == ep.Status.ERR_ROUTING


def test_relayout_reuses_handle():
    w = SMALL[1]
    a = synth.gen_routing(w)
    b = synth.gen_routing(synth.scaled(w, seed=9))
    lay_a, h = layout_both(w, a)
    check_layout(lay_a, h)
    ep.relayout(h, torch.from_numpy(b).to(DEV))
    check_layout(oracle.layout(w.P, w.S, w.E, w.K, w.A, b), h)
    h.check(ep.Config(w.P, w.S, w.H, w.K, w.E, w.A))
    with pytest.raises(ep.EpError) as ei:
        h.check(ep.Config(w.P, w.S, w.H, w.K, w.E, w.A * 2))
    assert ei.value.status == ep.Status.ERR_HANDLE_MISMATCH
    h.free()



SEQ = wl.Workload("seq-p8-s100-e32-k4", 8, 100, 32, 4, 256, 8, True, "uniform", seed=11)


def _routing_sequence(w):
    """Routings of very different shapes on one config, ordered so that state left
    over from one layout (padding lists, counters, status flags) would show in the next."""
    T, K, E = w.T, w.K, w.E
    one = np.full((T, K), -1, np.int64)
    one[:, 0] = 0  # every token to expert 0: one full window, all others empty
    none = np.full((T, K), -1, np.int64)  # no valid slot at all: zero expanded rows
    dup = np.full((T, K), E - 1, np.int64)  # K copies of the last expert in every token
    return [("uniform", synth.gen_routing(w)), ("one-expert", one),
            ("uniform-2", synth.gen_routing(synth.scaled(w, seed=w.seed + 77))), ("none", none),
            ("duplicates", dup), ("holes", routing_with_holes(w, 21)), ("uniform-again", synth.gen_routing(w))]


@pytest.mark.parametrize("fixed", [False, True], ids=["exact", "fixed"])
def test_relayout_sequence_leaves_no_stale_state(fixed):
    """One handle, relaid out for each routing in turn; after every relayout the layout,
    a fresh dispatch (bf16 then fp8, zero padding) and a combine match the oracle.  In
    fixed mode W = 512 rows per window: the one-expert and duplicate routings overflow
    a window and report truncation, and the routings after them must clear it."""
    w = SEQ
    x = synth.gen_bf16_rows(w.seed, wl.STREAM_X, w.T, w.H)
    wt = synth.gen_weights(w)
    xd, wd = dev_bf16(x), torch.from_numpy(wt).to(DEV)
    seq = _routing_sequence(w)
    W = 512 if fixed else 0
    h = ep.get_layout(ep.Config(w.P, w.S, w.H, w.K, w.E, w.A, num_worst_rows=W), torch.from_numpy(seq[0][1]).to(DEV))
    for i, (name, topk) in enumerate(seq):
        say("relayout sequence", "fixed" if fixed else "exact", i, name)
        ep.relayout(h, torch.from_numpy(topk).to(DEV))
        torch.cuda.synchronize()
        lay = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk)
        if fixed:
            check_fixed_layout(lay, h, W)
            exp_drop = int(np.maximum(lay.num_expanded - W, 0).sum())
            assert h.status() == (ep.STATUS_TRUNCATED if exp_drop else 0, exp_drop), name
            R = w.P * W
        else:
            check_layout(lay, h)
            assert h.status() == (0, 0)
            R = lay.total_rows
        fp8 = i % 2 == 1
        rx, sc, rw, rm = ep.dispatch(h, xd, wd, fp8=fp8, zero_padding=True)
        torch.cuda.synchronize()
        if fixed:
            ox, osc, ow, om, _ = oracle.dispatch_fixed(lay, w.H, W, x, wt, fp8, True)
        else:
            ox, osc, ow, om = oracle.dispatch(lay, w.H, x, wt, fp8, True)
        assert rx.shape[0] == R
        np.testing.assert_array_equal(rx.cpu().numpy() if fp8 else host_u16(rx), ox, err_msg=name)
        np.testing.assert_array_equal(rw.cpu().numpy().view(np.uint32), ow.view(np.uint32), err_msg=name)
        np.testing.assert_array_equal(rm.cpu().numpy(), om, err_msg=name)
        if fp8:
            np.testing.assert_array_equal(sc.cpu().numpy().view(np.uint32), osc.view(np.uint32), err_msg=name)
        y = synth.gen_expert_out(w, R)
        out = ep.combine(h, dev_bf16(y), wd)
        torch.cuda.synchronize()
        exp = oracle.combine_fixed(lay, w.H, W, y, wt) if fixed else oracle.combine(lay, w.H, y, wt)
        np.testing.assert_array_equal(host_u16(out), exp, err_msg=name)
    h.free()


DISPATCH_CASES = [w for w in SMALL if w.T > 0]


def _fp8_needs_hidden_multiple_of_128(w, W):
    """fp8 output has one scale per 128 channels, so a hidden size that is not a multiple of
    128 must be refused (EP_ERR_SHAPE) before anything is launched, fresh and cached."""
    topk_d = torch.from_numpy(synth.gen_routing(w)).to(DEV)
    h = ep.get_layout(ep.Config(w.P, w.S, w.H, w.K, w.E, w.A, num_worst_rows=W), topk_d)
    xd = dev_bf16(synth.gen_bf16_rows(w.seed, wl.STREAM_X, w.T, w.H))
    wd = torch.from_numpy(synth.gen_weights(w)).to(DEV)
    for call in (lambda: ep.dispatch(h, xd, wd, fp8=True), lambda: ep.dispatch_cached(h, xd, fp8=True)):
        with pytest.raises(ep.EpError) as ei:
            call()
        assert ei.value.status == ep.Status.ERR_SHAPE
    h.free()


@pytest.mark.parametrize("w", DISPATCH_CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_dispatch_and_combine_small(w, fp8):
    if fp8 and w.H % 128:
        _fp8_needs_hidden_multiple_of_128(w, 0)
        return
    topk = routing_with_holes(w, 12)
    x = synth.gen_bf16_rows(w.seed, wl.STREAM_X, w.T, w.H)
    x[:3, :128] = 0  # an all-zero 128-channel block (amax == 0)
    x[1, 5] = 0x8000  # -0.0 inside it
    wt = synth.gen_weights(w)
    lay, h = layout_both(w, topk)
    check_layout(lay, h)
    R = lay.total_rows
    xd, wd = dev_bf16(x), torch.from_numpy(wt).to(DEV)
    sentinel = 0x7F if fp8 else 0xFFFF
    pad = None
    for zp in (False, True):
        say("dispatch", w.name, "fp8" if fp8 else "bf16", "zero_padding" if zp else "no_padding")
        rx = torch.full((R, w.H), 0x7F if fp8 else -1, dtype=torch.uint8 if fp8 else torch.int16, device=DEV)
        if not fp8:
            rx = rx.view(torch.bfloat16)
        sc = torch.full((R, w.H // 128), float("nan"), dtype=torch.float32, device=DEV) if fp8 else None
        rw = torch.full((R,), float("nan"), dtype=torch.float32, device=DEV)
        rm = torch.full((R, 2), 77, dtype=torch.int32, device=DEV)
        ep.dispatch(h, xd, wd, fp8=fp8, zero_padding=zp, out=(rx, sc, rw, rm))
        torch.cuda.synchronize()
        ox, osc, ow, om = oracle.dispatch(lay, w.H, x, wt, fp8, zp, fill=sentinel)
        got_x = rx.cpu().numpy() if fp8 else host_u16(rx)
        np.testing.assert_array_equal(got_x, ox)
        np.testing.assert_array_equal(rw.cpu().numpy().view(np.uint32), ow.view(np.uint32))
        np.testing.assert_array_equal(rm.cpu().numpy(), om)
        pad = om[:, 0] < 0
        if fp8:
            gs = sc.cpu().numpy()
            rows = slice(None) if zp else ~pad
            np.testing.assert_array_equal(gs[rows].view(np.uint32), osc[rows].view(np.uint32))
            if not zp:
                assert np.all(np.isnan(gs[pad]))  # untouched
        # cached dispatch reproduces the fresh payload
        say("dispatch_cached", w.name)
        cx = torch.full_like(rx, 0) if zp else rx.clone()
        csc = torch.zeros_like(sc) if (fp8 and zp) else (sc.clone() if fp8 else None)
        ep.dispatch_cached(h, xd, fp8=fp8, zero_padding=zp, out=(cx, csc))
        torch.cuda.synchronize()
        assert torch.equal(cx.view(torch.uint8), rx.view(torch.uint8))
        if fp8:
            np.testing.assert_array_equal(csc.cpu().numpy().view(np.uint32)[~pad], osc.view(np.uint32)[~pad])

    # combine of arbitrary expert outputs (bf16) with and without weights
    y = synth.gen_expert_out(w, R)
    yd = dev_bf16(y)
    for weights in (wt, None):
        say("combine", w.name, "weighted" if weights is not None else "unit")
        out = ep.combine(h, yd, None if weights is None else wd)
        torch.cuda.synchronize()
        exp = oracle.combine(lay, w.H, y, weights)
        got = host_u16(out)
        assert ulp_diff(got, exp).max() <= 1  # the stated bar
        np.testing.assert_array_equal(got, exp)  # same arithmetic order: exact
    h.free()


def ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    def key(hh):
        hh = hh.astype(np.int32)
        return np.where(hh & 0x8000, 0x8000 - (hh & 0x7FFF), 0x8000 + (hh & 0x7FFF))
    return np.abs(key(a) - key(b))


# --------------------------------------------------------------------------
# full-size workloads
# --------------------------------------------------------------------------

def gather_rows(t: torch.Tensor, rows: np.ndarray) -> torch.Tensor:
    return t.index_select(0, torch.from_numpy(rows.astype(np.int64)).to(DEV))


def dequant_identity(rx: torch.Tensor, sc: torch.Tensor) -> torch.Tensor:
    """Identity expert on fp8 rows: bf16(decode(code) * scale)."""
    f = rx.view(torch.float8_e4m3fn).to(torch.float32)
    return (f * sc.repeat_interleave(128, dim=1)).to(torch.bfloat16)


def oracle_threads() -> int:
    """Host threads for the oracle at full size: the affinity mask, at most 16 (one GPU's
    share of the box).  ctypes releases the GIL during each oracle call, so a thread pool
    over row or token ranges runs them in parallel."""
    import os

    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_over_ranges(fn, n: int, out: np.ndarray, pieces_per_thread: int = 4):
    """out[a:b] = fn(a, b) over contiguous ranges of [0, n), in a thread pool."""
    from concurrent.futures import ThreadPoolExecutor

    nt = oracle_threads()
    step = max(1, -(-n // (nt * pieces_per_thread)))

    def run(a):
        b = min(n, a + step)
        out[a:b] = fn(a, b)

    with ThreadPoolExecutor(nt) as ex:
        list(ex.map(run, range(0, n, step)))
    return out


def quantize_all(x: np.ndarray, H: int):
    """The oracle's per-token fp8 encoding of every row of x (threaded over row ranges)."""
    T = x.shape[0]
    codes = np.empty((T, H), np.uint8)
    scales = np.empty((T, H // 128), np.float32)
    oracle_over_ranges(lambda a, b: oracle.quantize_rows(x, H, a, b)[0], T, codes)
    oracle_over_ranges(lambda a, b: oracle.quantize_rows(x, H, a, b)[1], T, scales)
    return codes, scales


def combine_identity_all(K, H, fp8, topk, x, wt, bias=None):
    """The oracle's combine(identity(dispatch(x))) for every token (threaded over token ranges)."""
    T = topk.shape[0]
    out = np.empty((T, H), np.uint16)
    return oracle_over_ranges(lambda a, b: oracle.combine_identity(K, H, fp8, topk, x, wt, a, b, bias=bias), T, out)


def check_payload_rows(rx, x_dev, lay, fp8, codes=None, scales=None, sc=None, chunk=4096):
    """Every valid slot's row equals its token's row (bf16) or the oracle's codes and scales
    (fp8), compared on the device: the oracle's per-token codes and scales are uploaded and
    gathered by token next to the rows gathered by slot."""
    El = lay.E // lay.P
    codes_d = torch.from_numpy(codes).to(DEV) if fp8 else None
    scales_d = torch.from_numpy(scales.view(np.int32)).to(DEV) if fp8 else None
    for u0 in range(0, lay.T, chunk):
        u1 = min(lay.T, u0 + chunk)
        tk = lay.topk_idx[u0:u1]
        for j in range(lay.K):
            m = tk[:, j] >= 0
            if not m.any():
                continue
            us = np.arange(u0, u1)[m]
            rows = lay.window_row_base[tk[m, j] // El] + lay.dst_slot[u0:u1][m, j]
            got = gather_rows(rx, rows)
            if not fp8:
                exp = gather_rows(x_dev, us)
                assert torch.equal(got.view(torch.int16), exp.view(torch.int16)), (u0, j)
            else:
                assert torch.equal(got, gather_rows(codes_d, us)), f"codes {u0} {j}"
                assert torch.equal(gather_rows(sc, rows).view(torch.int32), gather_rows(scales_d, us)), \
                    f"scales {u0} {j}"


FULL = [D[n] for n in wl.CONFIG_ORDER]


@pytest.mark.parametrize("w", FULL, ids=lambda w: w.name)
def test_full_size(w):
    topk = synth.gen_routing(w)
    lay, h = layout_both(w, topk)
    check_layout(lay, h)
    hint = ep.buffer_size_hint(ep.Config(w.P, w.S, w.H, w.K, w.E, w.A), fp8=w.fp8)
    assert h.total_rows <= hint["max_rows"]
    # a second handle's device arena is no more than the hint counts (up to allocation
    # granularity; small arenas may come from memory the runtime already holds): the routing is
    # on the device before the free memory is read, so only ep_get_layout allocates
    topk_d = torch.from_numpy(topk).to(DEV)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    h2 = ep.get_layout(ep.Config(w.P, w.S, w.H, w.K, w.E, w.A), topk_d)
    used = free0 - torch.cuda.mem_get_info()[0]
    h2.free()
    del topk_d
    assert used <= hint["handle_bytes"] + (8 << 20), (used, hint["handle_bytes"])
    R = lay.total_rows
    say("generate x", w.name)
    x = synth.gen_x(w)
    wt = synth.gen_weights(w)
    xd, wd = dev_bf16(x), torch.from_numpy(wt).to(DEV)
    fp8 = w.fp8
    say("dispatch", w.name, "fp8" if fp8 else "bf16", "rows", R)
    rx, sc, rw, rm = ep.dispatch(h, xd, wd, fp8=fp8, zero_padding=w.zero_padding)
    torch.cuda.synchronize()
    _, _, ow, om = oracle.dispatch(lay, w.H, None, wt, fp8, w.zero_padding)
    np.testing.assert_array_equal(rm.cpu().numpy(), om)
    np.testing.assert_array_equal(rw.cpu().numpy().view(np.uint32), ow.view(np.uint32))
    pad = np.flatnonzero(om[:, 0] < 0)
    if w.zero_padding and len(pad):
        assert int(gather_rows(rx.view(torch.uint8) if fp8 else rx.view(torch.int16), pad).abs().max()) == 0
        if fp8:
            assert float(gather_rows(sc, pad).abs().max()) == 0.0
    codes = scales = None
    if fp8:
        say("oracle quantize", w.name)
        codes, scales = quantize_all(x, w.H)
    say("payload rows", w.name)
    check_payload_rows(rx, xd, lay, fp8, codes, scales, sc)

    # combine(identity(dispatch(x))) against the oracle's composition, every token
    say("combine", w.name, "tokens", w.T, "oracle threads", oracle_threads())
    y = dequant_identity(rx, sc) if fp8 else rx
    out = ep.combine(h, y, wd)
    torch.cuda.synchronize()
    got = host_u16(out)
    exp = combine_identity_all(w.K, w.H, fp8, topk, x, wt)
    assert ulp_diff(got, exp).max() <= 1
    np.testing.assert_array_equal(got, exp)
    del y, out, got, exp

    if w.cached_iters:
        # every cached iteration's payload against the oracle's encoding of its own x
        say("cached iterations", w.cached_iters)
        cx, csc = torch.empty_like(rx), (torch.empty_like(sc) if fp8 else None)
        pad_d = torch.from_numpy(pad.astype(np.int64)).to(DEV)
        for it in range(1, w.cached_iters + 1):
            xi = synth.workloads.gen_cached_x(w, it)
            xid = dev_bf16(xi)
            cx.fill_(0x5A if fp8 else 1)  # stale bytes must not survive
            if fp8:
                csc.fill_(7.0)
            ep.dispatch_cached(h, xid, fp8=fp8, zero_padding=w.zero_padding, out=(cx, csc))
            torch.cuda.synchronize()
            ci, si = quantize_all(xi, w.H) if fp8 else (None, None)
            check_payload_rows(cx, xid, lay, fp8, ci, si, csc)
            if w.zero_padding and len(pad):
                assert int(cx.view(torch.uint8).index_select(0, pad_d).max()) == 0, it
                if fp8:
                    assert float(csc.index_select(0, pad_d).abs().max()) == 0.0, it
            del xid

    if w.backward:
        say("backward", w.name)
        g = synth.gen_grad_out(w)
        gd = dev_bf16(g)
        gy, _ = ep.dispatch_cached(h, gd, zero_padding=w.zero_padding)
        check_payload_rows(gy, gd, lay, False)
        gx = ep.combine(h, gy, wd)
        torch.cuda.synchronize()
        say("backward combine, every token")
        got = host_u16(gx)
        exp = combine_identity_all(w.K, w.H, False, topk, g, wt)
        assert ulp_diff(got, exp).max() <= 1
        np.testing.assert_array_equal(got, exp)
        del gy, gx, got, exp
    h.free()
    del rx, sc, rw, rm, xd
    torch.cuda.empty_cache()


def test_device_e4m3_conversion_matches_oracle():
    """The device fp32 -> E4M3FN conversion used by fp8 dispatch, on every 53rd fp32 pattern of
    magnitude <= 464 plus +-3 ulp around every rounding midpoint, both signs, against the oracle."""
    pats = np.arange(0, 0x43E80001, 53, dtype=np.uint32)
    codes = np.arange(0x7F, dtype=np.uint8)
    vals = np.sort(oracle.e4m3_decode(codes).astype(np.float64))
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32).view(np.uint32)
    near = (mids[:, None].astype(np.int64) + np.arange(-3, 4)[None, :]).ravel().astype(np.uint32)
    q = np.concatenate([pats, near]).view(np.float32)
    q = np.concatenate([q, -q])
    say("device e4m3 conversion on", q.size, "values")
    got = ep.debug_e4m3_encode(torch.from_numpy(q).to(DEV)).cpu().numpy()
    np.testing.assert_array_equal(got, oracle.e4m3_encode(q))


# --------------------------------------------------------------------------
# fixed output length (num_worst_rows): no read-back, tail rows, truncation
# --------------------------------------------------------------------------

def fixed_layout_both(w, topk, W):
    say("fixed layout", w.name, "W", W)
    lay = oracle.layout(w.P, w.S, w.E, w.K, w.A, np.where(topk >= w.E, -1, np.where(topk < -1, -1, topk)))
    h = ep.get_layout(ep.Config(w.P, w.S, w.H, w.K, w.E, w.A, num_worst_rows=W), torch.from_numpy(topk).to(DEV))
    assert h.total_rows == w.P * W  # known without waiting
    torch.cuda.synchronize()
    return lay, h


def check_fixed_layout(lay, h, W):
    for name in LAYOUT_TENSORS:
        if name == "window_row_base":
            continue
        got = h.tensor(name).cpu().numpy()
        exp = getattr(lay, name).reshape(-1)
        np.testing.assert_array_equal(got, exp.astype(got.dtype), err_msg=name)
    np.testing.assert_array_equal(h.tensor("window_row_base").cpu().numpy(), np.arange(lay.P + 1) * W)
    El = lay.E // lay.P
    rank = np.where(lay.topk_idx >= 0, lay.topk_idx // El, 0)
    exp_row = np.where((lay.dst_slot >= 0) & (lay.dst_slot < W), rank * W + lay.dst_slot, -1)
    np.testing.assert_array_equal(h.tensor("dst_row").cpu().numpy(), exp_row.reshape(-1))
    ne, nr, wb = h.counts()
    np.testing.assert_array_equal(ne, lay.num_expanded)
    np.testing.assert_array_equal(nr, lay.num_recv_tokens)
    np.testing.assert_array_equal(wb, np.arange(lay.P + 1) * W)


FIXED_CASES = [SMALL[0], SMALL[1], SMALL[2], SMALL[4], SMALL[6], SMALL[7], SMALL[10]]


@pytest.mark.parametrize("w", FIXED_CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("fit", ["roomy", "tight", "one"])
@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_fixed_windows_small(w, fit, fp8):
    if fp8 and w.H % 128:
        _fp8_needs_hidden_multiple_of_128(w, {"roomy": 4096, "tight": 8, "one": 1}[fit])
        return
    topk = routing_with_holes(w, 13)
    ne = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk).num_expanded
    W = {"roomy": int(ne.max()) + 37, "tight": max(1, int(np.median(ne))), "one": 1}[fit]
    x = synth.gen_bf16_rows(w.seed, wl.STREAM_X, w.T, w.H)
    x[:3, :128] = 0
    wt = synth.gen_weights(w)
    lay, h = fixed_layout_both(w, topk, W)
    check_fixed_layout(lay, h, W)
    flags, dropped = h.status()
    exp_drop = int(np.maximum(lay.num_expanded - W, 0).sum())
    assert dropped == exp_drop and flags == (ep.STATUS_TRUNCATED if exp_drop else 0)
    R = w.P * W
    xd, wd = dev_bf16(x), torch.from_numpy(wt).to(DEV)
    for zp in (False, True):
        say("fixed dispatch", w.name, fit, "fp8" if fp8 else "bf16", "zp" if zp else "no zp")
        rx = torch.full((R, w.H), 0x7F if fp8 else -1, dtype=torch.uint8 if fp8 else torch.int16, device=DEV)
        if not fp8:
            rx = rx.view(torch.bfloat16)
        sc = torch.full((R, w.H // 128), float("nan"), dtype=torch.float32, device=DEV) if fp8 else None
        rw = torch.full((R,), float("nan"), dtype=torch.float32, device=DEV)
        rm = torch.full((R, 2), 77, dtype=torch.int32, device=DEV)
        ep.dispatch(h, xd, wd, fp8=fp8, zero_padding=zp, out=(rx, sc, rw, rm))
        torch.cuda.synchronize()
        ox, osc, ow, om, odrop = oracle.dispatch_fixed(lay, w.H, W, x, wt, fp8, zp, fill=0x7F if fp8 else 0xFFFF)
        assert odrop == dropped
        np.testing.assert_array_equal(rx.cpu().numpy() if fp8 else host_u16(rx), ox)
        np.testing.assert_array_equal(rw.cpu().numpy().view(np.uint32), ow.view(np.uint32))
        np.testing.assert_array_equal(rm.cpu().numpy(), om)
        tail = np.arange(R) % W >= np.repeat(lay.num_expanded, W)
        touched = (om[:, 0] >= 0) | zp | tail  # rows whose payload and scales dispatch writes
        if fp8:
            gs = sc.cpu().numpy()
            np.testing.assert_array_equal(gs[touched].view(np.uint32), osc[touched].view(np.uint32))
            assert np.all(np.isnan(gs[~touched]))
        say("fixed dispatch_cached", w.name, fit)
        tmask = torch.from_numpy(touched).to(DEV)
        cx = rx.clone()
        cx.view(torch.uint8)[tmask] = 0x55
        csc = None
        if fp8:
            csc = sc.clone()
            csc[tmask] = 3.0
        ep.dispatch_cached(h, xd, fp8=fp8, zero_padding=zp, out=(cx, csc))
        torch.cuda.synchronize()
        assert torch.equal(cx.view(torch.uint8), rx.view(torch.uint8))
        if fp8:
            assert torch.equal(csc.view(torch.int32), sc.view(torch.int32))
    y = synth.gen_expert_out(w, R)
    say("fixed combine", w.name, fit)
    out = ep.combine(h, dev_bf16(y), wd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_u16(out), oracle.combine_fixed(lay, w.H, W, y, wt))
    # relayout in fixed mode: new routing, same W
    b = synth.gen_routing(synth.scaled(w, seed=w.seed + 50))
    ep.relayout(h, torch.from_numpy(b).to(DEV))
    assert h.total_rows == R
    check_fixed_layout(oracle.layout(w.P, w.S, w.E, w.K, w.A, b), h, W)
    h.free()


def test_fixed_windows_routing_error_is_a_status():
    w = D["tiny-p4-s64-e16-k2-h512"]
    topk = synth.gen_routing(w).copy()
    topk[5, 0], topk[77, 1] = 16, -7
    lay, h = fixed_layout_both(w, topk, 200)
    check_fixed_layout(lay, h, 200)  # the bad slots count as unused
    flags, dropped = h.status()
    assert flags & ep.STATUS_ROUTING and dropped == 0
    h.free()


def test_fixed_windows_empty_tokens():
    w = wl.Workload("empty-fixed", 4, 0, 16, 2, 128, 4, True, "uniform")
    lay, h = fixed_layout_both(w, np.zeros((0, 2), np.int64), 5)
    x = torch.zeros((0, 128), dtype=torch.bfloat16, device=DEV)
    rx, sc, rw, rm = ep.dispatch(h, x, torch.zeros((0, 2), dtype=torch.float32, device=DEV), fp8=True)
    torch.cuda.synchronize()
    assert rx.shape == (20, 128) and int(rx.max()) == 0
    assert float(sc.abs().max()) == 0 and float(rw.abs().max()) == 0 and bool((rm == -1).all())
    assert h.status() == (0, 0)
    h.free()


@pytest.mark.parametrize("name,fit", [("dsv3-bf16-p8-s4096-e256-k8-h7168", "bucket"),
                                      ("ep128-zipf-p128-s1024-e256-k6-h7168", "truncate")])
def test_fixed_windows_full_size(name, fit):
    """Full-size fixed windows: a safe bucket (no truncation) and, under Zipf skew, a capacity
    the hot windows overflow.  Metadata against the oracle, every published slot's payload,
    tails zero, and combine(identity) against the oracle with the dropped slots unused."""
    w = D[name]
    topk = synth.gen_routing(w)
    ne = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk).num_expanded
    W = int(-(-int(ne.max()) // 1024) * 1024) if fit == "bucket" else 8192
    lay, h = fixed_layout_both(w, topk, W)
    check_fixed_layout(lay, h, W)
    flags, dropped = h.status()
    exp_drop = int(np.maximum(lay.num_expanded - W, 0).sum())
    assert dropped == exp_drop and (exp_drop > 0) == (fit == "truncate")
    x = synth.gen_x(w)
    wt = synth.gen_weights(w)
    xd, wd = dev_bf16(x), torch.from_numpy(wt).to(DEV)
    say("fixed dispatch full", name, "W", W, "dropped", dropped)
    rx, _, rw, rm = ep.dispatch(h, xd, wd, zero_padding=w.zero_padding)
    torch.cuda.synchronize()
    _, _, ow, om, _ = oracle.dispatch_fixed(lay, w.H, W, None, wt, False, w.zero_padding)
    np.testing.assert_array_equal(rm.cpu().numpy(), om)
    np.testing.assert_array_equal(rw.cpu().numpy().view(np.uint32), ow.view(np.uint32))
    tail = np.flatnonzero(np.arange(w.P * W) % W >= np.repeat(lay.num_expanded, W))
    if len(tail):
        assert int(gather_rows(rx.view(torch.int16), tail).abs().max()) == 0
    kept = np.where((lay.dst_slot >= 0) & (lay.dst_slot < W), lay.topk_idx, -1)
    import dataclasses
    lay_w = dataclasses.replace(lay, topk_idx=kept, window_row_base=np.arange(w.P + 1, dtype=np.int64) * W)
    check_payload_rows(rx, xd, lay_w, False)
    toks = np.arange(0, w.T, 8)
    say("fixed combine full", name, "tokens", len(toks))
    out = ep.combine(h, rx, wd)
    torch.cuda.synchronize()
    got = host_u16(gather_rows(out, toks))
    exp = np.concatenate([oracle.combine_identity(w.K, w.H, False, kept, x, wt, u, u + 1) for u in toks])
    np.testing.assert_array_equal(got, exp)
    h.free()
    del rx, rw, rm, out, xd
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------
# API variants: column-major scales, pre-quantised fp8 input, combine bias
# --------------------------------------------------------------------------

VARIANT_CASES = [SMALL[0], SMALL[1], SMALL[2], SMALL[4], SMALL[7]]


def _dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


@pytest.mark.parametrize("w", VARIANT_CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("mode", ["exact", "fixed"])
def test_variants_small(w, mode):
    topk = routing_with_holes(w, 14)
    lay = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk)
    W = max(1, int(np.median(lay.num_expanded))) if mode == "fixed" else 0
    cfg = ep.Config(w.P, w.S, w.H, w.K, w.E, w.A, num_worst_rows=W)
    say("variants", w.name, mode, "W", W)
    h = ep.get_layout(cfg, torch.from_numpy(topk).to(DEV))
    R = h.total_rows
    x = synth.gen_bf16_rows(w.seed, wl.STREAM_X, w.T, w.H)
    wt = synth.gen_weights(w)
    xd, wd = dev_bf16(x), torch.from_numpy(wt).to(DEV)
    rng = np.random.default_rng(15)
    codes = rng.integers(0, 256, (w.T, w.H), dtype=np.uint8)
    scales = rng.standard_normal((w.T, w.H // 128)).astype(np.float32)
    nb = w.H // 128
    for src in ("fused", "prequant"):
        for cm in (False, True):
            for zp in (False, True):
                say("variant dispatch", w.name, mode, src, "col-major" if cm else "row-major", "zp" if zp else "")
                xin = xd if src == "fused" else (_dev_u8(codes), torch.from_numpy(scales).to(DEV))
                rx = torch.full((R, w.H), 0x7F, dtype=torch.uint8, device=DEV)
                sc = torch.full((nb, R) if cm else (R, nb), float("nan"), dtype=torch.float32, device=DEV)
                rw = torch.full((R,), float("nan"), dtype=torch.float32, device=DEV)
                rm = torch.full((R, 2), 77, dtype=torch.int32, device=DEV)
                ep.dispatch(h, xin, wd, fp8=True, zero_padding=zp, scales_col_major=cm, out=(rx, sc, rw, rm))
                torch.cuda.synchronize()
                kw = dict(x=x) if src == "fused" else dict(x_codes=codes, x_scales=scales)
                ox, osc, ow, om, _ = oracle.dispatch_general(lay, w.H, fp8=True, zero_padding=zp, topk_weights=wt,
                                                             capacity=W, scales_col_major=cm, fill=0x7F, **kw)
                np.testing.assert_array_equal(rx.cpu().numpy(), ox)
                np.testing.assert_array_equal(rm.cpu().numpy(), om)
                np.testing.assert_array_equal(rw.cpu().numpy().view(np.uint32), ow.view(np.uint32))
                tail = (np.arange(R) % W >= np.repeat(lay.num_expanded, W)) if W else np.zeros(R, bool)
                touched = (om[:, 0] >= 0) | zp | tail
                gs = sc.cpu().numpy()
                gs_rows = gs.T if cm else gs
                os_rows = osc.T if cm else osc
                np.testing.assert_array_equal(gs_rows[touched].view(np.uint32), os_rows[touched].view(np.uint32))
                assert np.all(np.isnan(gs_rows[~touched]))
                # cached dispatch of the same input reproduces payload and scales
                tmask = torch.from_numpy(touched).to(DEV)
                cx = rx.clone()
                cx[tmask] = 0x55
                csc = sc.clone()
                (csc.T if cm else csc)[tmask] = 3.0
                ep.dispatch_cached(h, xin, fp8=True, zero_padding=zp, scales_col_major=cm, out=(cx, csc))
                torch.cuda.synchronize()
                assert torch.equal(cx, rx)
                assert torch.equal(csc.view(torch.int32), sc.view(torch.int32))
    # combine with a bias, with and without weights
    y = synth.gen_expert_out(w, R)
    bias = synth.gen_bf16_rows(w.seed, wl.STREAM_GRAD_OUT, w.T, w.H)
    for weights in (wt, None):
        say("combine bias", w.name, mode, "weighted" if weights is not None else "unit")
        out = ep.combine(h, dev_bf16(y), None if weights is None else wd, bias=dev_bf16(bias))
        torch.cuda.synchronize()
        exp = oracle.combine_general(lay, w.H, y, weights, bias=bias, capacity=W)
        np.testing.assert_array_equal(host_u16(out), exp)
    h.free()


def test_variants_full_size():
    """DSv3 shapes: pre-quantised fp8 input with column-major scales, and combine with a
    bias (the shared-expert output in the pages' usage), against the oracle."""
    w = D["dsv3-fp8-p8-s4096-e256-k8-h7168"]
    topk = synth.gen_routing(w)
    lay, h = layout_both(w, topk)
    R = lay.total_rows
    x = synth.gen_x(w)
    wt = synth.gen_weights(w)
    xd, wd = dev_bf16(x), torch.from_numpy(wt).to(DEV)
    say("oracle quantize", w.name)
    codes, scales = quantize_all(x, w.H)
    say("prequant dispatch col-major", w.name)
    rx, sc, rw, rm = ep.dispatch(h, (_dev_u8(codes), torch.from_numpy(scales).to(DEV)), wd, zero_padding=True,
                                 scales_col_major=True)
    torch.cuda.synchronize()
    assert sc.shape == (w.H // 128, R)
    _, _, ow, om, _ = oracle.dispatch_general(lay, w.H, fp8=True, zero_padding=True, topk_weights=wt)
    np.testing.assert_array_equal(rm.cpu().numpy(), om)
    check_payload_rows(rx, None, lay, True, codes, scales, sc.t())
    fx, fsc, _, _ = ep.dispatch(h, xd, wd, fp8=True, zero_padding=True, scales_col_major=True)
    assert torch.equal(fx, rx) and torch.equal(fsc.view(torch.int32), sc.view(torch.int32))
    del rx, sc, fx, fsc
    say("combine with bias", w.name)
    y, _, _, _ = ep.dispatch(h, xd, wd, zero_padding=True)
    bias = synth.gen_grad_out(w)
    out = ep.combine(h, y, wd, bias=dev_bf16(bias))
    torch.cuda.synchronize()
    toks = np.arange(0, w.T, 4)
    got = host_u16(gather_rows(out, toks))
    exp = np.concatenate([oracle.combine_identity(w.K, w.H, False, topk, x, wt, u, u + 1, bias=bias)
                          for u in toks])
    np.testing.assert_array_equal(got, exp)
    h.free()
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------
# overlap API: calls on the communication stream, ordered by events
# --------------------------------------------------------------------------

@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("mode", ["exact", "fixed"])
def test_async_with_compute_stream_matches_sync(fp8, mode):
    """dispatch / cached dispatch / combine issued with async_with_compute_stream=True while a
    matmul runs on the compute stream give the same bytes as the synchronous calls; the input
    is produced on the compute stream right before the call, so the result also shows that the
    communication stream waited for it."""
    w = SMALL[1]
    topk = routing_with_holes(w, 16)
    lay = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk)
    W = int(lay.num_expanded.max()) if mode == "fixed" else 0
    h = ep.get_layout(ep.Config(w.P, w.S, w.H, w.K, w.E, w.A, num_worst_rows=W), torch.from_numpy(topk).to(DEV))
    x = synth.gen_bf16_rows(w.seed, wl.STREAM_X, w.T, w.H)
    wt = synth.gen_weights(w)
    xd, wd = dev_bf16(x), torch.from_numpy(wt).to(DEV)
    ref = ep.dispatch(h, xd, wd, fp8=fp8, zero_padding=True)
    ref_c = ep.dispatch_cached(h, xd, fp8=fp8, zero_padding=True)
    y = dev_bf16(synth.gen_expert_out(w, h.total_rows))
    bias = dev_bf16(synth.gen_bf16_rows(w.seed, wl.STREAM_GRAD_OUT, w.T, w.H))
    ref_out = ep.combine(h, y, wd, bias=bias)
    torch.cuda.synchronize()
    ox, osc, ow, om, dropped = oracle.dispatch_general(lay, w.H, fp8=fp8, zero_padding=True, topk_weights=wt, x=x,
                                                       capacity=W)
    assert dropped == 0
    oout = oracle.combine_general(lay, w.H, host_u16(y), wt, bias=host_u16(bias), capacity=W)
    a = torch.randn((2048, 2048), device=DEV)
    for it in range(3):
        say("async", mode, "fp8" if fp8 else "bf16", "iteration", it)
        x2 = xd * 1  # produced on the compute stream just before the call
        pending = ep.dispatch(h, x2, wd, fp8=fp8, zero_padding=True, async_with_compute_stream=True)
        busy = a @ a  # compute-stream work in between
        got = pending.wait()
        pc = ep.dispatch_cached(h, x2, fp8=fp8, zero_padding=True, async_with_compute_stream=True)
        got_c = pc.wait()
        po = ep.combine(h, y * 1, wd, bias=bias, async_with_compute_stream=True)
        busy = busy @ a
        out = po.wait()
        torch.cuda.synchronize()
        for r, g in zip(ref, got):
            if r is not None:
                assert torch.equal(r.view(torch.uint8), g.view(torch.uint8))
        for r, g in zip(ref_c, got_c):
            if r is not None:
                assert torch.equal(r.view(torch.uint8), g.view(torch.uint8))
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
        # and every async output against the oracle itself
        np.testing.assert_array_equal(got[0].cpu().numpy() if fp8 else host_u16(got[0]), ox)
        np.testing.assert_array_equal(got_c[0].cpu().numpy() if fp8 else host_u16(got_c[0]), ox)
        if fp8:
            np.testing.assert_array_equal(got[1].cpu().numpy().view(np.uint32), osc.view(np.uint32))
            np.testing.assert_array_equal(got_c[1].cpu().numpy().view(np.uint32), osc.view(np.uint32))
        np.testing.assert_array_equal(got[2].cpu().numpy().view(np.uint32), ow.view(np.uint32))
        np.testing.assert_array_equal(got[3].cpu().numpy(), om)
        np.testing.assert_array_equal(host_u16(out), oout)
    assert torch.isfinite(busy).any()
    h.free()


# --------------------------------------------------------------------------
# the build's limits
# --------------------------------------------------------------------------

@pytest.mark.parametrize("S,A", [(4, 1), (1, 8)])
def test_maximum_ranks_experts_topk(S, A):
    """1024 ranks, 4096 experts and top-32 at once (EP_MAX_RANKS, EP_MAX_EXPERTS, EP_MAX_TOPK),
    with unused slots and duplicate experts: layout, fresh dispatch and combine against the
    oracle.  A device whose workgroups cannot hold the rank kernel's LDS gets EP_ERR_SHAPE."""
    w = wl.Workload(f"max-p1024-s{S}-e4096-k32", 1024, S, 4096, 32, 128, A, True, "uniform", seed=21)
    topk = routing_with_holes(w, 17)
    lay = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk)
    say("maximum config", w.name)
    try:
        h = ep.get_layout(ep.Config(w.P, w.S, w.H, w.K, w.E, w.A), torch.from_numpy(topk).to(DEV))
    except ep.EpError as err:
        assert err.status == ep.Status.ERR_SHAPE and "LDS" in str(err)
        pytest.skip(f"device LDS per workgroup too small for this config: {err}")
    torch.cuda.synchronize()
    check_layout(lay, h)
    x = synth.gen_bf16_rows(w.seed, wl.STREAM_X, w.T, w.H)
    wt = synth.gen_weights(w)
    xd, wd = dev_bf16(x), torch.from_numpy(wt).to(DEV)
    for fp8 in (False, True):
        rx, sc, rw, rm = ep.dispatch(h, xd, wd, fp8=fp8, zero_padding=True)
        torch.cuda.synchronize()
        ox, osc, ow, om = oracle.dispatch(lay, w.H, x, wt, fp8, True)
        np.testing.assert_array_equal(rx.cpu().numpy() if fp8 else host_u16(rx), ox)
        np.testing.assert_array_equal(rm.cpu().numpy(), om)
        np.testing.assert_array_equal(rw.cpu().numpy().view(np.uint32), ow.view(np.uint32))
        if fp8:
            np.testing.assert_array_equal(sc.cpu().numpy().view(np.uint32), osc.view(np.uint32))
    y = synth.gen_expert_out(w, h.total_rows)
    out = ep.combine(h, dev_bf16(y), wd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_u16(out), oracle.combine(lay, w.H, y, wt))
    h.free()


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_symmetric_windows_dispatch_and_combine(fp8):
    """Symmetric windows (every window max_d num_expanded rows): the kernels map packed row
    positions to window rows by a search over the window bases; rows past a window's
    num_expanded stay untouched.  Then a relayout to another routing on the same handle."""
    w = SMALL[2]  # 128 ranks, Zipf: very uneven windows
    topk = routing_with_holes(w, 18)
    lay, h = layout_both(w, topk, symmetric=True)
    check_layout(lay, h)
    x = synth.gen_bf16_rows(w.seed, wl.STREAM_X, w.T, w.H)
    wt = synth.gen_weights(w)
    xd, wd = dev_bf16(x), torch.from_numpy(wt).to(DEV)
    for it, tk in enumerate((topk, synth.gen_routing(synth.scaled(w, seed=77)))):
        if it:
            ep.relayout(h, torch.from_numpy(tk).to(DEV))
            lay = oracle.layout(w.P, w.S, w.E, w.K, w.A, tk, True)
            check_layout(lay, h)
        R = h.total_rows
        say("symmetric dispatch", "fp8" if fp8 else "bf16", "layout", it, "rows", R)
        rx = torch.full((R, w.H), 0x7F if fp8 else -1, dtype=torch.uint8 if fp8 else torch.int16, device=DEV)
        if not fp8:
            rx = rx.view(torch.bfloat16)
        sc = torch.full((R, w.H // 128), float("nan"), dtype=torch.float32, device=DEV) if fp8 else None
        rw = torch.full((R,), float("nan"), dtype=torch.float32, device=DEV)
        rm = torch.full((R, 2), 77, dtype=torch.int32, device=DEV)
        ep.dispatch(h, xd, wd, fp8=fp8, zero_padding=True, out=(rx, sc, rw, rm))
        torch.cuda.synchronize()
        ox, osc, ow, om = oracle.dispatch(lay, w.H, x, wt, fp8, True, fill=0x7F if fp8 else 0xFFFF)
        np.testing.assert_array_equal(rx.cpu().numpy() if fp8 else host_u16(rx), ox)
        # rows past num_expanded (window tails) are not written: meta stays at its fill there
        used = np.zeros(R, bool)
        for d in range(w.P):
            b = int(lay.window_row_base[d])
            used[b:b + int(lay.num_expanded[d])] = True
        np.testing.assert_array_equal(rm.cpu().numpy()[used], om[used])
        assert np.all(rm.cpu().numpy()[~used] == 77)
        np.testing.assert_array_equal(rw.cpu().numpy().view(np.uint32)[used], ow.view(np.uint32)[used])
        if fp8:
            np.testing.assert_array_equal(sc.cpu().numpy()[used].view(np.uint32), osc[used].view(np.uint32))
        y = synth.gen_expert_out(w, R)
        out = ep.combine(h, dev_bf16(y), wd)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host_u16(out), oracle.combine(lay, w.H, y, wt))
    h.free()



def test_symmetric_windows_fp8_variants():
    """Symmetric windows with the fp8 variants: fused quantisation or pre-quantised input,
    row- or column-major scales, with and without zero padding, fresh then cached.  The
    column-major scales pass maps packed rows to window rows by its own search over the
    window bases; rows past each window's num_expanded must stay untouched."""
    w = SMALL[2]  # 128 ranks, Zipf: very uneven windows
    topk = routing_with_holes(w, 23)
    lay, h = layout_both(w, topk, symmetric=True)
    check_layout(lay, h)
    R, nb = h.total_rows, w.H // 128
    x = synth.gen_bf16_rows(w.seed, wl.STREAM_X, w.T, w.H)
    wt = synth.gen_weights(w)
    xd, wd = dev_bf16(x), torch.from_numpy(wt).to(DEV)
    rng = np.random.default_rng(24)
    codes = rng.integers(0, 256, (w.T, w.H), dtype=np.uint8)
    scales = rng.standard_normal((w.T, nb)).astype(np.float32)
    used = np.zeros(R, bool)
    for d in range(w.P):
        b = int(lay.window_row_base[d])
        used[b:b + int(lay.num_expanded[d])] = True
    for src in ("fused", "prequant"):
        xin = xd if src == "fused" else (_dev_u8(codes), torch.from_numpy(scales).to(DEV))
        kw = dict(x=x) if src == "fused" else dict(x_codes=codes, x_scales=scales)
        for cm in (False, True):
            for zp in (False, True):
                say("symmetric fp8 variant", src, "col-major" if cm else "row-major", "zp" if zp else "")
                rx = torch.full((R, w.H), 0x7F, dtype=torch.uint8, device=DEV)
                sc = torch.full((nb, R) if cm else (R, nb), float("nan"), dtype=torch.float32, device=DEV)
                rw = torch.full((R,), float("nan"), dtype=torch.float32, device=DEV)
                rm = torch.full((R, 2), 77, dtype=torch.int32, device=DEV)
                ep.dispatch(h, xin, wd, fp8=True, zero_padding=zp, scales_col_major=cm, out=(rx, sc, rw, rm))
                torch.cuda.synchronize()
                ox, osc, ow, om, _ = oracle.dispatch_general(lay, w.H, fp8=True, zero_padding=zp, topk_weights=wt,
                                                             scales_col_major=cm, fill=0x7F, **kw)
                np.testing.assert_array_equal(rx.cpu().numpy(), ox)
                gm = rm.cpu().numpy()
                np.testing.assert_array_equal(gm[used], om[used])
                assert np.all(gm[~used] == 77)
                np.testing.assert_array_equal(rw.cpu().numpy().view(np.uint32)[used], ow.view(np.uint32)[used])
                written = used & ((om[:, 0] >= 0) | zp)  # rows whose scales dispatch writes
                gs = sc.cpu().numpy()
                gs_rows, os_rows = (gs.T, osc.T) if cm else (gs, osc)
                np.testing.assert_array_equal(gs_rows[written].view(np.uint32), os_rows[written].view(np.uint32))
                assert np.all(np.isnan(gs_rows[~written]))
                # cached dispatch of the same input reproduces payload and scales
                cx = rx.clone()
                wmask = torch.from_numpy(written).to(DEV)
                cx[wmask] = 0x55
                csc = sc.clone()
                (csc.T if cm else csc)[wmask] = 3.0
                ep.dispatch_cached(h, xin, fp8=True, zero_padding=zp, scales_col_major=cm, out=(cx, csc))
                torch.cuda.synchronize()
                assert torch.equal(cx, rx)
                assert torch.equal(csc.view(torch.int32), sc.view(torch.int32))
    h.free()



def test_two_handles_on_two_streams():
    """Calls are re-entrant across distinct handles: two handles of different shapes (an fp8
    dispatch with column-major scales on one, a bf16 dispatch on the other, then a combine
    on each) enqueued interleaved on two streams with nothing ordering them; each result
    must match the oracle."""
    wa = SMALL[1]                                                             # P=8, E=256, H=7168
    wb = wl.Workload("two-handles-b", 16, 96, 64, 4, 512, 8, True, "uniform", seed=31)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    runs = []
    for w, stream, fp8 in ((wa, s1, True), (wb, s2, False)):
        topk = routing_with_holes(w, 32)
        lay = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk)
        x = synth.gen_bf16_rows(w.seed, wl.STREAM_X, w.T, w.H)
        wt = synth.gen_weights(w)
        y = synth.gen_expert_out(w, lay.total_rows)
        with torch.cuda.stream(stream):
            h = ep.get_layout(ep.Config(w.P, w.S, w.H, w.K, w.E, w.A), torch.from_numpy(topk).to(DEV))
        torch.cuda.synchronize()
        runs.append(dict(w=w, s=stream, fp8=fp8, lay=lay, h=h, x=x, wt=wt, y=y, xd=dev_bf16(x),
                         wd=torch.from_numpy(wt).to(DEV), yd=dev_bf16(y)))
    torch.cuda.synchronize()
    for step in ("dispatch", "combine"):
        for r in runs:  # interleaved: a's call, then b's, each on its own stream
            with torch.cuda.stream(r["s"]):
                if step == "dispatch":
                    r["out"] = ep.dispatch(r["h"], r["xd"], r["wd"], fp8=r["fp8"], zero_padding=True,
                                           scales_col_major=r["fp8"])
                else:
                    r["comb"] = ep.combine(r["h"], r["yd"], r["wd"])
    torch.cuda.synchronize()
    for r in runs:
        w, lay = r["w"], r["lay"]
        say("two handles", w.name, "fp8" if r["fp8"] else "bf16")
        ox, osc, ow, om, _ = oracle.dispatch_general(lay, w.H, fp8=r["fp8"], zero_padding=True, topk_weights=r["wt"],
                                                     x=r["x"], scales_col_major=r["fp8"])
        rx, sc, rw, rm = r["out"]
        np.testing.assert_array_equal(rx.cpu().numpy() if r["fp8"] else host_u16(rx), ox)
        np.testing.assert_array_equal(rm.cpu().numpy(), om)
        np.testing.assert_array_equal(rw.cpu().numpy().view(np.uint32), ow.view(np.uint32))
        if r["fp8"]:
            np.testing.assert_array_equal(sc.cpu().numpy().view(np.uint32), osc.view(np.uint32))
        np.testing.assert_array_equal(host_u16(r["comb"]), oracle.combine(lay, w.H, r["y"], r["wt"]))
        r["h"].free()



def _edge_value_rows(T, H, seed):
    """bf16 rows whose 128-channel blocks stress the fp8 arithmetic: all subnormal (the
    scale amax / 448 is then an fp32 subnormal), one normal value among subnormals (codes
    that underflow to zero or to E4M3 subnormals), magnitudes spread over many binades, the
    largest finite bf16 (0x7F7F), signed zeros, and non-finite blocks: a NaN (either sign,
    quiet or signalling payload) among normal values, +-Inf among normal values, and a
    block of -Inf only."""
    rng = np.random.default_rng(seed)
    x = np.zeros((T, H), np.uint16)
    for u in range(T):
        for b in range(H // 128):
            kind = (u + b) % 8
            blk = np.zeros(128, np.uint16)
            sign = rng.integers(0, 2, 128).astype(np.uint16) << 15
            if kind == 0:    # all subnormal: exponent 0, random non-zero mantissas
                blk = sign | rng.integers(1, 0x80, 128).astype(np.uint16)
            elif kind == 1:  # one normal value, the rest subnormal
                blk = sign | rng.integers(1, 0x80, 128).astype(np.uint16)
                blk[rng.integers(0, 128)] = 0x3F80 | sign[0]
            elif kind == 2:  # magnitudes across ~60 binades
                e = rng.integers(60, 121, 128).astype(np.uint16)
                blk = sign | (e << 7) | rng.integers(0, 0x80, 128).astype(np.uint16)
            elif kind == 3:  # the largest finite bf16 and small neighbours
                blk = sign | rng.integers(0x3000, 0x4000, 128).astype(np.uint16)
                blk[rng.integers(0, 128)] = 0x7F7F
            elif kind == 4:  # signed zeros with one tiny subnormal
                blk = sign.copy()
                blk[rng.integers(0, 128)] |= 0x0001
            elif kind == 5:  # one NaN among normal values
                blk = sign | rng.integers(0x3000, 0x4000, 128).astype(np.uint16)
                blk[rng.integers(0, 128)] = int(rng.choice([0x7FC0, 0xFFC0, 0x7F81, 0xFFFF]))
            elif kind == 6:  # +Inf and -Inf among normal values
                blk = sign | rng.integers(0x3000, 0x4000, 128).astype(np.uint16)
                blk[rng.integers(0, 64)] = 0x7F80
                blk[64 + rng.integers(0, 64)] = 0xFF80
            else:            # -Inf only
                blk = np.full(128, 0xFF80, np.uint16)
            x[u, 128 * b:128 * (b + 1)] = blk
    return x


@pytest.mark.parametrize("cm", [False, True], ids=["row-major", "col-major"])
def test_fp8_dispatch_on_subnormal_and_extreme_values(cm):
    """The fp8 dispatch's scale (amax / 448) and codes (x / scale, E4M3 RNE) on blocks the
    synthetic workloads never produce, bit for bit against the oracle, NaN and Inf blocks
    included (their scale and codes follow the oracle's stated rule)."""
    w = D["tiny-p4-s64-e16-k2-h512"]
    topk = synth.gen_routing(w)
    x = _edge_value_rows(w.T, w.H, 41)
    wt = synth.gen_weights(w)
    lay, h = layout_both(w, topk)
    rx, sc, rw, rm = ep.dispatch(h, dev_bf16(x), torch.from_numpy(wt).to(DEV), fp8=True, zero_padding=True,
                                 scales_col_major=cm)
    torch.cuda.synchronize()
    ox, osc, _, _, _ = oracle.dispatch_general(lay, w.H, fp8=True, zero_padding=True, topk_weights=wt, x=x,
                                               scales_col_major=cm)
    gs = sc.cpu().numpy()
    # scales first: a flushed subnormal scale would show here
    np.testing.assert_array_equal(gs.view(np.uint32), osc.view(np.uint32))
    np.testing.assert_array_equal(rx.cpu().numpy(), ox)
    assert np.any((osc.view(np.uint32) & 0x7F800000) == 0) and np.any(osc > 0)  # subnormal scales were exercised
    assert np.any(osc.view(np.uint32) == 0x7FC00000) and np.any(osc.view(np.uint32) == 0x7F800000)  # NaN, Inf
    h.free()



@pytest.mark.parametrize("H", [8320, 16384], ids=["h8320-65-blocks", "h16384-128-blocks"])
@pytest.mark.parametrize("mode", ["exact", "fixed"])
def test_large_hidden_sizes(H, mode):
    """Hidden sizes above the workloads' 7168: more column parts per row, and more than 64
    fp8 scale blocks, so the column-major scales pass transposes in several slabs (8320: a
    second slab of one block; 16384: two full slabs).  bf16 and fp8 (fused and pre-quantised,
    row- and column-major scales), then combine, against the oracle."""
    w = wl.Workload(f"large-h{H}", 4, 40, 16, 4, H, 4, True, "uniform", seed=61)
    topk = routing_with_holes(w, 62)
    lay = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk)
    W = max(1, int(np.median(lay.num_expanded))) if mode == "fixed" else 0
    h = ep.get_layout(ep.Config(w.P, w.S, w.H, w.K, w.E, w.A, num_worst_rows=W), torch.from_numpy(topk).to(DEV))
    R, nb = h.total_rows, H // 128
    x = synth.gen_bf16_rows(w.seed, wl.STREAM_X, w.T, H)
    wt = synth.gen_weights(w)
    xd, wd = dev_bf16(x), torch.from_numpy(wt).to(DEV)
    rng = np.random.default_rng(63)
    codes = rng.integers(0, 256, (w.T, H), dtype=np.uint8)
    scales = rng.standard_normal((w.T, nb)).astype(np.float32)
    # bf16
    rx, _, rw, rm = ep.dispatch(h, xd, wd, zero_padding=True)
    torch.cuda.synchronize()
    ox, _, ow, om, _ = oracle.dispatch_general(lay, H, fp8=False, zero_padding=True, topk_weights=wt, x=x, capacity=W)
    np.testing.assert_array_equal(host_u16(rx), ox)
    np.testing.assert_array_equal(rm.cpu().numpy(), om)
    np.testing.assert_array_equal(rw.cpu().numpy().view(np.uint32), ow.view(np.uint32))
    # fp8 variants
    for src in ("fused", "prequant"):
        xin = xd if src == "fused" else (_dev_u8(codes), torch.from_numpy(scales).to(DEV))
        kw = dict(x=x) if src == "fused" else dict(x_codes=codes, x_scales=scales)
        for cm in (False, True):
            say("large hidden", H, mode, src, "col-major" if cm else "row-major")
            qx, qs, _, _ = ep.dispatch(h, xin, wd, fp8=True, zero_padding=True, scales_col_major=cm)
            torch.cuda.synchronize()
            ox, osc, _, _, _ = oracle.dispatch_general(lay, H, fp8=True, zero_padding=True, topk_weights=wt,
                                                       capacity=W, scales_col_major=cm, **kw)
            np.testing.assert_array_equal(qx.cpu().numpy(), ox)
            np.testing.assert_array_equal(qs.cpu().numpy().view(np.uint32), osc.view(np.uint32))
    # combine
    y = synth.gen_expert_out(w, R)
    out = ep.combine(h, dev_bf16(y), wd)
    torch.cuda.synchronize()
    exp = oracle.combine_general(lay, H, y, wt, capacity=W)
    np.testing.assert_array_equal(host_u16(out), exp)
    h.free()


def test_debug_copy_is_a_copy():
    """The calibration copy moves every byte (a few MiB, an odd number of KiB)."""
    src = torch.randint(0, 256, ((4 << 20) + 3 * 1024,), dtype=torch.uint8, device=DEV)
    dst = torch.zeros_like(src)
    ep.debug_copy(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)


def test_c_abi_program_roundtrip():
    """The C ABI from C++ alone (tests/c_abi/roundtrip.cpp), run as a child process, against
    the oracle: layout, bf16 / fp8 / cached dispatch and combine; output buffers sized by
    ep_buffer_size_hint; fp8 with UE8M0 scales; ep_dispatch_noalloc with column-major
    scales; fixed-length windows (dispatch with zero tails, status, combine)."""
    import os
    import subprocess

    exe = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "roundtrip")
    assert os.path.exists(exe), "build tests/c_abi/roundtrip first (__graft_entry__.build())"
    say("c abi roundtrip")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0 and "ok" in r.stdout, (r.returncode, r.stdout, r.stderr)


def test_fixed_windows_capture_in_a_graph():
    """Fixed windows never wait on the host, so relayout + dispatch + combine can be captured
    in one graph.  Each replay (new x copied into the captured input between replays, with
    eager work and synchronisations in between) must match the eager calls."""
    w = SMALL[1]
    topk = synth.gen_routing(w)
    lay = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk)
    W = int(lay.num_expanded.max()) + 64
    topk_d = torch.from_numpy(topk).to(DEV)
    h = ep.get_layout(ep.Config(w.P, w.S, w.H, w.K, w.E, w.A, num_worst_rows=W), topk_d)
    wt = synth.gen_weights(w)
    wd = torch.from_numpy(wt).to(DEV)
    x_static = dev_bf16(synth.gen_bf16_rows(w.seed, wl.STREAM_X, w.T, w.H))
    R = h.total_rows
    rx = torch.empty((R, w.H), dtype=torch.bfloat16, device=DEV)
    rw = torch.empty(R, dtype=torch.float32, device=DEV)
    rm = torch.empty((R, 2), dtype=torch.int32, device=DEV)
    out = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=DEV)

    def step():
        ep.relayout(h, topk_d)
        ep.dispatch(h, x_static, wd, zero_padding=True, out=(rx, None, rw, rm))
        ep.combine(h, rx, wd, out=out)

    step()  # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("capture fixed-window step")
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for it in range(3):
        xi = dev_bf16(synth.gen_bf16_rows(w.seed + 100 + it, wl.STREAM_X, w.T, w.H))
        x_static.copy_(xi)
        torch.cuda.synchronize()
        say("graph replay", it)
        g.replay()
        torch.cuda.synchronize()
        got = (rx.clone(), rw.clone(), rm.clone(), out.clone())
        step()  # eager reference on the same input
        torch.cuda.synchronize()
        assert torch.equal(got[0].view(torch.int16), rx.view(torch.int16))
        assert torch.equal(got[1].view(torch.int32), rw.view(torch.int32))
        assert torch.equal(got[2], rm)
        assert torch.equal(got[3].view(torch.int16), out.view(torch.int16))
        # and against the oracle
        np.testing.assert_array_equal(host_u16(got[3]), oracle.combine_identity(w.K, w.H, False, topk,
                                                                                 host_u16(xi), wt, 0, w.T))
    assert h.status() == (0, 0)
    del g
    h.free()



def test_fixed_windows_fp8_graph_replays_with_new_routing():
    """Fixed windows, fp8 with column-major scales, captured as relayout + dispatch in one
    graph.  Before each replay a new routing and new x are copied into the captured inputs,
    so every replay recomputes the whole layout; each replay must match the eager calls and
    the oracle."""
    w = SMALL[1]
    nb = w.H // 128
    routings = [synth.gen_routing(synth.scaled(w, seed=w.seed + 200 + i)) for i in range(4)]
    lays = [oracle.layout(w.P, w.S, w.E, w.K, w.A, r) for r in routings]
    W = max(int(l.num_expanded.max()) for l in lays) + 64
    topk_d = torch.from_numpy(routings[0]).to(DEV)
    h = ep.get_layout(ep.Config(w.P, w.S, w.H, w.K, w.E, w.A, num_worst_rows=W), topk_d)
    wt = synth.gen_weights(w)
    wd = torch.from_numpy(wt).to(DEV)
    x_static = dev_bf16(synth.gen_bf16_rows(w.seed, wl.STREAM_X, w.T, w.H))
    R = h.total_rows
    rq = torch.empty((R, w.H), dtype=torch.uint8, device=DEV)
    scm = torch.empty((nb, R), dtype=torch.float32, device=DEV)
    rw = torch.empty(R, dtype=torch.float32, device=DEV)
    rm = torch.empty((R, 2), dtype=torch.int32, device=DEV)

    def step():
        ep.relayout(h, topk_d)
        ep.dispatch(h, x_static, wd, fp8=True, zero_padding=True, scales_col_major=True, out=(rq, scm, rw, rm))

    step()  # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("capture fixed-window fp8 step")
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for it in range(1, 4):
        xi = synth.gen_bf16_rows(w.seed + 300 + it, wl.STREAM_X, w.T, w.H)
        topk_d.copy_(torch.from_numpy(routings[it]).to(DEV))
        x_static.copy_(dev_bf16(xi))
        torch.cuda.synchronize()
        say("fp8 graph replay", it)
        g.replay()
        torch.cuda.synchronize()
        got = (rq.clone(), scm.clone(), rw.clone(), rm.clone())
        ox, osc, ow, om, dropped = oracle.dispatch_general(lays[it], w.H, fp8=True, zero_padding=True,
                                                           topk_weights=wt, x=xi, capacity=W, scales_col_major=True)
        assert dropped == 0
        np.testing.assert_array_equal(got[0].cpu().numpy(), ox)
        np.testing.assert_array_equal(got[1].cpu().numpy().view(np.uint32), osc.view(np.uint32))
        np.testing.assert_array_equal(got[2].cpu().numpy().view(np.uint32), ow.view(np.uint32))
        np.testing.assert_array_equal(got[3].cpu().numpy(), om)
        step()  # eager on the same inputs
        torch.cuda.synchronize()
        assert torch.equal(got[0], rq) and torch.equal(got[1].view(torch.int32), scm.view(torch.int32))
        assert torch.equal(got[2].view(torch.int32), rw.view(torch.int32)) and torch.equal(got[3], rm)
        check_fixed_layout(lays[it], h, W)
    assert h.status() == (0, 0)
    del g
    h.free()


def test_fixed_windows_status_follows_graph_replays():
    """A fixed-window relayout captured in a graph, replayed with routings copied into the
    captured input and no eager layout in between: after each replay (and a wait for it),
    the handle's status and counts are those of that replay's routing, truncation included,
    and cleared again by the next replay that fits."""
    w = SMALL[1]
    fits = synth.gen_routing(w)
    hot = fits.copy()
    hot[:, 0] = 0  # every token's first slot to expert 0: rank 0's window overflows
    lay_fit = oracle.layout(w.P, w.S, w.E, w.K, w.A, fits)
    lay_hot = oracle.layout(w.P, w.S, w.E, w.K, w.A, hot)
    W = int(lay_fit.num_expanded.max()) + 16
    assert int(lay_hot.num_expanded.max()) > W
    dropped_hot = int(np.maximum(lay_hot.num_expanded - W, 0).sum())
    topk_d = torch.from_numpy(fits).to(DEV)
    h = ep.get_layout(ep.Config(w.P, w.S, w.H, w.K, w.E, w.A, num_worst_rows=W), topk_d)
    torch.cuda.synchronize()
    assert h.status() == (0, 0)
    g = torch.cuda.CUDAGraph()
    say("capture fixed-window relayout")
    with torch.cuda.graph(g):
        ep.relayout(h, topk_d)
    torch.cuda.synchronize()
    for it, (routing, lay) in enumerate([(hot, lay_hot), (fits, lay_fit), (hot, lay_hot)]):
        topk_d.copy_(torch.from_numpy(routing).to(DEV))
        torch.cuda.synchronize()
        say("status replay", it)
        g.replay()
        torch.cuda.synchronize()
        exp = (ep.STATUS_TRUNCATED, dropped_hot) if routing is hot else (0, 0)
        assert h.status() == exp, (it, h.status(), exp)
        ne, nr, _ = h.counts()
        np.testing.assert_array_equal(ne, lay.num_expanded)
        np.testing.assert_array_equal(nr, lay.num_recv_tokens)
        check_fixed_layout(lay, h, W)
    del g
    h.free()


def test_exact_windows_layout_refuses_graph_capture():
    """An exact-window layout waits for the row counts on the host, which a captured graph
    cannot do: relayout on a capturing stream fails before enqueuing anything, and the
    handle works again after an eager relayout."""
    w = SMALL[1]
    topk = synth.gen_routing(w)
    lay, h = layout_both(w, topk)
    topk_d = torch.from_numpy(topk).to(DEV)
    g = torch.cuda.CUDAGraph()
    with pytest.raises(ep.EpError) as ei:
        with torch.cuda.graph(g):
            ep.relayout(h, topk_d)
    assert "captured" in str(ei.value)
    del g
    torch.cuda.synchronize()
    ep.relayout(h, topk_d)
    torch.cuda.synchronize()
    check_layout(lay, h)
    h.free()


def test_combine_lds_grid_limit_falls_back_to_register_kernel():
    """At 2^22 tokens the LDS combine's grid (one 512-thread workgroup per token) would reach
    2^31 work-items; combine then runs the register kernel, which is correct for every
    shape.  P=1, S=2^22, E=1, K=1, H=8: dispatch and combine against the oracle."""
    w = wl.Workload("lds-grid-limit", 1, 1 << 22, 1, 1, 8, 1, True, "uniform", seed=71)
    topk = np.zeros((w.T, 1), np.int64)
    topk[::7, 0] = -1  # some unused slots
    lay, h = layout_both(w, topk)
    x = synth.gen_bf16_rows(72, wl.STREAM_X, w.T, w.H)
    wt = np.random.default_rng(73).random((w.T, 1), dtype=np.float32)
    xd, wd = dev_bf16(x), torch.from_numpy(wt).to(DEV)
    rx, _, _, _ = ep.dispatch(h, xd, wd, zero_padding=True)
    out = ep.combine(h, rx, wd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_u16(out), oracle.combine_identity(1, w.H, False, topk, x, wt, 0, w.T))
    h.free()


def test_exact_windows_dispatch_and_combine_capture_in_a_graph():
    """With exact windows the layout waits on the host once, so it stays outside; the
    dispatches (bf16 fresh, fp8 cached) and the combine with a bias are captured.  Each replay
    (new x and bias copied into the captured inputs, with eager work and synchronisations in
    between) must match the eager calls, and the combine the oracle."""
    w = SMALL[1]
    topk = synth.gen_routing(w)
    topk_d = torch.from_numpy(topk).to(DEV)
    h = ep.get_layout(ep.Config(w.P, w.S, w.H, w.K, w.E, w.A), topk_d)
    wt = synth.gen_weights(w)
    wd = torch.from_numpy(wt).to(DEV)
    x_static = dev_bf16(synth.gen_bf16_rows(w.seed, wl.STREAM_X, w.T, w.H))
    b_static = dev_bf16(synth.gen_bf16_rows(w.seed + 7, wl.STREAM_X, w.T, w.H))
    R = h.total_rows
    rx = torch.empty((R, w.H), dtype=torch.bfloat16, device=DEV)
    rw = torch.empty(R, dtype=torch.float32, device=DEV)
    rm = torch.empty((R, 2), dtype=torch.int32, device=DEV)
    q8 = torch.empty((R, w.H), dtype=torch.uint8, device=DEV)
    s8 = torch.empty((R, w.H // 128), dtype=torch.float32, device=DEV)
    out = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=DEV)

    def step():
        ep.dispatch(h, x_static, wd, zero_padding=True, out=(rx, None, rw, rm))
        ep.dispatch_cached(h, x_static, fp8=True, zero_padding=True, out=(q8, s8))
        ep.combine(h, rx, wd, bias=b_static, out=out)

    step()  # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("capture exact-window dispatch + combine")
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for it in range(3):
        xi = dev_bf16(synth.gen_bf16_rows(w.seed + 200 + it, wl.STREAM_X, w.T, w.H))
        bi = dev_bf16(synth.gen_bf16_rows(w.seed + 300 + it, wl.STREAM_X, w.T, w.H))
        x_static.copy_(xi)
        b_static.copy_(bi)
        torch.cuda.synchronize()
        say("graph replay", it)
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (rx, rw, rm, q8, s8, out)]
        step()  # eager reference on the same inputs
        torch.cuda.synchronize()
        for a, b in zip(got, (rx, rw, rm, q8, s8, out)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
        np.testing.assert_array_equal(
            host_u16(got[5]),
            oracle.combine_identity(w.K, w.H, False, topk, host_u16(xi), wt, 0, w.T, bias=host_u16(bi)))
    del g
    h.free()


def test_binding_rejects_wrong_output_tensors():
    """The C ABI takes bare pointers, so the binding checks every caller-provided tensor
    (dtype, shape, contiguity, device) before anything is launched."""
    w = D["tiny-p4-s64-e16-k2-h512"]
    topk_d = torch.from_numpy(synth.gen_routing(w)).to(DEV)
    h = ep.get_layout(ep.Config(w.P, w.S, w.H, w.K, w.E, w.A), topk_d)
    R = h.total_rows
    xd = dev_bf16(synth.gen_bf16_rows(w.seed, wl.STREAM_X, w.T, w.H))
    wd = torch.from_numpy(synth.gen_weights(w)).to(DEV)
    good = (torch.empty((R, w.H), dtype=torch.bfloat16, device=DEV), None,
            torch.empty(R, dtype=torch.float32, device=DEV), torch.empty((R, 2), dtype=torch.int32, device=DEV))
    bad_cases = [
        ((torch.empty((R - 1, w.H), dtype=torch.bfloat16, device=DEV),) + good[1:], ValueError),  # one row short
        ((torch.empty((R, w.H), dtype=torch.float16, device=DEV),) + good[1:], TypeError),
        ((torch.empty((w.H, R), dtype=torch.bfloat16, device=DEV).T,) + good[1:], ValueError),  # not contiguous
        (good[:2] + (torch.empty(R - 1, dtype=torch.float32, device=DEV), good[3]), ValueError),
        (good[:3] + (torch.empty((R, 3), dtype=torch.int32, device=DEV),), ValueError),
        ((good[0].cpu(),) + good[1:], ValueError),
    ]
    for out, exc in bad_cases:
        with pytest.raises(exc):
            ep.dispatch(h, xd, wd, zero_padding=True, out=out)
    # fp8: scales required, in the layout the flags ask for
    q8 = torch.empty((R, w.H), dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        ep.dispatch(h, xd, wd, fp8=True, out=(q8, None, good[2], good[3]))
    with pytest.raises(ValueError):
        ep.dispatch_cached(h, xd, fp8=True, scales_col_major=True,
                           out=(q8, torch.empty((R, w.H // 128), dtype=torch.float32, device=DEV)))
    with pytest.raises(ValueError):
        ep.combine(h, good[0], wd, out=torch.empty((w.T - 1, w.H), dtype=torch.bfloat16, device=DEV))
    # and the well-formed call still works
    rx, _, _, _ = ep.dispatch(h, xd, wd, zero_padding=True, out=good)
    out = ep.combine(h, rx, wd)
    torch.cuda.synchronize()
    assert out.shape == (w.T, w.H)
    h.free()


@pytest.mark.parametrize("H", [8, 4104], ids=["lds-kernel", "register-kernel"])
def test_combine_arithmetic_order_on_adversarial_values(H):
    """Values for which another summation order, a fused multiply-add, or adding the bias
    first changes the bf16 result (the oracle's pins derive each expected value by hand):
    both combine kernels must give exactly these."""
    B = float(np.float32(2.0**25 + 2.0**17))
    cases = [  # (weights, y row bits per slot, bias bits or None, expected out bits)
        ([B, 1.0, 1.0, 1.0], None, None, 0x4C00),
        ([1.0, 1.0, 1.0, B], None, None, 0x4C01),
        ([-(1.0 + 2.0**-7 + 2.0**-23), 1.0 + 2.0**-23], [0x3F80, 0x3F81], None, 0x0000),
        ([1.0, 1.0, B], None, 0x3F80, 0x4C00),
    ]
    for weights, rows, bias, expect in cases:
        K = len(weights)
        topk = np.arange(K, dtype=np.int64)[None, :]
        h = ep.get_layout(ep.Config(1, 1, H, K, K, 1), torch.from_numpy(topk).to(DEV))
        assert h.total_rows == K
        rows = [0x3F80] * K if rows is None else rows
        y = np.repeat(np.asarray(rows, np.uint16)[:, None], H, 1)
        wd = torch.tensor([weights], dtype=torch.float32, device=DEV)
        bd = None if bias is None else dev_bf16(np.full((1, H), bias, np.uint16))
        say("adversarial combine", H, K, expect)
        out = ep.combine(h, dev_bf16(y), wd, bias=bd)
        torch.cuda.synchronize()
        got = host_u16(out)
        assert np.all(got == expect), (weights, hex(int(got[0, 0])), hex(expect))
        lay = oracle.layout(1, 1, K, K, 1, topk)
        np.testing.assert_array_equal(got, oracle.combine_general(
            lay, H, y, np.asarray([weights], np.float32), bias=None if bias is None else np.full((1, H), bias, np.uint16)))
        h.free()



@pytest.mark.parametrize("H", [512, 4104], ids=["lds-kernel", "register-kernel"])
def test_combine_on_subnormal_and_extreme_values(H):
    """Combine where products and sums reach the fp32 and bf16 subnormal ranges: expert rows
    mixing bf16 subnormals, tiny, moderate and large (up to 2^120) values, weights down to
    2^-120.  Magnitudes stay low enough that no sum overflows, so the result has no NaN.
    Bit for bit against the oracle, through both combine kernels."""
    P, S, E, K, A = 4, 40, 16, 4, 4
    w = wl.Workload(f"extreme-combine-h{H}", P, S, E, K, H, A, True, "uniform", seed=51)
    topk = synth.gen_routing(w)
    lay, h = layout_both(w, topk)
    rng = np.random.default_rng(52)
    R = lay.total_rows
    cls = rng.integers(0, 5, (R, H))
    sign = (rng.integers(0, 2, (R, H)) << 15).astype(np.uint16)
    mant = rng.integers(0, 0x80, (R, H)).astype(np.uint16)
    expo = np.select([cls == 0, cls == 1, cls == 2, cls == 3], [0, rng.integers(1, 20, (R, H)),
                     rng.integers(100, 150, (R, H)), rng.integers(200, 247, (R, H))], 0).astype(np.uint16)
    y = sign | (expo << 7) | np.where(cls == 0, np.maximum(mant, 1), mant).astype(np.uint16)
    y[cls == 4] = sign[cls == 4]  # signed zeros
    wt = synth.gen_weights(w).copy()
    tiny = rng.random(wt.shape) < 0.3
    wt[tiny] = np.ldexp(np.float32(1.0), -rng.integers(60, 121, int(tiny.sum()))).astype(np.float32)
    out = ep.combine(h, dev_bf16(y), torch.from_numpy(wt).to(DEV))
    torch.cuda.synchronize()
    exp = oracle.combine(lay, H, y, wt)
    got = host_u16(out)
    assert not np.any(((exp & 0x7F80) == 0x7F80) & ((exp & 0x7F) != 0))  # no NaN expected
    assert np.any(((exp & 0x7F80) == 0) & ((exp & 0x7F) != 0))  # subnormal outputs were exercised
    np.testing.assert_array_equal(got, exp)
    h.free()


@pytest.mark.parametrize("H", [512, 4104], ids=["lds-kernel", "register-kernel"])
def test_combine_on_non_finite_values(H):
    """Combine with Inf and NaN among the expert rows and one overflowing sum.  Which NaN an
    fp32 operation returns is the hardware's choice (the host's default NaN is negative, the
    GPU's positive), so NaN outputs are compared as NaN; every other output, the infinities
    included, bit for bit against the oracle, through both combine kernels."""
    P, S, E, K, A = 4, 40, 16, 4, 4
    w = wl.Workload(f"nonfinite-combine-h{H}", P, S, E, K, H, A, True, "uniform", seed=61)
    topk = synth.gen_routing(w)
    lay, h = layout_both(w, topk)
    rng = np.random.default_rng(62)
    R = lay.total_rows
    y = synth.gen_bf16_rows(63, wl.STREAM_X, R, H)
    pick = rng.random((R, H))
    y[pick < 0.01] = 0x7F80                                        # +Inf
    y[(pick >= 0.01) & (pick < 0.02)] = 0xFF80                     # -Inf
    y[(pick >= 0.02) & (pick < 0.025)] = 0x7FC0                    # NaN
    y[(pick >= 0.025) & (pick < 0.03)] = 0x7F7F                    # largest finite: sums overflow
    wt = synth.gen_weights(w)
    out = ep.combine(h, dev_bf16(y), torch.from_numpy(wt).to(DEV))
    torch.cuda.synchronize()
    exp = oracle.combine(lay, H, y, wt)
    got = host_u16(out)
    is_nan = lambda a: ((a & 0x7F80) == 0x7F80) & ((a & 0x7F) != 0)  # noqa: E731
    np.testing.assert_array_equal(is_nan(got), is_nan(exp))
    fin = ~is_nan(exp)
    np.testing.assert_array_equal(got[fin], exp[fin])
    assert is_nan(exp).any() and ((exp & 0x7FFF) == 0x7F80).any()  # NaN and Inf outputs were exercised
    h.free()


def test_relayout_and_free_wait_for_pending_async_calls():
    """An async dispatch reads the handle on the communication stream.  A relayout enqueued
    right after it must not overwrite the arrays under it, and free() must not release them:
    the binding orders the relayout after the pending call and waits for it in free()."""
    w = SMALL[1]
    topk_a = synth.gen_routing(w)
    topk_b = synth.gen_routing(wl.Workload(w.name, w.P, w.S, w.E, w.K, w.H, w.A, True, "uniform", seed=99))
    x = synth.gen_bf16_rows(w.seed, wl.STREAM_X, w.T, w.H)
    wt = synth.gen_weights(w)
    xd, wd = dev_bf16(x), torch.from_numpy(wt).to(DEV)
    lay_a = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk_a)
    ox, _, _, om = oracle.dispatch(lay_a, w.H, x, wt, False, True)
    for action in ("relayout", "free"):
        h = ep.get_layout(ep.Config(w.P, w.S, w.H, w.K, w.E, w.A), torch.from_numpy(topk_a).to(DEV))
        say("async dispatch then", action)
        pending = ep.dispatch(h, xd, wd, zero_padding=True, async_with_compute_stream=True)
        if action == "relayout":
            ep.relayout(h, torch.from_numpy(topk_b).to(DEV))
        else:
            h.free()
        rx, _, _, rm = pending.wait()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host_u16(rx), ox)
        np.testing.assert_array_equal(rm.cpu().numpy(), om)
        if action == "relayout":
            lay_b = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk_b)
            np.testing.assert_array_equal(h.tensor("dst_slot").cpu().numpy(), lay_b.dst_slot.reshape(-1))
            h.free()


def test_column_major_fp8_calls_on_two_streams_do_not_share_scratch():
    """fp8 dispatch with column-major scales stages per-token scales in the handle.  An async
    call on the communication stream followed at once by a synchronous one on the current
    stream must each keep their own scales: the library orders the second after the first."""
    w = SMALL[1]
    topk = synth.gen_routing(w)
    wt = synth.gen_weights(w)
    wd = torch.from_numpy(wt).to(DEV)
    x1 = synth.gen_bf16_rows(w.seed + 1, wl.STREAM_X, w.T, w.H)
    x2 = synth.gen_bf16_rows(w.seed + 2, wl.STREAM_X, w.T, w.H)
    lay = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk)
    h = ep.get_layout(ep.Config(w.P, w.S, w.H, w.K, w.E, w.A), torch.from_numpy(topk).to(DEV))
    say("async col-major fp8 then sync col-major fp8")
    pending = ep.dispatch(h, dev_bf16(x1), wd, fp8=True, zero_padding=True, scales_col_major=True,
                          async_with_compute_stream=True)
    r2 = ep.dispatch(h, dev_bf16(x2), wd, fp8=True, zero_padding=True, scales_col_major=True)
    r1 = pending.wait()
    torch.cuda.synchronize()
    for (rx, sc, _, _), x in ((r1, x1), (r2, x2)):
        ox, osc, _, _, _ = oracle.dispatch_general(lay, w.H, fp8=True, zero_padding=True, topk_weights=wt, x=x,
                                                   scales_col_major=True)
        np.testing.assert_array_equal(rx.cpu().numpy(), ox)
        np.testing.assert_array_equal(sc.cpu().numpy().view(np.uint32), osc.view(np.uint32))
    h.free()


def test_column_major_fp8_calls_through_the_c_abi_on_two_streams():
    """The same ordering without the Python binding's help: two ep_dispatch calls (fp8,
    column-major scales) on one handle, issued back to back through the C ABI on two
    unordered streams, the first with a longer queue ahead of it.  Each call's codes and
    scales must match the oracle for its own x."""
    import ctypes

    w = SMALL[1]
    topk = synth.gen_routing(w)
    wt = synth.gen_weights(w)
    wd = torch.from_numpy(wt).to(DEV)
    xs = [synth.gen_bf16_rows(w.seed + 11 + i, wl.STREAM_X, w.T, w.H) for i in range(2)]
    xds = [dev_bf16(x) for x in xs]
    lay = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk)
    h = ep.get_layout(ep.Config(w.P, w.S, w.H, w.K, w.E, w.A), torch.from_numpy(topk).to(DEV))
    R, nb = h.total_rows, w.H // 128
    outs = [(torch.empty((R, w.H), dtype=torch.uint8, device=DEV), torch.empty((nb, R), dtype=torch.float32, device=DEV),
             torch.empty(R, dtype=torch.float32, device=DEV), torch.empty((R, 2), dtype=torch.int32, device=DEV))
            for _ in range(2)]
    streams = [torch.cuda.Stream(DEV), torch.cuda.Stream(DEV)]
    torch.cuda.synchronize()
    L = ep.lib()
    flags = 1 | 2 | 4  # EP_DISPATCH_FP8 | EP_DISPATCH_ZERO_PADDING | EP_DISPATCH_SCALES_COL_MAJOR
    say("two col-major fp8 dispatches through the C ABI on two streams")
    with torch.cuda.stream(streams[0]):
        busy = torch.empty(1 << 26, dtype=torch.float32, device=DEV)
        for _ in range(4):
            busy.mul_(1.0001)  # work queued ahead of the first call
    for i in range(2):
        rx, sc, rw, rm = outs[i]
        st = L.ep_dispatch(ctypes.c_void_p(h.ptr), flags, ctypes.c_void_p(xds[i].data_ptr()),
                           ctypes.c_void_p(wd.data_ptr()), ctypes.c_void_p(rx.data_ptr()),
                           ctypes.c_void_p(sc.data_ptr()), ctypes.c_void_p(rw.data_ptr()),
                           ctypes.c_void_p(rm.data_ptr()), ctypes.c_void_p(streams[i].cuda_stream))
        assert st == 0, L.ep_last_error()
    torch.cuda.synchronize()
    for i in range(2):
        ox, osc, _, _, _ = oracle.dispatch_general(lay, w.H, fp8=True, zero_padding=True, topk_weights=wt, x=xs[i],
                                                   scales_col_major=True)
        np.testing.assert_array_equal(outs[i][0].cpu().numpy(), ox)
        np.testing.assert_array_equal(outs[i][1].cpu().numpy().view(np.uint32), osc.view(np.uint32))
    del busy
    h.free()


# --------------------------------------------------------------------------
# UE8M0 scales: one power-of-two exponent byte per 32 channels
# --------------------------------------------------------------------------

UE8M0_CASES = [D["tiny-p4-s64-e16-k2-h512"],
               synth.scaled(D["dsv3-bf16-p8-s4096-e256-k8-h7168"], S=300),
               synth.scaled(D["ep128-zipf-p128-s1024-e256-k6-h7168"], S=70, H=1024),
               wl.Workload("ue8m0-p4-s65-e32-k3-h8320", 4, 65, 32, 3, 8320, 8, True, "uniform", seed=81)]


def _ue8m0_edge_rows(T, H, seed):
    """bf16 rows whose 32-channel blocks exercise the exponent choice: the maximum exactly
    448 * 2^k, a mantissa just above 1.75, exact powers of two, zeros, subnormals, the
    smallest normal, the largest finite bf16, NaN and Inf; the rest N(0,1)."""
    rng = np.random.default_rng(seed)
    x = synth.gen_bf16_rows(seed, wl.STREAM_X, T, H).copy()
    for u in range(T):
        for b in range(H // 32):
            blk = x[u, 32 * b:32 * (b + 1)]
            kind = (u + b) % 10
            at = int(rng.integers(0, 32))
            if kind == 1:
                blk[at] = (((127 + 8 + int(rng.integers(-30, 30))) << 7) | 0x60)
            elif kind == 2:
                blk[at] = (int(rng.integers(100, 150)) << 7) | 0x61
            elif kind == 3:
                blk[:] = 0x8000 * rng.integers(0, 2, 32).astype(np.uint16)
            elif kind == 4:
                blk[:] = rng.integers(1, 0x80, 32).astype(np.uint16)
                blk[at] = 0x0080
            elif kind == 5:
                blk[at] = 0x7F7F
            elif kind == 6:
                blk[at] = int(rng.choice([0x7FC0, 0xFF81]))
            elif kind == 7:
                blk[at] = int(rng.choice([0x7F80, 0xFF80]))
            x[u, 32 * b:32 * (b + 1)] = blk
    return x


@pytest.mark.parametrize("w", UE8M0_CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("mode", ["exact", "fixed"])
@pytest.mark.parametrize("zp", [True, False], ids=["zero-pad", "no-pad"])
def test_ue8m0_dispatch_small(w, mode, zp):
    """Fresh and cached fp8 dispatch with UE8M0 scales, codes and exponent bytes bit for bit
    against the oracle (edge-value rows: NaN, Inf, exact 448 * 2^k maxima, subnormals),
    exact and fixed windows, with and without zero padding."""
    topk = routing_with_holes(w, 23)
    lay = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk)
    W = int(lay.num_expanded.max()) + 5 if mode == "fixed" else 0
    h = ep.get_layout(ep.Config(w.P, w.S, w.H, w.K, w.E, w.A, num_worst_rows=W), torch.from_numpy(topk).to(DEV))
    x = _ue8m0_edge_rows(w.T, w.H, 24)
    wt = synth.gen_weights(w)
    xd, wd = dev_bf16(x), torch.from_numpy(wt).to(DEV)
    R = h.total_rows
    rx = torch.full((R, w.H), 0x33, dtype=torch.uint8, device=DEV)
    sc = torch.full((R, w.H // 32), 0x33, dtype=torch.uint8, device=DEV)
    rw = torch.empty(R, dtype=torch.float32, device=DEV)
    rm = torch.empty((R, 2), dtype=torch.int32, device=DEV)
    say("ue8m0", w.name, mode, zp)
    ep.dispatch(h, xd, wd, zero_padding=zp, scales_ue8m0=True, out=(rx, sc, rw, rm))
    torch.cuda.synchronize()
    ox, osc, ow, om, _ = oracle.dispatch_general(lay, w.H, fp8=True, zero_padding=zp, topk_weights=wt, x=x,
                                                 capacity=W, scales_ue8m0=True, fill=0x33)
    np.testing.assert_array_equal(rx.cpu().numpy(), ox)
    np.testing.assert_array_equal(sc.cpu().numpy(), osc)
    np.testing.assert_array_equal(rw.cpu().numpy().view(np.uint32), ow.view(np.uint32))
    np.testing.assert_array_equal(rm.cpu().numpy(), om)
    assert (osc == 0xFF).any() and (osc == 0).any()
    # cached dispatch of other x into the same buffers
    x2 = synth.gen_bf16_rows(w.seed + 5, wl.STREAM_X, w.T, w.H)
    ep.dispatch_cached(h, dev_bf16(x2), zero_padding=zp, scales_ue8m0=True, out=(rx, sc))
    torch.cuda.synchronize()
    ox2, osc2, _, _, _ = oracle.dispatch_general(lay, w.H, fp8=True, zero_padding=zp, x=x2, capacity=W,
                                                 scales_ue8m0=True, with_meta=False, fill=0x33)
    # rows the cached call leaves alone still hold the first fill, as the oracle's do
    np.testing.assert_array_equal(rx.cpu().numpy(), ox2)
    np.testing.assert_array_equal(sc.cpu().numpy(), osc2)
    h.free()


def test_ue8m0_full_size():
    """The DSv3 fp8 workload with UE8M0 scales: every valid row's codes and exponent bytes
    against the oracle's per-token encoding, zero padding, and one cached iteration."""
    w = D["dsv3-fp8-p8-s4096-e256-k8-h7168"]
    topk = synth.gen_routing(w)
    lay, h = layout_both(w, topk)
    x = synth.gen_x(w)
    wt = synth.gen_weights(w)
    xd, wd = dev_bf16(x), torch.from_numpy(wt).to(DEV)
    rx, sc, rw, rm = ep.dispatch(h, xd, wd, zero_padding=True, scales_ue8m0=True)
    torch.cuda.synchronize()
    assert sc.dtype == torch.uint8 and tuple(sc.shape) == (h.total_rows, w.H // 32)
    for it in (0, 1):
        if it:
            x = synth.workloads.gen_cached_x(w, 1)
            xd = dev_bf16(x)
            rx.fill_(0x33)
            sc.fill_(0x33)
            ep.dispatch_cached(h, xd, zero_padding=True, scales_ue8m0=True, out=(rx, sc))
            torch.cuda.synchronize()
        say("ue8m0 full size, iteration", it)
        codes = np.empty((w.T, w.H), np.uint8)
        exps = np.empty((w.T, w.H // 32), np.uint8)
        oracle_over_ranges(lambda a, b: oracle.quantize_rows_ue8m0(x, w.H, a, b)[0], w.T, codes)
        oracle_over_ranges(lambda a, b: oracle.quantize_rows_ue8m0(x, w.H, a, b)[1], w.T, exps)
        codes_d, exps_d = torch.from_numpy(codes).to(DEV), torch.from_numpy(exps).to(DEV)
        El = w.E // w.P
        for j in range(w.K):
            m = topk[:, j] >= 0
            us = np.flatnonzero(m)
            rows = lay.window_row_base[topk[m, j] // El] + lay.dst_slot[m, j]
            assert torch.equal(gather_rows(rx, rows), gather_rows(codes_d, us)), j
            assert torch.equal(gather_rows(sc, rows), gather_rows(exps_d, us)), j
        pad = np.flatnonzero(rm.cpu().numpy()[:, 0] < 0)
        assert int(gather_rows(rx, pad).max()) == 0 and int(gather_rows(sc, pad).max()) == 0
    h.free()


def test_ue8m0_refusals():
    """UE8M0 scales are row-major and come from the fused quantisation: with column-major
    scales or pre-quantised input the call fails before anything is enqueued."""
    w = SMALL[0]
    topk = synth.gen_routing(w)
    h = ep.get_layout(ep.Config(w.P, w.S, w.H, w.K, w.E, w.A), torch.from_numpy(topk).to(DEV))
    R = h.total_rows
    xd = dev_bf16(synth.gen_x(w))
    wd = torch.from_numpy(synth.gen_weights(w)).to(DEV)
    L = ep.lib()
    import ctypes
    vp = ctypes.c_void_p
    rx = torch.full((R, w.H), 0x33, dtype=torch.uint8, device=DEV)
    sc = torch.full((R, w.H // 32), 0x33, dtype=torch.uint8, device=DEV)
    rw = torch.empty(R, dtype=torch.float32, device=DEV)
    rm = torch.empty((R, 2), dtype=torch.int32, device=DEV)
    st = L.ep_dispatch(vp(h.ptr), 1 | 4 | 8, vp(xd.data_ptr()), vp(wd.data_ptr()), vp(rx.data_ptr()),
                       vp(sc.data_ptr()), vp(rw.data_ptr()), vp(rm.data_ptr()), vp(0))
    assert st == ep.Status.ERR_SHAPE and b"UE8M0" in L.ep_last_error()
    codes = torch.zeros((w.T, w.H), dtype=torch.uint8, device=DEV)
    xs = torch.zeros((w.T, w.H // 128), dtype=torch.float32, device=DEV)
    st = L.ep_dispatch_prequant(vp(h.ptr), 8, vp(codes.data_ptr()), vp(xs.data_ptr()), vp(wd.data_ptr()),
                                vp(rx.data_ptr()), vp(sc.data_ptr()), vp(rw.data_ptr()), vp(rm.data_ptr()), vp(0))
    assert st == ep.Status.ERR_SHAPE
    torch.cuda.synchronize()
    assert bool((rx == 0x33).all()) and bool((sc == 0x33).all())
    h.free()
