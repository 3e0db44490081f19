"""Throughput of the MoE dispatch/combine hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic tokens.  On
the default workload (the forward+backward one: P=32 virtual ranks x S=8192
tokens, E=256, top-8 group-limited routing, hidden 4096) that is: fresh layout
of the routing (ep_relayout: counts, scans, stable ranks, the one D->H read of
the window sizes), fresh dispatch of x into the expanded expert-grouped layout
(bf16, zero padding), identity experts, weighted combine back to token order;
then the backward with the same handle: cached dispatch of the upstream
gradient and its weighted combine.  On a workload without a backward the step
stops after the forward combine.  Inputs are resident in HBM before the timed
region; the handle and the expanded tensors are long-lived buffers reused
every step, as the pages recommend for the EP buffer.

Beside the headline step the JSON line carries:
  "configs"        every other full-size workload timed per call (HIP events,
                   median of 20, each call behind a head start so that the
                   host's launch time stays outside the events): fresh
                   dispatch, cached dispatch (for the fp8
                   workload: 20 iterations, each with new x), combine, each
                   with its ledger bytes and fraction of the HBM peak;
  "fixed_windows"  the headline forward step with fixed-length windows
                   (num_worst_rows: a 1024-row bucket above the largest
                   window, no read-back);
  "cpu_baseline"   the CPU oracle on the headline workload, on 1 thread and
                   on N threads (a bounded sample: see cpu_baseline).

Before the timed steps, the outputs of the last warm-up step are checked at
full size with plain torch ops on a seeded sample of tokens (expanded rows,
their weights and metadata, zero padding, and the combine bit for bit, forward
and backward); "parity" in the JSON line says what was checked.

Prints ONE JSON line.  Usage:
    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload NAME] [--no-cpu]
                    [--no-fixed] [--no-configs]

`python bench.py --calls` instead times every call of the library on every
workload (HIP events; median and minimum of 20 calls, each timed alone after
3 untimed ones and behind a head start, once right after the previous call and
once with the L2s and the memory-side cache flushed by a 1 GiB scratch buffer;
layout rows are host wall-clock times) and prints one
JSON line per workload: layout, dispatch, cached dispatch, combine, combine
with a bias, fixed-window dispatch, and for fp8 workloads the pre-quantised
and column-major-scale dispatches, each with its ledger bytes and % of HBM;
and the fixed-window step (layout + dispatch + combine), which needs no host
sync, run eagerly and replayed from one captured HIP graph.

`python bench.py --overlap` times the pages' overlap pattern on the DSv3 BF16
workload: dispatch issued on the library's communication stream while the
shared experts (a bf16 MLP, hidden 7168 -> 2 x 2048 -> 7168, torch.matmul)
run on the compute stream, against the two run back to back.  It runs at
several tokens-per-rank counts (`--overlap-tokens`, default 128,512,4096:
decode-sized batches to the full workload), one JSON line each, GPU time
only (each timed region behind a head start).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "dispatch & combine payload GB/s + tokens/s on 1 MI355X; % HBM roofline"
DEFAULT_WORKLOAD = "ep32-group-fwdbwd-p32-s8192-e256-k8-h4096"
# full-size workloads timed per call beside the headline step
PER_CONFIG = ["dsv3-bf16-p8-s4096-e256-k8-h7168", "dsv3-fp8-p8-s4096-e256-k8-h7168",
              "ep128-zipf-p128-s1024-e256-k6-h7168"]
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, 8 TB/s
# the dispatch / combine kernels and their launch configuration: a committed counter
# summary counts only while these are unchanged
KERNEL_SOURCES = ["combine_topk_idx_expert_amd/csrc/ep_dispatch.hpp",
                  "combine_topk_idx_expert_amd/csrc/ep_device.hpp",
                  "combine_topk_idx_expert_amd/csrc/ep_launch.hpp"]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic byte ledger (what the method must move, not hardware traffic)
# ---------------------------------------------------------------------------

def ledger(T: int, K: int, H: int, rows: int, pad: int, fp8: bool, zero_padding: bool) -> dict:
    """Bytes read / written per call.

    rows = valid slots (expanded rows carrying a token), pad = alignment padding rows.
    dispatch: read x (T*H*2) + per slot its weight and destination row (8 B);
              write rows*(H*b + sf) payload, (rows+pad)*12 B of row metadata
              (weight + source (u, j)), and pad*(H*b + sf) zeros when zero padding.
    combine:  read rows*H*2 expert outputs + per slot weight and row (8 B);
              write T*H*2.
    """
    b = 1 if fp8 else 2
    sf = 4 * (H // 128) if fp8 else 0
    d_read = T * H * 2 + 8 * T * K
    d_write = rows * (H * b + sf) + (rows + pad) * 12 + (pad * (H * b + sf) if zero_padding else 0)
    c_read = rows * H * 2 + 8 * T * K
    c_write = T * H * 2
    return dict(dispatch_read=d_read, dispatch_write=d_write, dispatch=d_read + d_write,
                combine_read=c_read, combine_write=c_write, combine=c_read + c_write)


def page_style_payload(num_recv_total: int, T: int, K: int, H: int, fp8: bool) -> float:
    """The pages' bandwidth numerator: received tokens x logical bytes per token
    (x, topk_idx, topk_weights), no padding ("Measure time and bytes correctly first";
    tutorial section 7.4)."""
    per_tok = (H * (1 if fp8 else 2) + (4 * (H // 128) if fp8 else 0)) + 8 * K + 4 * K
    return float(num_recv_total) * per_tok


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != kernel_hash():
        return None
    return d.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, as it stands
# ---------------------------------------------------------------------------

def host_threads() -> tuple[int, int]:
    """(threads used, CPUs in the affinity mask): at most 16, one GPU's share of the box."""
    n = len(os.sched_getaffinity(0))
    return max(1, min(16, n)), n


def cpu_baseline(w, topk, x, g, wt, threads: int) -> dict:
    """The CPU oracle (oracle/, as it stands) on the headline workload, on 1 thread and on
    `threads` threads.  Each oracle call is one ctypes call, which releases the GIL, so the
    threaded leg runs the calls over disjoint row or token ranges in a thread pool.

    Per leg: the layout (one call; the oracle's layout is one sequential pass), the fresh
    dispatch of every expanded row and, with a backward, the cached dispatch of the gradient,
    both streamed one destination window per call (a window's rows are produced and dropped,
    so host memory stays at one window per thread); and the combine (forward and backward)
    on a bounded sample, the tokens of the first source ranks, whose time is scaled to all T
    tokens.  The sample's expert rows are filled with the identity experts' outputs (x, or
    the gradient, at each of their rows) before the timed call."""
    import statistics
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle

    T, K, H, P = w.T, w.K, w.H, w.P
    lay = oracle.layout(P, w.S, w.E, K, w.A, topk)
    R = lay.total_rows
    wrb = lay.window_row_base
    windows = [(int(wrb[d]), int(wrb[d + 1])) for d in range(P)]
    t_sample = min(T, 4 * w.S)
    # expert rows of the sampled tokens, and the identity experts' outputs there
    El = w.E // P
    tk = topk[:t_sample]
    valid = tk >= 0
    rows = (wrb[np.where(valid, tk // El, 0)] + lay.dst_slot[:t_sample])[valid]
    src = np.broadcast_to(np.arange(t_sample)[:, None], tk.shape)[valid]
    y = np.empty((R, H), np.uint16)  # only the sampled tokens' rows are ever touched

    def leg(nt: int) -> dict:
        pool = ThreadPoolExecutor(nt) if nt > 1 else None

        def run(fn, items):
            if pool is None:
                for it in items:
                    fn(it)
            else:
                list(pool.map(fn, items))

        sec = {}
        t0 = time.perf_counter()
        oracle.layout(P, w.S, w.E, K, w.A, topk)
        sec["layout"] = time.perf_counter() - t0
        t0 = time.perf_counter()
        run(lambda ab: oracle.dispatch(lay, H, x, wt, False, w.zero_padding, ab[0], ab[1]), windows)
        sec["dispatch"] = time.perf_counter() - t0
        tok_ranges = [(a, min(t_sample, a + -(-t_sample // nt))) for a in range(0, t_sample, -(-t_sample // nt))]
        y[rows] = x[src]
        t0 = time.perf_counter()
        run(lambda ab: oracle.combine(lay, H, y, wt, ab[0], ab[1]), tok_ranges)
        sec["combine_sample"] = time.perf_counter() - t0
        sec["combine"] = sec["combine_sample"] * T / t_sample
        if w.backward:
            t0 = time.perf_counter()
            run(lambda ab: oracle.dispatch(lay, H, g, None, False, w.zero_padding, ab[0], ab[1], with_meta=False),
                windows)
            sec["dispatch_cached_grad"] = time.perf_counter() - t0
            y[rows] = g[src]
            t0 = time.perf_counter()
            run(lambda ab: oracle.combine(lay, H, y, wt, ab[0], ab[1]), tok_ranges)
            sec["combine_grad_sample"] = time.perf_counter() - t0
            sec["combine_grad"] = sec["combine_grad_sample"] * T / t_sample
        if pool is not None:
            pool.shutdown()
        sec["step"] = sec["layout"] + sec["dispatch"] + sec["combine"] + \
            sec.get("dispatch_cached_grad", 0.0) + sec.get("combine_grad", 0.0)
        return {"value": T / sec["step"], "threads": nt, "seconds": sec}

    one = leg(1)
    many = leg(threads) if threads > 1 else one
    del y
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    _, affinity = host_threads()
    steps = "layout, dispatch of every expanded row" + (", cached dispatch of the gradient" if w.backward else "")
    comb = "forward and backward combine" if w.backward else "combine"
    return {"value": many["value"], "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model, "affinity_cpus": affinity,
            "sample": (f"headline workload {w.name} ({T} tokens, {R} expanded rows): {steps} in full, one "
                       f"destination window per call; {comb} on the tokens of the first "
                       f"{t_sample // max(w.S, 1)} source ranks ({t_sample} tokens), time scaled to all {T}; "
                       f"value = tokens/s of the whole step on {threads} threads"),
            "seconds": many["seconds"], "single_thread": one}


# ---------------------------------------------------------------------------
# fixed-length windows
# ---------------------------------------------------------------------------

def fixed_leg(ep, h_exact, w, topk, topk_d, x_d, w_d, out, steps: int, warmup: int) -> dict:
    """The step with every window fixed at W rows (W = the largest window rounded up to
    1024 rows): layout without any read-back, dispatch (tails zeroed), combine."""
    import numpy as np
    import torch

    ne, _, _ = h_exact.counts()
    W = int(-(-int(ne.max()) // 1024) * 1024)
    T, K, H = w.T, w.K, w.H
    dev = x_d.device
    log("fixed windows W =", W)
    h = ep.get_layout(ep.Config(w.P, w.S, H, K, w.E, w.A, num_worst_rows=W), topk_d)
    R = h.total_rows
    recv_x = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
    recv_w = torch.empty(R, dtype=torch.float32, device=dev)
    recv_m = torch.empty((R, 2), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        ep.relayout(h, topk_d)
        if ev is not None:
            ev[1].record(stream)
        ep.dispatch(h, x_d, w_d, fp8=False, zero_padding=w.zero_padding, out=(recv_x, None, recv_w, recv_m))
        if ev is not None:
            ev[2].record(stream)
        ep.combine(h, recv_x, w_d, out=out)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    flags, dropped = h.status()
    l_us = 1e3 * sum(e[0].elapsed_time(e[1]) for e in events) / steps
    d_us = 1e3 * sum(e[1].elapsed_time(e[2]) for e in events) / steps
    c_us = 1e3 * sum(e[2].elapsed_time(e[3]) for e in events) / steps
    rows = int((topk >= 0).sum())
    zeroed = R - rows if w.zero_padding else int(np.maximum(W - ne, 0).sum())
    led = ledger(T, K, H, rows, zeroed, False, True)
    led["dispatch"] += (R - rows - zeroed) * 12  # metadata of padding rows left unzeroed
    h.free()
    return {"num_worst_rows": W, "rows": R, "tail_rows": int(np.maximum(W - ne, 0).sum()),
            "dropped_rows": dropped, "status_flags": flags, "ms_per_step": ms_step,
            "tokens_per_s": T / (ms_step * 1e-3), "layout_us_device": l_us, "dispatch_us": d_us,
            "combine_us": c_us, "dispatch_bytes": led["dispatch"],
            "dispatch_frac_hbm": led["dispatch"] / (d_us * 1e3) / HBM_PEAK_GBPS,
            "combine_frac_hbm": led["combine"] / (c_us * 1e3) / HBM_PEAK_GBPS}


# ---------------------------------------------------------------------------
# device ceilings
# ---------------------------------------------------------------------------

def full_size_check(h, w, x_d, w_d, recv_x, recv_w, recv_m, out, n_sample: int = 4096) -> dict:
    """Checks the last step's outputs at full size with plain torch ops, before
    timing: for a seeded sample of tokens, every expanded row holds its token's
    x row bit for bit with its weight and (u, j); every padding row is zero
    with metadata (-1, -1) and weight 0; and the combine of the identity experts'
    outputs equals, bit for bit, the fp32 sum of w_j * x over the slots in
    order (separate multiply and add, from +0), rounded once to bf16.  Raises
    on any mismatch."""
    import numpy as np
    import torch

    T, K = w.T, w.K
    dev = recv_x.device
    dst = h.tensor("dst_row").view(T, K).long()
    rng = np.random.default_rng(12345)
    idx = torch.from_numpy(np.sort(rng.choice(T, size=min(n_sample, T), replace=False))).to(dev)
    rows = dst[idx]  # [n, K]
    acc = torch.zeros((idx.numel(), w.H), dtype=torch.float32, device=dev)
    xs = x_d[idx]
    for j in range(K):
        r = rows[:, j]
        ok = r >= 0
        rv, iv = r[ok], idx[ok]
        if not torch.equal(recv_x[rv].view(torch.int16), x_d[iv].view(torch.int16)):
            raise AssertionError(f"dispatch: expanded rows differ from x (slot {j})")
        if not torch.equal(recv_w[rv], w_d[iv, j]):
            raise AssertionError(f"dispatch: row weights differ (slot {j})")
        meta = torch.stack([iv.int(), torch.full_like(iv, j).int()], 1)
        if not torch.equal(recv_m[rv], meta):
            raise AssertionError(f"dispatch: row metadata differs (slot {j})")
        prod = w_d[idx, j:j + 1] * xs.float()  # identity experts: y = recv_x
        acc = torch.where(ok[:, None], acc + prod, acc)
    if not torch.equal(out[idx].view(torch.int16), acc.to(torch.bfloat16).view(torch.int16)):
        raise AssertionError("combine: output differs from the in-order fp32 sum rounded to bf16")
    used = torch.zeros(recv_x.shape[0], dtype=torch.bool, device=dev)
    flat = dst.reshape(-1)
    used[flat[flat >= 0]] = True
    pad = torch.nonzero(~used).reshape(-1)
    if w.zero_padding and pad.numel():
        for c in range(0, pad.numel(), 4096):
            if torch.count_nonzero(recv_x[pad[c:c + 4096]].view(torch.int16)).item():
                raise AssertionError("dispatch: a padding row is not zero")
    if pad.numel() and not (bool((recv_m[pad] == -1).all()) and bool((recv_w[pad] == 0).all())):
        raise AssertionError("dispatch: padding-row metadata is not (-1, -1) / 0")
    return {"sampled_tokens": int(idx.numel()), "rows_checked": int((rows >= 0).sum()),
            "padding_rows_checked": int(pad.numel()), "dispatch_bitwise": True, "combine_bitwise": True}


def backward_check(h, w, g_d, w_d, gy, gx, n_sample: int = 4096) -> dict:
    """The backward's outputs, as full_size_check checks the forward's: for a seeded sample
    of tokens every expanded row of the cached dispatch holds the token's gradient row bit
    for bit, and the backward combine equals the in-order fp32 sum of w_j * g (separate
    multiply and add, from +0) rounded once to bf16, bit for bit.  Raises on a mismatch."""
    import numpy as np
    import torch

    T, K = w.T, w.K
    dev = gy.device
    dst = h.tensor("dst_row").view(T, K).long()
    rng = np.random.default_rng(54321)
    idx = torch.from_numpy(np.sort(rng.choice(T, size=min(n_sample, T), replace=False))).to(dev)
    rows = dst[idx]
    acc = torch.zeros((idx.numel(), w.H), dtype=torch.float32, device=dev)
    gs = g_d[idx]
    for j in range(K):
        r = rows[:, j]
        ok = r >= 0
        if not torch.equal(gy[r[ok]].view(torch.int16), g_d[idx[ok]].view(torch.int16)):
            raise AssertionError(f"backward: cached dispatch rows differ from the gradient (slot {j})")
        acc = torch.where(ok[:, None], acc + w_d[idx, j:j + 1] * gs.float(), acc)
    if not torch.equal(gx[idx].view(torch.int16), acc.to(torch.bfloat16).view(torch.int16)):
        raise AssertionError("backward: combine differs from the in-order fp32 sum rounded to bf16")
    return {"sampled_tokens": int(idx.numel()), "rows_checked": int((rows >= 0).sum()),
            "dispatch_cached_bitwise": True, "combine_bitwise": True}


def device_ceilings(dev) -> dict:
    """Context for the roofline: the memory clock and bus width the device reports,
    and what a plain streaming copy reaches on this machine (the library's calibration copy,
    one wave per KiB with 16-byte nontemporal accesses like the row kernels; read +
    write bytes over the kernel time, median of 5 copies of 2 GiB)."""
    import ctypes

    import torch

    import combine_topk_idx_expert_amd as ep

    out = {}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        clk, bus = ctypes.c_int(), ctypes.c_int()
        # hipDeviceAttributeMemoryClockRate = 60 (kHz), hipDeviceAttributeMemoryBusWidth = 59 (bits)
        if hip.hipDeviceGetAttribute(ctypes.byref(clk), 60, dev.index or 0) == 0 and \
                hip.hipDeviceGetAttribute(ctypes.byref(bus), 59, dev.index or 0) == 0:
            out["memory_clock_khz"] = clk.value
            out["memory_bus_bits"] = bus.value
    except OSError:
        pass
    n = 2 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty(n, dtype=torch.uint8, device=dev)
    ep.debug_copy(b, a)
    torch.cuda.synchronize()
    ts = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        ep.debug_copy(b, a)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    out["copy_2GiB_GBps"] = 2.0 * n / (sorted(ts)[len(ts) // 2] * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
# per-call table
# ---------------------------------------------------------------------------

_last_min_us = [0.0]

# A spin kernel of this many shader cycles (~0.1 ms) runs before every timed call, outside
# its events: the GPU is then still busy while the host checks the call's arguments and
# launches it, so the events bracket the call alone and not the host's launch time (after a
# synchronisation the GPU would otherwise sit idle inside the first event).  It touches no
# memory, so the caches stay as the previous call left them.
HEAD_START_CYCLES = 250_000


def _head_start() -> None:
    import torch

    torch.cuda._sleep(HEAD_START_CYCLES)


def _median_us(fn, reps: int = 20, warmup: int = 3, flush=None) -> float:
    """Median of `reps` timed calls (HIP events), each timed alone between two
    synchronisations, after `warmup` untimed ones and behind a head start (see
    HEAD_START_CYCLES); the minimum is kept in _last_min_us.  `flush`, if given,
    runs before every timed call, outside the events."""
    import statistics

    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        if flush is not None:
            flush()
        _head_start()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    _last_min_us[0] = min(ts) * 1e3
    return statistics.median(ts) * 1e3


def _cache_flusher(dev):
    """Writes, then reads, a 1 GiB scratch buffer: every line of the L2s and of the
    256 MB memory-side cache is then someone else's, and clean, when the timed call
    starts."""
    import torch

    scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)

    def flush():
        scratch.fill_(1.0)
        scratch.sum()

    return flush


def calls_table() -> int:
    import statistics

    import numpy as np
    import torch

    import combine_topk_idx_expert_amd as ep
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    flush = _cache_flusher(dev)
    for name in synth.CONFIG_ORDER:
        w = synth.CONFIGS[name]
        T, K, H = w.T, w.K, w.H
        log("calls", name)
        topk = synth.gen_routing(w)
        x = synth.gen_x(w)
        wt = synth.gen_weights(w)
        topk_d = torch.from_numpy(topk).to(dev)
        x_d = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        w_d = torch.from_numpy(wt).to(dev)
        h = ep.get_layout(ep.Config(w.P, w.S, H, K, w.E, w.A), topk_d)
        R = h.total_rows
        ne, _, _ = h.counts()
        rows = int((topk >= 0).sum())
        pad = R - rows
        fp8 = w.fp8
        nb = H // 128
        r = {"workload": name, "T": T, "rows": rows, "pad": pad, "dtype": "fp8" if fp8 else "bf16"}

        def put(key, fn, nbytes):
            # each call twice: right after the previous one, and with the caches flushed first
            us = _median_us(fn)
            r[key + "_us"] = round(us, 1)
            r[key + "_min_us"] = round(_last_min_us[0], 1)
            r[key + "_GBps"] = round(nbytes / us / 1e3, 1)
            r[key + "_frac_hbm"] = round(nbytes / us / 1e3 / HBM_PEAK_GBPS, 4)
            us = _median_us(fn, flush=flush)
            r[key + "_flushed_us"] = round(us, 1)
            r[key + "_flushed_min_us"] = round(_last_min_us[0], 1)
            r[key + "_flushed_frac_hbm"] = round(nbytes / us / 1e3 / HBM_PEAK_GBPS, 4)

        torch.cuda.synchronize()
        lt = []
        for _ in range(10):
            t0 = time.perf_counter()
            ep.relayout(h, topk_d)
            lt.append(time.perf_counter() - t0)
        r["layout_us_incl_host_sync"] = round(statistics.median(lt) * 1e6, 1)
        r["layout_min_us_incl_host_sync"] = round(min(lt) * 1e6, 1)
        led = ledger(T, K, H, rows, pad, fp8, w.zero_padding)
        rx = torch.empty((R, H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev)
        sc = torch.empty((R, nb), dtype=torch.float32, device=dev) if fp8 else None
        rw = torch.empty(R, dtype=torch.float32, device=dev)
        rm = torch.empty((R, 2), dtype=torch.int32, device=dev)
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        put("dispatch", lambda: ep.dispatch(h, x_d, w_d, fp8, w.zero_padding, out=(rx, sc, rw, rm)),
            led["dispatch"])
        # fresh end to end: layout with its read-back, then dispatch (host wall clock)
        torch.cuda.synchronize()
        ft = []
        for _ in range(10):
            t0 = time.perf_counter()
            ep.relayout(h, topk_d)
            ep.dispatch(h, x_d, w_d, fp8, w.zero_padding, out=(rx, sc, rw, rm))
            torch.cuda.synchronize()
            ft.append(time.perf_counter() - t0)
        r["fresh_layout_and_dispatch_us"] = round(statistics.median(ft) * 1e6, 1)
        b = 1 if fp8 else 2
        sf = 4 * nb if fp8 else 0
        cached = T * H * 2 + 4 * T * K + rows * (H * b + sf) + (pad * (H * b + sf) if w.zero_padding else 0)
        put("cached", lambda: ep.dispatch_cached(h, x_d, fp8, w.zero_padding, out=(rx, sc)), cached)
        y = torch.empty((R, H), dtype=torch.bfloat16, device=dev).normal_()
        put("combine", lambda: ep.combine(h, y, w_d, out=out), led["combine"])
        bias = torch.empty((T, H), dtype=torch.bfloat16, device=dev).normal_()
        put("combine_bias", lambda: ep.combine(h, y, w_d, bias=bias, out=out), led["combine"] + T * H * 2)
        if fp8:
            sc8 = torch.empty((R, H // 32), dtype=torch.uint8, device=dev)
            put("dispatch_ue8m0", lambda: ep.dispatch(h, x_d, w_d, zero_padding=w.zero_padding, scales_ue8m0=True,
                                                      out=(rx, sc8, rw, rm)), led["dispatch"])
            del sc8
            codes = torch.randint(0, 256, (T, H), dtype=torch.uint8, device=dev)
            xs = torch.rand((T, nb), dtype=torch.float32, device=dev)
            pre = T * H + T * nb * 4 + 8 * T * K + (led["dispatch"] - led["dispatch_read"])
            put("dispatch_prequant",
                lambda: ep.dispatch(h, (codes, xs), w_d, zero_padding=w.zero_padding, out=(rx, sc, rw, rm)), pre)
            sc_cm = torch.empty((nb, R), dtype=torch.float32, device=dev)
            put("dispatch_col_major_scales",
                lambda: ep.dispatch(h, x_d, w_d, True, w.zero_padding, scales_col_major=True,
                                    out=(rx, sc_cm, rw, rm)), led["dispatch"])
            del codes, xs, sc_cm
        del rx, sc, rw, rm, y, bias
        torch.cuda.empty_cache()
        # fixed windows: a 1024-row bucket above the largest window
        W = int(-(-int(ne.max()) // 1024) * 1024)
        hf = ep.get_layout(ep.Config(w.P, w.S, H, K, w.E, w.A, num_worst_rows=W), topk_d)
        RF = hf.total_rows
        torch.cuda.synchronize()
        lt = []
        for _ in range(10):
            t0 = time.perf_counter()
            ep.relayout(hf, topk_d)
            lt.append(time.perf_counter() - t0)
        torch.cuda.synchronize()
        r["fixed_num_worst_rows"] = W
        r["fixed_layout_host_us"] = round(statistics.median(lt) * 1e6, 1)
        r["fixed_layout_device_us"] = round(_median_us(lambda: ep.relayout(hf, topk_d)), 1)
        rxf = torch.empty((RF, H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev)
        scf = torch.empty((RF, nb), dtype=torch.float32, device=dev) if fp8 else None
        rwf = torch.empty(RF, dtype=torch.float32, device=dev)
        rmf = torch.empty((RF, 2), dtype=torch.int32, device=dev)
        tail = int(np.maximum(W - ne, 0).sum())
        zeroed = (pad if w.zero_padding else 0) + tail
        fixed_bytes = (T * H * 2 + 8 * T * K + rows * (H * b + sf) + RF * 12 + zeroed * (H * b + sf))
        put("fixed_dispatch", lambda: ep.dispatch(hf, x_d, w_d, fp8, w.zero_padding, out=(rxf, scf, rwf, rmf)),
            fixed_bytes)
        # The fixed-window step needs no host sync, so it can be captured in one HIP graph:
        # layout + dispatch (+ combine of the identity experts' rows for bf16), timed on the host
        # clock until it has finished, eagerly and as graph replays (median of 20 each).
        def fixed_step():
            ep.relayout(hf, topk_d)
            ep.dispatch(hf, x_d, w_d, fp8, w.zero_padding, out=(rxf, scf, rwf, rmf))
            if not fp8:
                ep.combine(hf, rxf, w_d, out=out)

        def host_us(fn):
            fn()
            torch.cuda.synchronize()
            ts = []
            for _ in range(20):
                t0 = time.perf_counter()
                fn()
                torch.cuda.synchronize()
                ts.append(time.perf_counter() - t0)
            return round(statistics.median(ts) * 1e6, 1)

        r["fixed_step_eager_us"] = host_us(fixed_step)
        eager_out = (out.clone() if not fp8 else rxf.clone())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fixed_step()
        torch.cuda.synchronize()
        r["fixed_step_graph_us"] = host_us(g.replay)
        got = out if not fp8 else rxf
        if not torch.equal(got.view(torch.uint8), eager_out.view(torch.uint8)):
            raise RuntimeError(f"{name}: the graph replay of the fixed-window step differs from the eager step")
        r["fixed_step_calls"] = "relayout + dispatch" + ("" if fp8 else " + combine")
        del g, eager_out
        hf.free()
        h.free()
        del rxf, scf, rwf, rmf, out, x_d
        torch.cuda.empty_cache()
        print(json.dumps(r), flush=True)
    return 0


# ---------------------------------------------------------------------------
# overlap with compute
# ---------------------------------------------------------------------------

def overlap_table(workload: str, steps: int, tokens_per_rank: list[int]) -> int:
    """The overlap pattern at each tokens-per-rank count S (the workload scaled to S): one
    JSON line per S."""
    import synth

    for S in tokens_per_rank:
        w = synth.CONFIGS[workload]
        if S != w.S:
            w = synth.scaled(w, S=S)
        _overlap_one(w, steps)
    return 0


def _overlap_one(w, steps: int) -> None:
    import statistics

    import numpy as np
    import torch

    import combine_topk_idx_expert_amd as ep
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    T, K, H = w.T, w.K, w.H
    topk_d = torch.from_numpy(synth.gen_routing(w)).to(dev)
    x_d = torch.from_numpy(synth.gen_x(w).view(np.int16)).to(dev).view(torch.bfloat16)
    w_d = torch.from_numpy(synth.gen_weights(w)).to(dev)
    h = ep.get_layout(ep.Config(w.P, w.S, H, K, w.E, w.A), topk_d)
    R = h.total_rows
    outs = (torch.empty((R, H), dtype=torch.bfloat16, device=dev), None,
            torch.empty(R, dtype=torch.float32, device=dev), torch.empty((R, 2), dtype=torch.int32, device=dev))
    inter = 2048  # shared-expert width of the DSv3-like shape
    g = torch.Generator(device=dev).manual_seed(0)
    w1 = (torch.randn((H, 2 * inter), device=dev, generator=g) * H ** -0.5).to(torch.bfloat16)
    w2 = (torch.randn((inter, H), device=dev, generator=g) * inter ** -0.5).to(torch.bfloat16)

    def shared():
        gu = torch.matmul(x_d, w1)
        a = torch.nn.functional.silu(gu[:, :inter]) * gu[:, inter:]
        return torch.matmul(a, w2)

    def disp():
        return ep.dispatch(h, x_d, w_d, zero_padding=w.zero_padding, out=outs)

    def serial():
        shared()
        disp()

    def overlapped():
        pending = ep.dispatch(h, x_d, w_d, zero_padding=w.zero_padding, out=outs, async_with_compute_stream=True)
        shared()
        pending.wait()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(steps):
            _head_start()  # the host's launches stay outside the events: GPU time only
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e3)
        return statistics.median(ts)

    res = {}
    for _ in range(2):  # interleaved twice; the second pass is reported
        res = {"dispatch_us": timed(disp), "shared_experts_us": timed(shared), "serial_us": timed(serial),
               "overlapped_us": timed(overlapped)}
    d, sh = res["dispatch_us"], res["shared_experts_us"]
    res["hidden_frac_of_dispatch"] = (res["serial_us"] - res["overlapped_us"]) / d
    flops = 2.0 * T * H * 2 * inter + 2.0 * T * inter * H
    res["shared_experts_TFLOPs"] = flops / (sh * 1e-6) / 1e12
    out = {"workload": w.name, "P": w.P, "S": w.S, "T": T, "overlap": {k: round(v, 3) for k, v in res.items()}}
    h.free()
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------------------
# the other full-size workloads, per call
# ---------------------------------------------------------------------------

def per_config(name: str, reps: int) -> dict:
    """One full-size workload timed per call (HIP events on the launch stream, each call
    alone between two synchronisations after 3 untimed ones and behind a head start, median
    of `reps`): fresh
    dispatch (the workload's dtype), cached dispatch, combine.  A workload with cached
    iterations times each of them with its own new x (drawn on the device, resident before
    timing).  Fractions use the same ledger as the headline."""
    import statistics

    import numpy as np
    import torch

    import combine_topk_idx_expert_amd as ep
    import synth

    dev = torch.device("cuda:0")
    w = synth.CONFIGS[name]
    T, K, H = w.T, w.K, w.H
    log("per-call workload", name)
    topk = synth.gen_routing(w)
    topk_d = torch.from_numpy(topk).to(dev)
    x_d = torch.from_numpy(synth.gen_x(w).view(np.int16)).to(dev).view(torch.bfloat16)
    w_d = torch.from_numpy(synth.gen_weights(w)).to(dev)
    h = ep.get_layout(ep.Config(w.P, w.S, H, K, w.E, w.A), topk_d)
    R = h.total_rows
    rows = int((topk >= 0).sum())
    pad = R - rows
    fp8, nb = w.fp8, H // 128
    b = 1 if fp8 else 2
    sf = 4 * nb if fp8 else 0
    led = ledger(T, K, H, rows, pad, fp8, w.zero_padding)
    cached_bytes = T * H * 2 + 4 * T * K + rows * (H * b + sf) + (pad * (H * b + sf) if w.zero_padding else 0)
    rx = torch.empty((R, H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev)
    sc = torch.empty((R, nb), dtype=torch.float32, device=dev) if fp8 else None
    rw = torch.empty(R, dtype=torch.float32, device=dev)
    rm = torch.empty((R, 2), dtype=torch.int32, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    r = {"workload": name, "T": T, "rows": rows, "padding_rows": pad, "dtype": "fp8" if fp8 else "bf16"}

    def put(key, us, nbytes):
        r[key + "_us"] = us
        r[key + "_GBps"] = nbytes / us / 1e3
        r[key + "_frac_hbm"] = nbytes / us / 1e3 / HBM_PEAK_GBPS
        r[key + "_tokens_per_s"] = T / (us * 1e-6)
        r[key + "_bytes"] = nbytes

    put("dispatch", _median_us(lambda: ep.dispatch(h, x_d, w_d, fp8, w.zero_padding, out=(rx, sc, rw, rm)), reps),
        led["dispatch"])
    if fp8:  # UE8M0 scales: H/32 exponent bytes per row, the same bytes as H/128 fp32 scales
        sc8 = torch.empty((R, H // 32), dtype=torch.uint8, device=dev)
        put("dispatch_ue8m0", _median_us(lambda: ep.dispatch(h, x_d, w_d, zero_padding=w.zero_padding,
                                                              scales_ue8m0=True, out=(rx, sc8, rw, rm)), reps),
            led["dispatch"])
        del sc8
    if w.cached_iters:
        # new x for every iteration, drawn on the device with a seeded generator
        xs = []
        for it in range(1, w.cached_iters + 1):
            gen = torch.Generator(device=dev).manual_seed(1000 + it)
            xs.append(torch.randn((T, H), generator=gen, device=dev).to(torch.bfloat16))
        for xi in xs[:3]:  # untimed
            ep.dispatch_cached(h, xi, fp8, w.zero_padding, out=(rx, sc))
        torch.cuda.synchronize()
        ts = []
        for xi in xs:
            _head_start()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            ep.dispatch_cached(h, xi, fp8, w.zero_padding, out=(rx, sc))
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        put("cached", statistics.median(ts), cached_bytes)
        r["cached_iterations"] = len(ts)
        r["cached_us_each"] = [round(t, 1) for t in ts]
        del xs
    else:
        put("cached", _median_us(lambda: ep.dispatch_cached(h, x_d, fp8, w.zero_padding, out=(rx, sc)), reps),
            cached_bytes)
    if fp8:  # expert outputs in bf16 for the combine
        gen = torch.Generator(device=dev).manual_seed(77)
        y = torch.randn((R, H), generator=gen, device=dev).to(torch.bfloat16)
    else:
        y = rx  # identity experts
    put("combine", _median_us(lambda: ep.combine(h, y, w_d, out=out), reps), led["combine"])
    h.free()
    del rx, sc, rw, rm, out, y, x_d
    torch.cuda.empty_cache()
    return {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}


# ---------------------------------------------------------------------------
# main
# ---------------------------------------------------------------------------

def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-fixed", action="store_true", help="skip the fixed-length-window leg")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-call legs of the other workloads")
    ap.add_argument("--calls", action="store_true", help="per-call table over all workloads")
    ap.add_argument("--overlap", action="store_true", help="dispatch overlapped with shared experts")
    ap.add_argument("--overlap-tokens", default="128,512,4096",
                    help="--overlap: tokens per rank to run at (the workload scaled), comma-separated")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="first run a plain torch copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only (asked for --gpus {args.gpus}); the P "
              "expert-parallel ranks are virtual windows in one GPU's HBM.", file=sys.stderr)
        return 2
    if args.calls:
        return calls_table()
    if args.overlap:
        wl = args.workload if args.workload != DEFAULT_WORKLOAD else "dsv3-bf16-p8-s4096-e256-k8-h7168"
        return overlap_table(wl, args.steps, [int(v) for v in args.overlap_tokens.split(",")])

    import numpy as np
    import torch

    import combine_topk_idx_expert_amd as ep
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.CONFIGS[args.workload]
    T, K, H = w.T, w.K, w.H
    bwd = w.backward

    if args.copy_calib_mib:
        n = args.copy_calib_mib << 20
        a_ = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b_ = torch.empty(n, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        b_.copy_(a_)  # the plain copy kernel the hardware counters are scaled against
        torch.cuda.synchronize()
        del a_, b_
    log("generating inputs", w.name)
    topk = synth.gen_routing(w)
    x = synth.gen_x(w)
    wt = synth.gen_weights(w)
    g = synth.gen_grad_out(w) if bwd else None
    topk_d = torch.from_numpy(topk).to(dev)
    x_d = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    w_d = torch.from_numpy(wt).to(dev)
    g_d = torch.from_numpy(g.view(np.int16)).to(dev).view(torch.bfloat16) if bwd else None

    h = ep.get_layout(ep.Config(w.P, w.S, H, K, w.E, w.A), topk_d)
    R = h.total_rows
    _, num_recv, _ = h.counts()
    rows_valid = int((topk >= 0).sum())
    pad = R - rows_valid
    recv_x = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
    recv_w = torch.empty(R, dtype=torch.float32, device=dev)
    recv_m = torch.empty((R, 2), dtype=torch.int32, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    gy = torch.empty((R, H), dtype=torch.bfloat16, device=dev) if bwd else None
    gx = torch.empty((T, H), dtype=torch.bfloat16, device=dev) if bwd else None
    stream = torch.cuda.current_stream(dev)
    n_ev = 5 if bwd else 3

    def step(ev=None):
        ep.relayout(h, topk_d)
        if ev is not None:
            ev[0].record(stream)
        ep.dispatch(h, x_d, w_d, fp8=False, zero_padding=w.zero_padding, out=(recv_x, None, recv_w, recv_m))
        if ev is not None:
            ev[1].record(stream)
        ep.combine(h, recv_x, w_d, out=out)  # identity experts: y = recv_x
        if ev is not None:
            ev[2].record(stream)
        if bwd:  # backward with the same handle: dispatch of the gradient, then its combine
            ep.dispatch_cached(h, g_d, fp8=False, zero_padding=w.zero_padding, out=(gy, None))
            if ev is not None:
                ev[3].record(stream)
            ep.combine(h, gy, w_d, out=gx)
            if ev is not None:
                ev[4].record(stream)

    log("warmup", args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    def checks():
        c = full_size_check(h, w, x_d, w_d, recv_x, recv_w, recv_m, out)
        if bwd:
            c["backward"] = backward_check(h, w, g_d, w_d, gy, gx)
        torch.cuda.synchronize()
        return c

    check = None
    if args.warmup > 0:  # otherwise checked after the timed steps
        log("full-size check of the last warm-up step's outputs")
        check = checks()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    log("timing", args.steps, "steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    if check is None:
        log("full-size check of the last timed step's outputs")
        check = checks()

    def avg_us(i0, i1):
        v = [1e3 * e[i0].elapsed_time(e[i1]) for e in events]
        return sum(v) / len(v), sorted(v)[len(v) // 2], min(v)

    ms_step = elapsed * 1e3 / args.steps
    led = ledger(T, K, H, rows_valid, pad, False, w.zero_padding)
    cached_bytes = T * H * 2 + 4 * T * K + rows_valid * H * 2 + (pad * H * 2 if w.zero_padding else 0)
    d_us, d_med, d_min = avg_us(0, 1)
    c_us, c_med, c_min = avg_us(1, 2)
    launches = {"dispatch": (d_us, led["dispatch"]), "combine": (c_us, led["combine"])}
    calls = {"dispatch_us": d_us, "dispatch_us_median": d_med, "dispatch_us_min": d_min,
             "combine_us": c_us, "combine_us_median": c_med, "combine_us_min": c_min}
    kernel_us = d_us + c_us
    if bwd:
        dc_us, dc_med, dc_min = avg_us(2, 3)
        cb_us, cb_med, cb_min = avg_us(3, 4)
        launches["dispatch_cached_grad"] = (dc_us, cached_bytes)
        launches["combine_grad"] = (cb_us, led["combine"])
        calls.update({"dispatch_cached_grad_us": dc_us, "dispatch_cached_grad_us_median": dc_med,
                      "dispatch_cached_grad_us_min": dc_min, "combine_grad_us": cb_us,
                      "combine_grad_us_median": cb_med, "combine_grad_us_min": cb_min})
        kernel_us += dc_us + cb_us
    for k, (us, nbytes) in launches.items():
        calls[k + "_bytes"] = nbytes
        calls[k + "_GBps"] = nbytes / (us * 1e3)
        calls[k + "_frac_hbm"] = nbytes / (us * 1e3) / HBM_PEAK_GBPS
        calls[k + "_tokens_per_s"] = T / (us * 1e-6)
    calls["layout_us_incl_host_sync"] = ms_step * 1e3 - kernel_us
    calls["page_style_payload_GBps_dispatch"] = page_style_payload(int(num_recv.sum()), T, K, H, False) / (d_us * 1e3)
    calls["expanded_rows"] = R
    calls["padding_rows"] = pad

    # The dominant kernel: the kernel function with the largest share of the step's kernel
    # time (dispatch_kernel runs the fresh and the cached dispatch, combine the forward and
    # the backward combine).  Its roofline point is its algorithmic bytes per launch over its
    # average launch duration, both averaged over its launches in the step.
    fam = {"dispatch": [k for k in launches if k.startswith("dispatch")],
           "combine": [k for k in launches if k.startswith("combine")]}
    fam_us = {f: sum(launches[k][0] for k in ks) for f, ks in fam.items()}
    dominant = max(fam_us, key=fam_us.get)
    ks = fam[dominant]
    dom_us = fam_us[dominant] / len(ks)
    dom_bytes = sum(launches[k][1] for k in ks) / len(ks)
    achieved = dom_bytes / (dom_us * 1e3)
    combine_kernel = "combine_lds_kernel" if (K <= 8 and H <= 4096) else "combine_kernel"
    dom_kernel = "dispatch_kernel" if dominant == "dispatch" else combine_kernel
    traffic = traffic_from_profiles(dom_kernel, w.name)
    step_desc = "relayout + dispatch(bf16) + identity + combine(fp32 acc)"
    if bwd:
        step_desc += " + dispatch_cached(grad) + combine(grad)"

    result = {
        "metric": METRIC,
        "value": T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "P": w.P, "S": w.S, "T": T, "E": w.E, "K": K, "H": H, "A": w.A,
                   "routing": w.routing, "zero_padding": w.zero_padding, "seed": w.seed, "step": step_desc},
        "roofline": {"bound": "hbm", "kernel": dom_kernel, "launches": ks, "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_us": dom_us,
                     "share_of_step_kernel_time": fam_us[dominant] / kernel_us},
        "calls": calls,
        "parity": check,
    }
    result["device"] = device_ceilings(dev)

    if not args.no_fixed:
        result["fixed_windows"] = fixed_leg(ep, h, w, topk, topk_d, x_d, w_d, out, args.steps, args.warmup)
    h.free()
    del recv_x, recv_w, recv_m, out, gy, gx, x_d, g_d
    torch.cuda.empty_cache()

    if not args.no_configs:
        result["configs"] = [per_config(n, 20) for n in PER_CONFIG if n != w.name]

    if not args.no_cpu:
        nt, _ = host_threads()
        log(f"cpu baseline (oracle, 1 and {nt} threads)")
        result["cpu_baseline"] = cpu_baseline(w, topk, x, g, wt, nt)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
