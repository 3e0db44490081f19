"""Pins of the CPU oracle against things other than itself.

Each test ties one oracle function to a value printed on the pages, a closed
form, an invariant, a library routine (numpy stable sort, torch's float8 and
bfloat16 casts) or brute force on tiny inputs, chosen so that a plausible slip
(dropped term, wrong sign or index, transposed operand) fails at least one.
CPU only.
"""

from math import comb

import numpy as np
import pytest
import torch

import oracle
import synth

# ---------------------------------------------------------------------------
# helpers written independently of oracle.c
# ---------------------------------------------------------------------------


def finite_e4m3_table():
    """(codes, values) of the 254 finite E4M3FN codes, from the bit-field definition."""
    codes, vals = [], []
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            continue
        v = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        codes.append(c)
        vals.append(-v if s else v)
    return np.array(codes, np.uint8), np.array(vals, np.float64)


def brute_force_e4m3(q: np.ndarray) -> np.ndarray:
    """Nearest finite code by exhaustive search, ties to the even mantissa; |q| > 464 -> NaN."""
    codes, vals = finite_e4m3_table()
    out = np.empty(q.shape, np.uint8)
    for i, x in enumerate(q.astype(np.float64)):
        if abs(x) > 464.0:
            out[i] = 0xFF if x < 0 else 0x7F
            continue
        # same-sign candidates only, so +-0 keep their sign
        neg = np.signbit(x)
        sel = (codes >= 0x80) if neg else (codes < 0x80)
        cc, vv = codes[sel], vals[sel]
        d = np.abs(vv - x)
        best = np.flatnonzero(d == d.min())
        if len(best) > 1:
            best = [b for b in best if (cc[b] & 1) == 0]
        out[i] = cc[best[0]]
    return out


def bf16_bits_to_f64(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def torch_bf16_bits(f: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(f, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def small_workload(P=4, S=64, E=16, K=2, H=512, A=16, routing="uniform", seed=0, zero_padding=True):
    return synth.Workload("t", P, S, E, K, H, A, zero_padding, routing, seed=seed)


# ---------------------------------------------------------------------------
# scalar encodings
# ---------------------------------------------------------------------------


def test_e4m3_encode_matches_brute_force_search():
    rng = np.random.default_rng(1)
    codes, vals = finite_e4m3_table()
    pos = np.sort(vals[vals > 0])
    mids = (pos[1:] + pos[:-1]) / 2
    q = np.concatenate([
        rng.uniform(-464, 464, 3000), rng.normal(0, 1, 2000) * 2.0 ** rng.integers(-12, 8, 2000),
        mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1000), vals, [0.0, -0.0, 464.0, 448.0, 465.0, -470.0],
        np.arange(0, 20) * 2.0 ** -10,  # subnormal grid and its midpoints
    ]).astype(np.float32)
    np.testing.assert_array_equal(oracle.e4m3_encode(q), brute_force_e4m3(q))


def test_e4m3_encode_matches_torch_cast_on_dense_sample():
    # every 97th fp32 pattern in [0, 464] plus +-3 ulp around every midpoint
    pats = np.arange(0, 0x43E80001, 97, dtype=np.uint32)
    _, vals = finite_e4m3_table()
    pos = np.sort(vals[vals > 0]).astype(np.float32)
    mids = ((pos[1:].astype(np.float64) + pos[:-1]) / 2).astype(np.float32).view(np.uint32)
    near = (mids[:, None].astype(np.int64) + np.arange(-3, 4)[None, :]).ravel().astype(np.uint32)
    q = np.concatenate([pats, near]).view(np.float32)
    q = np.concatenate([q, -q])
    ref = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.e4m3_encode(q), ref)


def test_e4m3_decode_matches_torch():
    c = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = oracle.e4m3_decode(c)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok].view(np.uint32), ref[ok].view(np.uint32))


def test_bf16_round_matches_torch_including_ties():
    rng = np.random.default_rng(2)
    r = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    ties = (r & 0xFFFF0000) | 0x8000  # exact halfway cases
    near = np.concatenate([ties - 1, ties + 1])
    f = np.concatenate([r, ties, near]).view(np.float32)
    f = f[np.isfinite(f)]
    f = np.concatenate([f, np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, 1e-40], np.float32)])
    np.testing.assert_array_equal(oracle.bf16_round(f), torch_bf16_bits(f))


# ---------------------------------------------------------------------------
# layout
# ---------------------------------------------------------------------------


def brute_force_layout(P, S, E, K, A, topk):
    """Definitions written out with direct counts (quadratic, tiny inputs only)."""
    T, El = P * S, E // P
    itr = np.zeros((T, P), np.uint8)
    for u in range(T):
        for j in range(K):
            if topk[u, j] >= 0:
                itr[u, topk[u, j] // El] = 1
    ntpr = np.array([[itr[s * S:(s + 1) * S, d].sum() for d in range(P)] for s in range(P)])
    ntpe = np.array([[(topk[s * S:(s + 1) * S] == e).sum() for e in range(E)] for s in range(P)])
    send_head = np.full((T, P), -1)
    for u in range(T):
        for d in range(P):
            if itr[u, d]:
                send_head[u, d] = itr[:u, d].sum()  # #{u' < u : itr[u'][d]}
    return itr, ntpr, ntpe, send_head


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_layout_tiny_brute_force(seed):
    w = synth.CONFIGS["tiny-p4-s64-e16-k2-h512"] if seed == 0 else small_workload(seed=seed)
    topk = synth.gen_routing(w)
    if seed == 2:  # unused slots and duplicate experts inside a token
        topk = topk.copy()
        topk[::7, 1] = -1
        topk[3::11, 1] = topk[3::11, 0]
    lay = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk)
    itr, ntpr, ntpe, send_head = brute_force_layout(w.P, w.S, w.E, w.K, w.A, topk)
    np.testing.assert_array_equal(lay.is_token_in_rank, itr)
    np.testing.assert_array_equal(lay.num_tokens_per_rank, ntpr)
    np.testing.assert_array_equal(lay.num_tokens_per_expert, ntpe)
    np.testing.assert_array_equal(lay.rank_prefix_matrix, np.cumsum(ntpr, axis=0))
    np.testing.assert_array_equal(lay.num_recv_tokens, ntpr.sum(0))
    np.testing.assert_array_equal(lay.send_head, send_head)
    # recv_src_idx is the inverse of send_head: recv_src_idx[d][send_head[u][d]] = t(u)
    for u in range(w.T):
        for d in range(w.P):
            if send_head[u, d] >= 0:
                assert lay.recv_src_idx[lay.recv_src_base[d] + send_head[u, d]] == u % w.S
    # the source rank of a received token is the s with rank_prefix[s-1][d] <= i < rank_prefix[s][d]
    for d in range(w.P):
        for i in range(int(lay.num_recv_tokens[d])):
            s = int(np.searchsorted(lay.rank_prefix_matrix[:, d], i, side="right"))
            u = s * w.S + int(lay.recv_src_idx[lay.recv_src_base[d] + i])
            assert send_head[u, d] == i


def test_layout_dst_slot_is_stable_sort_by_expert():
    """dst_slot equals numpy's stable argsort of the flattened (u, j) stream by expert,
    and the tutorial's deterministic key expert * 1e10 + src_token_global_idx."""
    for w in [synth.CONFIGS["tiny-p4-s64-e16-k2-h512"], small_workload(P=8, S=300, E=64, K=6, A=8, seed=5),
              small_workload(P=8, S=96, E=32, K=4, A=1, routing="zipf", seed=3)]:
        topk = synth.gen_routing(w)
        if w.K > 2:
            topk = topk.copy()
            topk[::5, -1] = -1
            topk[1::9, 2] = topk[1::9, 1]  # duplicates
        lay = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk)
        El = w.E // w.P
        flat = topk.ravel()
        valid = np.flatnonzero(flat >= 0)
        keys = flat[valid]
        order = np.argsort(keys, kind="stable")
        sk = keys[order]
        rank_in_expert = np.empty(len(keys), np.int64)
        rank_in_expert[order] = np.arange(len(keys)) - np.searchsorted(sk, sk, side="left")
        expect = np.full(flat.shape, -1, np.int64)
        expect[valid] = lay.expert_offset[keys // El, keys % El] + rank_in_expert
        np.testing.assert_array_equal(lay.dst_slot.ravel(), expect)
        # page key (exact in float64: 256 * 1e10 < 2**53); within-token ties keep slot order
        u = valid // w.K
        page_key = keys.astype(np.float64) * 1e10 + u
        np.testing.assert_array_equal(np.argsort(page_key, kind="stable"), order)


@pytest.mark.parametrize("A", [1, 16, 128])
def test_num_expanded_closed_form(A):
    w = small_workload(P=8, S=512, E=64, K=4, A=A, routing="zipf", seed=7)
    topk = synth.gen_routing(w)
    lay = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk)
    n = np.bincount(topk[topk >= 0], minlength=w.E)
    np.testing.assert_array_equal(lay.num_tokens_per_expert_total, n)
    padded = -(-n // A) * A
    El = w.E // w.P
    np.testing.assert_array_equal(lay.num_expanded, padded.reshape(w.P, El).sum(1))
    assert np.all(lay.expert_offset % A == 0)
    np.testing.assert_array_equal(lay.window_row_base, np.concatenate([[0], np.cumsum(lay.num_expanded)]))
    # dst_slot is a bijection from valid slots onto the non-padding rows
    rows = lay.window_row_base[topk[topk >= 0] // El] + lay.dst_slot[topk >= 0]
    assert len(np.unique(rows)) == len(rows)
    e_of = np.repeat(np.arange(w.E), n)
    starts = lay.window_row_base[e_of // El] + lay.expert_offset[e_of // El, e_of % El]
    within = np.concatenate([np.arange(c) for c in n]) if len(n) else np.array([])
    np.testing.assert_array_equal(np.sort(rows), np.sort(starts + within))


def test_distinct_ranks_with_replacement_matches_page_formula():
    """Tutorial section 1.3: expected distinct ranks per token R(1-(1-1/R)^k) for independent slots."""
    rng = np.random.default_rng(11)
    for R, E, K in [(8, 256, 6), (8, 256, 8), (32, 256, 8), (128, 256, 6)]:
        T = R * (40000 // R)
        topk = rng.integers(0, E, (T, K)).astype(np.int64)  # duplicates allowed -> dedup exercised
        lay = oracle.layout(R, T // R, E, K, 1, topk)
        cnt = lay.is_token_in_rank.sum(1).astype(np.float64)
        expect = R * (1 - (1 - 1 / R) ** K)
        assert abs(cnt.mean() - expect) < 5 * cnt.std() / np.sqrt(T) + 1e-9, (R, K, cnt.mean(), expect)


def test_distinct_ranks_without_replacement_exact_mean():
    """Distinct experts (the workloads' routing): mean distinct ranks is R(1 - C(E-E_l,K)/C(E,K))."""
    for w in [synth.CONFIGS["dsv3-bf16-p8-s4096-e256-k8-h7168"], synth.CONFIGS["tiny-p4-s64-e16-k2-h512"]]:
        topk = synth.gen_routing(w)
        lay = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk)
        cnt = lay.is_token_in_rank.sum(1).astype(np.float64)
        El = w.E // w.P
        exact = w.P * (1 - comb(w.E - El, w.K) / comb(w.E, w.K))
        assert abs(cnt.mean() - exact) < 5 * cnt.std() / np.sqrt(w.T) + 1e-9
        page = w.P * (1 - (1 - 1 / w.P) ** w.K)
        if w.T > 1000:  # the with-replacement formula is within 1% for 8 ranks x top-8
            assert abs(cnt.mean() - page) / page < 0.01


def test_local_experts_and_ledger_values_from_pages(golden):
    g = golden["local_experts"]
    assert g["num_experts"] // 8 == g["ep8_local"] and g["num_experts"] // 128 == g["ep128_local"]
    # Dispatch one token with K=6 distinct experts at H=7168: the oracle writes exactly K rows
    # of H*b payload bytes per token; combine reads K bf16 rows plus K fp32 weights.
    led = golden["byte_ledger"]
    K, H = led["k"], led["hidden"]
    P, E = 8, 256
    topk = np.array([[3, 40, 77, 150, 151, 250]] + [[-1] * K] * (P - 1), np.int64)
    x = synth.gen_bf16_rows(0, 1, P, H)
    w = np.full((P, K), 1.0 / K, np.float32)
    lay = oracle.layout(P, 1, E, K, 1, topk)
    for fp8, fill, b, key in [(True, 0x7F, 1, "fp8_dispatch_bytes_per_token"),
                              (False, 0xFFFF, 2, "bf16_dispatch_bytes_per_token")]:
        rx, sc, rw, meta = oracle.dispatch(lay, H, x, w, fp8, False, fill=fill)
        rows_of_token0 = np.flatnonzero(meta[:, 0] == 0)
        payload = rx[rows_of_token0]
        assert payload.size * b == led[key]
        assert not np.any(payload == fill)  # every byte of those rows was written
        if fp8:
            assert sc.shape[1] * 4 // 2 == golden["fp8_scale_packs"]["num_sf_packs_int16"]
    combine_bytes = len(rows_of_token0) * H * 2 + K * 4
    assert combine_bytes == led["bf16_combine_bytes_per_token_with_weights"]


def test_routing_errors_and_unused_slots():
    topk = np.array([[0, 1], [2, -1], [-1, -1], [3, 3]], np.int64)
    lay = oracle.layout(2, 2, 4, 2, 2, topk)
    np.testing.assert_array_equal(lay.dst_slot, [[0, 2], [0, -1], [-1, -1], [2, 3]])
    np.testing.assert_array_equal(lay.is_token_in_rank, [[1, 0], [0, 1], [0, 0], [0, 1]])
    np.testing.assert_array_equal(lay.num_expanded, [4, 4])
    for bad in (4, -2, 1 << 40):
        t2 = topk.copy()
        t2[1, 1] = bad
        with pytest.raises(oracle.OracleError) as ei:
            oracle.layout(2, 2, 4, 2, 2, t2)
        assert ei.value.status == oracle.ERR_ROUTING


def test_symmetric_windows_only_move_bases():
    w = small_workload(P=8, S=256, E=32, K=4, A=8, routing="zipf", seed=4)
    topk = synth.gen_routing(w)
    a = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk)
    b = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk, symmetric=True)
    for f in ("dst_slot", "send_head", "expert_offset", "num_expanded", "recv_src_idx", "rank_prefix_matrix"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    np.testing.assert_array_equal(b.window_row_base, np.arange(w.P + 1) * a.num_expanded.max())


@pytest.mark.parametrize("shape", [(1, 50, 4, 3, 4), (4, 0, 8, 2, 4), (3, 17, 3, 1, 1), (4, 33, 64, 8, 5)])
def test_layout_edge_shapes(shape):
    P, S, E, K, A = shape
    rng = np.random.default_rng(sum(shape))
    topk = np.stack([rng.permutation(E)[:K] for _ in range(P * S)]) if P * S else np.zeros((0, K), np.int64)
    lay = oracle.layout(P, S, E, K, A, topk)
    itr, ntpr, ntpe, send_head = brute_force_layout(P, S, E, K, A, topk.astype(np.int64))
    np.testing.assert_array_equal(lay.is_token_in_rank, itr)
    np.testing.assert_array_equal(lay.send_head, send_head)
    n = np.bincount(topk[topk >= 0].ravel(), minlength=E)
    assert lay.total_rows == int((-(-n // A) * A).sum())


# ---------------------------------------------------------------------------
# dispatch
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("zero_padding", [True, False])
def test_dispatch_bf16_rows_are_token_copies(zero_padding):
    w = small_workload(P=4, S=64, E=16, K=3, H=256, A=16, seed=9)
    topk = synth.gen_routing(w).copy()
    topk[::13, 2] = -1
    x = synth.gen_bf16_rows(1, 1, w.T, w.H)
    wt = synth.gen_weights(w)
    lay = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk)
    rx, _, rw, meta = oracle.dispatch(lay, w.H, x, wt, False, zero_padding, fill=0xFFFF)
    El = w.E // w.P
    covered = np.zeros(lay.total_rows, bool)
    for u in range(w.T):
        for j in range(w.K):
            e = topk[u, j]
            if e < 0:
                continue
            r = lay.window_row_base[e // El] + lay.dst_slot[u, j]
            np.testing.assert_array_equal(rx[r], x[u])
            assert rw[r] == wt[u, j] and tuple(meta[r]) == (u, j)
            covered[r] = True
    pad = ~covered
    assert np.all(meta[pad] == -1) and np.all(rw[pad] == 0)
    assert np.all(rx[pad] == (0 if zero_padding else 0xFFFF))
    n = np.bincount(topk[topk >= 0], minlength=w.E)
    assert pad.sum() == int((-(-n // w.A) * w.A - n).sum())


def test_quantize_row_scale_codes_and_error_bound():
    rng = np.random.default_rng(3)
    H = 1024
    x = synth.gen_bf16_rows(2, 1, 4, H)
    x[1, 128:256] = 0  # amax == 0 block
    x[1, 130] = 0x8000  # -0.0 inside it
    x[2, 256:384] = torch_bf16_bits(rng.normal(0, 1e-3, 128).astype(np.float32))
    x[3, 0:128] = torch_bf16_bits((rng.normal(0, 1, 128) * 2.0 ** -120).astype(np.float32))  # tiny
    # bf16 subnormal inputs (exponent field 0): an all-subnormal block, and one normal value
    # among subnormals, so that the scale and most codes fall in the subnormal ranges
    sub = np.zeros((1, H), np.uint16)
    sub[0, :256] = (rng.integers(0, 2, 256) << 15).astype(np.uint16) | rng.integers(1, 0x80, 256).astype(np.uint16)
    sub[0, 200] = 0x3F80
    x = np.vstack([x, sub])
    for r in range(5):
        codes, scales = oracle.quantize_row(x[r])
        xf = bf16_bits_to_f64(x[r]).astype(np.float32)
        for b in range(H // 128):
            blk = xf[128 * b:128 * (b + 1)]
            amax = np.abs(blk).max()
            assert scales[b].view(np.uint32) == (np.float32(amax) / np.float32(448.0)).view(np.uint32)
            cb = codes[128 * b:128 * (b + 1)]
            if amax == 0:
                np.testing.assert_array_equal(cb, np.where(np.signbit(blk), 0x80, 0x00))
                continue
            q = blk / scales[b]  # numpy float32 division (IEEE)
            np.testing.assert_array_equal(cb, brute_force_e4m3(q))
            i = int(np.argmax(np.abs(blk)))
            assert cb[i] == (0xFE if blk[i] < 0 else 0x7E)
            deq = oracle.e4m3_decode(cb).astype(np.float64) * np.float64(scales[b])
            err = np.abs(deq - blk.astype(np.float64))
            normal = np.abs(q) >= 2.0 ** -6
            assert np.all(err[normal] <= (2.0 ** -4 + 2.0 ** -20) * np.abs(blk.astype(np.float64))[normal])
            assert np.all(err[~normal] <= (2.0 ** -10 + 2.0 ** -30) * scales[b])


def test_quantize_row_non_finite_blocks():
    """Blocks holding NaN or +-Inf follow the stated rule, written here from numpy alone: the
    block maximum is numpy's max of |x| (NaN wins over everything), the scale is that
    maximum / 448 in fp32 with a NaN maximum giving the quiet NaN 0x7FC00000, and each code
    is the E4M3 code of x / scale with every NaN quotient written 0x7F.  Finite blocks of the
    same rows are unaffected.  Also the batched form equals the per-row form."""
    rng = np.random.default_rng(11)
    H = 768
    x = synth.gen_bf16_rows(4, 1, 6, H)
    NAN_P, NAN_N, NAN_PAYLOAD, INF_P, INF_N = 0x7FC0, 0xFFC0, 0x7F81, 0x7F80, 0xFF80
    x[0, 5] = NAN_P                     # one positive NaN in block 0
    x[1, 128 + 7] = NAN_N               # one negative NaN in block 1
    x[1, 128 + 9] = INF_N
    x[2, 256:384] = 0
    x[2, 300] = NAN_PAYLOAD             # NaN among zeros, signalling payload
    x[3, 384 + 1] = INF_P               # +Inf among finite values
    x[3, 384 + 2] = INF_N               # and -Inf
    x[4, 512:640] = INF_N               # a block of -Inf only
    x[5, 640 + rng.integers(0, 128)] = INF_P
    x[5, 0] = 0x8000
    for r in range(x.shape[0]):
        codes, scales = oracle.quantize_row(x[r])
        xf = bf16_bits_to_f64(x[r]).astype(np.float32)
        for b in range(H // 128):
            blk = xf[128 * b:128 * (b + 1)]
            with np.errstate(invalid="ignore", divide="ignore"):
                amax = np.abs(blk).max()  # numpy's max propagates NaN
                exp_scale = np.float32(np.nan) if np.isnan(amax) else np.float32(amax) / np.float32(448.0)
                if np.isnan(amax):
                    assert scales[b].view(np.uint32) == 0x7FC00000, (r, b)
                else:
                    assert scales[b].view(np.uint32) == exp_scale.view(np.uint32), (r, b)
                cb = codes[128 * b:128 * (b + 1)]
                if amax == 0:
                    np.testing.assert_array_equal(cb, np.where(np.signbit(blk), 0x80, 0x00))
                    continue
                q = blk / exp_scale
            nanq = np.isnan(q)
            exp = np.full(128, 0x7F, np.uint8)
            if (~nanq).any():
                exp[~nanq] = brute_force_e4m3(q[~nanq])
            np.testing.assert_array_equal(cb, exp, err_msg=f"row {r} block {b}")
            if not np.isfinite(amax):
                # the rule in words: NaN blocks are all 0x7F; Inf blocks give signed zeros for
                # finite x and 0x7F for the infinities
                fin = np.isfinite(blk)
                if np.isnan(amax):
                    assert (cb == 0x7F).all()
                else:
                    np.testing.assert_array_equal(cb[fin], np.where(np.signbit(blk[fin]), 0x80, 0x00))
                    assert (cb[~fin] == 0x7F).all()
    bc, bs = oracle.quantize_rows(x, H)
    for r in range(x.shape[0]):
        c1, s1 = oracle.quantize_row(x[r])
        np.testing.assert_array_equal(bc[r], c1)
        np.testing.assert_array_equal(bs[r].view(np.uint32), s1.view(np.uint32))
    bc2, bs2 = oracle.quantize_rows(x, H, 2, 5)
    np.testing.assert_array_equal(bc2, bc[2:5])
    np.testing.assert_array_equal(bs2.view(np.uint32), bs[2:5].view(np.uint32))


def _ue8m0_rows(rng, H):
    """bf16 rows whose 32-channel blocks exercise the exponent choice: N(0,1) values, blocks
    whose maximum is exactly 448 * 2^k (the bound met with equality), a maximum just above
    1.75 * 2^E (mantissa 0x61: forces the next power of two), maxima of 1.0 * 2^E, all-zero
    and signed-zero blocks, bf16 subnormals, the smallest normal and the largest finite bf16,
    values spread over many binades, and NaN / Inf blocks."""
    rows = []
    for r in range(12):
        x = synth.gen_bf16_rows(50 + r, 1, 1, H)[0].copy()
        for b in range(H // 32):
            blk = x[32 * b:32 * (b + 1)]
            kind = (r + b) % 12
            sign = (rng.integers(0, 2, 32) << 15).astype(np.uint16)
            if kind == 1:    # maximum exactly 448 * 2^k: 1.75 * 2^(8+k), bf16 0x3F60 + ((8+k) << 7)
                k = int(rng.integers(-20, 20))
                blk[:] = sign | rng.integers(0x3000, 0x3F00, 32).astype(np.uint16)
                blk[rng.integers(0, 32)] = (((127 + 8 + k) << 7) | 0x60) | int(sign[0])
            elif kind == 2:  # maximum 1.7578125 * 2^E (mantissa 0x61)
                e = int(rng.integers(100, 140))
                blk[:] = sign | rng.integers(0x3000, 0x3F00, 32).astype(np.uint16)
                blk[rng.integers(0, 32)] = (e << 7) | 0x61
            elif kind == 3:  # maximum 2^E exactly
                e = int(rng.integers(90, 160))
                blk[:] = sign | rng.integers(0x2000, 0x2F00, 32).astype(np.uint16)
                blk[rng.integers(0, 32)] = e << 7
            elif kind == 4:  # zeros of both signs
                blk[:] = sign
            elif kind == 5:  # bf16 subnormals
                blk[:] = sign | rng.integers(1, 0x80, 32).astype(np.uint16)
            elif kind == 6:  # smallest normal among subnormals
                blk[:] = sign | rng.integers(0, 0x80, 32).astype(np.uint16)
                blk[rng.integers(0, 32)] = 0x0080
            elif kind == 7:  # the largest finite bf16
                blk[:] = sign | rng.integers(0x7000, 0x7F00, 32).astype(np.uint16)
                blk[rng.integers(0, 32)] = 0x7F7F | int(sign[0])
            elif kind == 8:  # many binades
                blk[:] = sign | (rng.integers(1, 254, 32) << 7).astype(np.uint16) | rng.integers(0, 0x80, 32).astype(np.uint16)
            elif kind == 9:  # a NaN
                blk[rng.integers(0, 32)] = int(rng.choice([0x7FC0, 0xFFC1]))
            elif kind == 10:  # an infinity
                blk[rng.integers(0, 32)] = int(rng.choice([0x7F80, 0xFF80]))
            x[32 * b:32 * (b + 1)] = blk
        rows.append(x)
    return np.stack(rows)


def test_quantize_row_ue8m0_exponent_codes_and_packs(golden):
    """UE8M0 quantisation against the stated rule, written here in plain Python.
    Per 32-channel block, for a finite maximum amax: the exponent byte e gives a scale
    2^(e-127) with 448 * 2^(e-127) >= amax, and halving it would push amax past 448 (or
    e = 0); the same byte from frexp; every code is the nearest E4M3 value of x / 2^(e-127)
    (exact quotient, brute force), never a NaN code.  Non-finite blocks: byte 0xFF and the
    codes of the non-finite rule.  The bytes, viewed as int16 packs, number ceil(H/64) per
    token (the page's 112 at hidden 7168), two UE8M0 per pack, block 2i in the low byte."""
    import math

    rng = np.random.default_rng(21)
    H = golden["ue8m0_scale_packs"]["hidden"]
    x = _ue8m0_rows(rng, H)
    seen_eq = seen_up = False
    for r in range(x.shape[0]):
        codes, exps = oracle.quantize_row_ue8m0(x[r])
        assert exps.shape == (H // 32,)
        packs = exps.view(np.int16)
        assert packs.size == -(-H // 64) == golden["ue8m0_scale_packs"]["num_sf_packs_int16"]
        assert golden["ue8m0_scale_packs"]["ue8m0_per_pack"] == 2
        lo, hi = (packs.view(np.uint16) & 0xFF).astype(np.uint8), (packs.view(np.uint16) >> 8).astype(np.uint8)
        np.testing.assert_array_equal(lo, exps[0::2])
        np.testing.assert_array_equal(hi, exps[1::2])
        xf = bf16_bits_to_f64(x[r])
        for b in range(H // 32):
            blk = xf[32 * b:32 * (b + 1)]
            cb = codes[32 * b:32 * (b + 1)]
            e = int(exps[b])
            if not np.all(np.isfinite(blk)):
                assert e == 0xFF
                exp_codes = np.where(np.isnan(blk).any() | np.isinf(blk), 0x7F, np.where(np.signbit(blk), 0x80, 0x00))
                np.testing.assert_array_equal(cb, exp_codes.astype(np.uint8))
                continue
            amax = float(np.abs(blk).max())
            k = e - 127
            assert 0 <= e <= 254
            assert math.ldexp(448.0, k) >= amax, (r, b, e, amax)
            assert e == 0 or math.ldexp(448.0, k - 1) < amax, (r, b, e, amax)
            # closed form from frexp: amax = M * 2^E, M in [1, 2); k = E - 8 + (M > 1.75)
            if amax < 2.0 ** -126:
                e_cf = 0
            else:
                f, ex = math.frexp(amax)
                e_cf = max(0, (ex - 1) - 8 + (1 if 2 * f > 1.75 else 0) + 127)
            assert e == e_cf, (r, b, e, e_cf)
            seen_eq |= amax == math.ldexp(448.0, k) and e > 0
            seen_up |= e > 0 and 2 * math.frexp(amax)[0] > 1.75  # mantissa above 1.75: next power up
            q = np.ldexp(blk, -k)  # exact in float64
            np.testing.assert_array_equal(cb, brute_force_e4m3(q), err_msg=f"row {r} block {b}")
            assert np.all((cb & 0x7F) <= 0x7E)
    assert seen_eq and seen_up
    bc, be = oracle.quantize_rows_ue8m0(x, H, 3, 9)  # the batched form is the per-row form
    for r in range(3, 9):
        c1, e1 = oracle.quantize_row_ue8m0(x[r])
        np.testing.assert_array_equal(bc[r - 3], c1)
        np.testing.assert_array_equal(be[r - 3], e1)


def test_dispatch_fp8_ue8m0_rows():
    """Fused UE8M0 dispatch: every valid row carries its token's codes and exponent bytes
    (oracle_quantize_row_ue8m0), padding rows zero bytes with zero padding, fixed-window
    tails zero bytes; pre-quantised input and column-major layout are refused."""
    w = small_workload(H=512)
    topk = synth.gen_routing(w)
    x = _ue8m0_rows(np.random.default_rng(22), w.H)
    x = np.vstack([x] * (-(-w.T // x.shape[0])))[:w.T]
    wt = synth.gen_weights(w)
    lay = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk)
    El = w.E // w.P
    for capacity in (0, int(lay.num_expanded.max()) + 7):
        rx, sc, rw, rm, _ = oracle.dispatch_general(lay, w.H, fp8=True, zero_padding=True, topk_weights=wt, x=x,
                                                    capacity=capacity, scales_ue8m0=True, fill=0x33)
        assert sc.dtype == np.uint8 and sc.shape == (rx.shape[0], w.H // 32)
        covered = np.zeros(rx.shape[0], bool)
        for u in range(w.T):
            c, e = oracle.quantize_row_ue8m0(x[u])
            for j in range(w.K):
                ex = topk[u, j]
                if ex < 0:
                    continue
                base = (ex // El) * capacity if capacity else lay.window_row_base[ex // El]
                row = base + lay.dst_slot[u, j]
                np.testing.assert_array_equal(rx[row], c)
                np.testing.assert_array_equal(sc[row], e)
                covered[row] = True
        assert (rx[~covered] == 0).all() and (sc[~covered] == 0).all()
        assert (rm[~covered] == -1).all()
    with pytest.raises(oracle.OracleError):
        oracle.dispatch_general(lay, w.H, fp8=True, zero_padding=True, topk_weights=wt,
                                x_codes=np.zeros((w.T, w.H), np.uint8),
                                x_scales=np.zeros((w.T, w.H // 128), np.float32), scales_ue8m0=True)


def test_dispatch_fp8_rows_and_zero_padding():
    w = small_workload(P=4, S=32, E=8, K=2, H=384, A=8, seed=12)
    topk = synth.gen_routing(w)
    x = synth.gen_bf16_rows(5, 1, w.T, w.H)
    wt = synth.gen_weights(w)
    lay = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk)
    rx, sc, rw, meta = oracle.dispatch(lay, w.H, x, wt, True, True, fill=0x7F)
    El = w.E // w.P
    for u in range(w.T):
        codes, scales = oracle.quantize_row(x[u])
        for j in range(w.K):
            r = lay.window_row_base[topk[u, j] // El] + lay.dst_slot[u, j]
            np.testing.assert_array_equal(rx[r], codes)
            np.testing.assert_array_equal(sc[r], scales)
    pad = meta[:, 0] < 0
    assert np.all(rx[pad] == 0) and np.all(sc[pad] == 0)
    # partial row ranges reproduce the same rows
    lo, hi = 5, lay.total_rows - 3
    rx2, sc2, rw2, meta2 = oracle.dispatch(lay, w.H, x, wt, True, True, lo, hi, fill=0x7F)
    np.testing.assert_array_equal(rx2, rx[lo:hi])
    np.testing.assert_array_equal(meta2, meta[lo:hi])


# ---------------------------------------------------------------------------
# combine
# ---------------------------------------------------------------------------


def bf16_ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in bf16 units in the last place (monotone integer mapping of the bit patterns)."""
    def key(h):
        h = h.astype(np.int32)
        return np.where(h & 0x8000, 0x8000 - (h & 0x7FFF), 0x8000 + (h & 0x7FFF))
    return np.abs(key(a) - key(b))


def test_combine_unit_weights_is_exact_k_times_x():
    """With unit weights every valid row carries x[u]; K*x is exact in fp32 for bf16 x and
    K <= 8, so out == bf16(K_valid * x) bit-exactly whatever the order or fusion."""
    w = small_workload(P=4, S=64, E=16, K=4, H=256, A=4, seed=21)
    topk = synth.gen_routing(w).copy()
    topk[::3, 3] = -1
    topk[::10] = -1  # tokens with no valid slot combine to +0
    x = synth.gen_bf16_rows(6, 1, w.T, w.H)
    lay = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk)
    y, _, _, _ = oracle.dispatch(lay, w.H, x, np.ones((w.T, w.K), np.float32), False, True)
    out = oracle.combine(lay, w.H, y, None)
    kv = (topk >= 0).sum(1).astype(np.float64)
    expect = torch_bf16_bits((bf16_bits_to_f64(x) * kv[:, None]).astype(np.float32))
    expect[kv == 0] = 0  # no valid slot: the empty sum is +0
    np.testing.assert_array_equal(out, expect)
    out_id = oracle.combine_identity(w.K, w.H, False, topk, x, None, 0, w.T)
    np.testing.assert_array_equal(out_id, expect)
    assert np.all(out[::10] == 0)



def test_combine_unit_weights_on_subnormals_closed_form():
    """K equal bf16 subnormal rows with unit weights: K*v is exact in fp32, and below 2^-125
    a bf16 value's bit pattern, read as an integer, is the value in units of 2^-133 (the
    subnormals, then the first normal binade, continue the same integer scale).  So the
    output bits are sign | (mantissa * K) whenever that stays below 256: a closed form that
    no floating-point arithmetic enters."""
    H = 128
    rng = np.random.default_rng(71)
    for K in (1, 2, 3, 4, 8):
        topk = np.arange(K, dtype=np.int64)[None, :]
        lay = oracle.layout(1, 1, K, K, 1, topk)
        top = min(127, 255 // K)  # inputs subnormal (7-bit mantissa), sums below 2^-125
        mant = rng.integers(1, top + 1, H).astype(np.uint16)
        mant[:4] = [1, 2, top, max(1, 127 // K)]
        sign = (rng.integers(0, 2, H) << 15).astype(np.uint16)
        v = sign | mant  # exponent field 0: bf16 subnormals
        y = np.repeat(v[None, :], K, 0)
        out = oracle.combine(lay, H, y, None)
        np.testing.assert_array_equal(out[0], sign | (mant * K).astype(np.uint16), err_msg=f"K={K}")


def test_combine_general_rows_within_one_ulp_of_exact_sum():
    w = small_workload(P=4, S=96, E=32, K=8, H=256, A=8, seed=22)
    topk = synth.gen_routing(w)
    wt = synth.gen_weights(w)
    lay = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk)
    y = synth.gen_bf16_rows(7, 4, lay.total_rows, w.H)
    out = oracle.combine(lay, w.H, y, wt)
    El = w.E // w.P
    rows = lay.window_row_base[topk // El] + lay.dst_slot  # [T, K]
    exact = np.einsum("tk,tkh->th", wt.astype(np.float64), bf16_bits_to_f64(y[rows]))
    ref = torch_bf16_bits(exact.astype(np.float32))
    ulp = bf16_ulp_diff(out, ref)
    assert ulp.max() <= 1
    assert (ulp == 0).mean() > 0.99
    # transposed weights (a plausible index slip) must be caught
    out_bad = oracle.combine(lay, w.H, y, np.ascontiguousarray(wt[:, ::-1]))
    assert bf16_ulp_diff(out_bad, ref).max() > 1


def test_combine_identity_equals_x_times_weight_sum():
    """combine(dispatch(x)) with identity experts is x * sum(w) within 1 bf16 ulp."""
    w = small_workload(P=8, S=64, E=64, K=8, H=512, A=16, seed=23)
    topk = synth.gen_routing(w)
    wt = synth.gen_weights(w)
    x = synth.gen_bf16_rows(8, 1, w.T, w.H)
    out = oracle.combine_identity(w.K, w.H, False, topk, x, wt, 0, w.T)
    ref = torch_bf16_bits((bf16_bits_to_f64(x) * wt.astype(np.float64).sum(1)[:, None]).astype(np.float32))
    assert bf16_ulp_diff(out, ref).max() <= 1
    lay = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk)
    y, _, _, _ = oracle.dispatch(lay, w.H, x, wt, False, True)
    np.testing.assert_array_equal(oracle.combine(lay, w.H, y, wt), out)


def test_combine_identity_fp8_error_bound():
    w = small_workload(P=4, S=32, E=16, K=4, H=512, A=8, seed=24)
    topk = synth.gen_routing(w)
    wt = synth.gen_weights(w)
    x = synth.gen_bf16_rows(9, 1, w.T, w.H)
    out = bf16_bits_to_f64(oracle.combine_identity(w.K, w.H, True, topk, x, wt, 0, w.T))
    xf = bf16_bits_to_f64(x)
    sw = wt.astype(np.float64).sum(1)[:, None]
    # |out - x*sum(w)| <= sum(w)*|x - dequant(x)| + bf16 rounding of the dequant and of the sum
    bound = sw * (2.0 ** -4 * np.abs(xf) + 2.0 ** -8 * np.abs(xf)) + 2.0 ** -7 * np.abs(xf * sw) + 1e-30
    scale_floor = np.repeat(np.abs(xf).reshape(w.T, -1, 128).max(2) / 448 * 2.0 ** -9, 128, axis=1)
    assert np.all(np.abs(out - xf * sw) <= bound + sw * scale_floor)


# ---------------------------------------------------------------------------
# fixed output length ("Ascend DeepEP MoE Dispatch Optimization", section on the
# dynamic and fixed output-length modes)
# ---------------------------------------------------------------------------


def test_fixed_length_worked_example_from_pages(golden):
    """The page's example: a rank that receives 237 rows, exposed as 256 rows, the last 19
    of them padding (index -1, x / weights 0) -- also without the zero-padding flag."""
    ex = golden["num_worst_tokens_example"]
    valid, public, tail = ex["valid_rows"], ex["public_rows"], ex["padding_rows"]
    assert valid + tail == public
    P, S, E, K, A, H = 2, 200, 4, 1, 1, 128
    topk = np.full((P * S, K), -1, np.int64)
    topk[:valid, 0] = np.arange(valid) % 2          # rank 0's experts 0 and 1
    topk[valid:valid + 120, 0] = 2 + np.arange(120) % 2  # rank 1: 120 rows
    x = synth.gen_bf16_rows(5, 1, P * S, H)
    wt = np.linspace(0.5, 1.5, P * S * K, dtype=np.float32).reshape(P * S, K)
    lay = oracle.layout(P, S, E, K, A, topk)
    assert int(lay.num_expanded[0]) == valid
    rx, _, rw, meta, dropped = oracle.dispatch_fixed(lay, H, public, x, wt, False, False, fill=0xFFFF)
    assert dropped == 0 and rx.shape == (P * public, H)
    # rank 0: the first 237 rows hold the tokens, the last 19 are the tail
    assert np.all(meta[:valid, 0] >= 0)
    assert np.all(meta[valid:public] == -1) and np.all(rw[valid:public] == 0)
    assert np.all(rx[valid:public] == 0)
    assert (meta[:public, 0] < 0).sum() == tail
    for r in range(valid):
        u = meta[r, 0]
        np.testing.assert_array_equal(rx[r], x[u])
    # rank 1: 120 rows then 136 tail rows
    assert np.all(meta[public:public + 120, 0] >= 0) and np.all(meta[public + 120:] == -1)


def _exact_and_fixed(w, topk, W, fp8, zero_padding, seed):
    x = synth.gen_bf16_rows(seed, 1, w.T, w.H)
    wt = synth.gen_weights(w)
    lay = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk)
    ex = oracle.dispatch(lay, w.H, x, wt, fp8, zero_padding, fill=0xAB)
    fx = oracle.dispatch_fixed(lay, w.H, W, x, wt, fp8, zero_padding, fill=0xCD)
    return lay, x, wt, ex, fx


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("zero_padding", [True, False])
def test_fixed_length_is_exact_window_plus_tail(fp8, zero_padding):
    """With a capacity at least every window's rows, window d of the fixed output is the
    exact window d followed by a zero tail (index -1): the same rows at the same
    window-local positions, nothing dropped."""
    w = small_workload(P=4, S=64, E=16, K=3, H=256, A=16, seed=31)
    topk = synth.gen_routing(w).copy()
    topk[::11, 1] = -1
    lay0 = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk)
    W = int(lay0.num_expanded.max()) + 37
    lay, x, wt, (erx, esc, erw, emeta), (frx, fsc, frw, fmeta, dropped) = _exact_and_fixed(
        w, topk, W, fp8, zero_padding, 32)
    assert dropped == 0
    for d in range(w.P):
        b, n = int(lay.window_row_base[d]), int(lay.num_expanded[d])
        f = slice(d * W, d * W + n)
        e = slice(b, b + n)
        np.testing.assert_array_equal(fmeta[f], emeta[e])
        np.testing.assert_array_equal(frw[f], erw[e])
        defined = (emeta[e, 0] >= 0) | zero_padding  # padding payload is defined only with zero padding
        np.testing.assert_array_equal(frx[f][defined], erx[e][defined])
        if fp8:
            np.testing.assert_array_equal(fsc[f][defined], esc[e][defined])
        t = slice(d * W + n, (d + 1) * W)
        assert np.all(fmeta[t] == -1) and np.all(frw[t] == 0) and np.all(frx[t] == 0)
        if fp8:
            assert np.all(fsc[t] == 0)
    # combine over the fixed windows equals the exact combine bit for bit
    y_exact = erx if not fp8 else oracle.dispatch(lay, w.H, x, wt, False, True)[0]
    y_fixed = frx if not fp8 else oracle.dispatch_fixed(lay, w.H, W, x, wt, False, True)[0]
    np.testing.assert_array_equal(oracle.combine_fixed(lay, w.H, W, y_fixed, wt),
                                  oracle.combine(lay, w.H, y_exact, wt))


@pytest.mark.parametrize("A", [1, 8])
@pytest.mark.parametrize("which", ["median", "small"])
def test_fixed_length_truncation_drops_tail_rows_and_their_slots(A, which):
    """A capacity below some window's row count publishes the first W rows of each window;
    the dropped count is sum_d max(0, num_expanded[d] - W) (num_expanded from its closed
    form); combine then equals the exact combine with the dropped slots' weights zeroed."""
    w = small_workload(P=4, S=80, E=16, K=4, H=128, A=A, routing="zipf", seed=33)
    topk = synth.gen_routing(w)
    n = np.bincount(topk[topk >= 0], minlength=w.E)
    ne = (-(-n // A) * A).reshape(w.P, -1).sum(1)
    if which == "median":
        W = int(np.sort(ne)[w.P // 2])  # about half the windows overflow
        assert (ne > W).any() and (ne < W).any()
    else:
        W = max(1, int(ne.min()) // 2)  # every window overflows, the first ones too: a row
        assert (ne > W).all()            # index reaching W must not land in the next window
    lay, x, wt, (erx, _, erw, emeta), (frx, _, frw, fmeta, dropped) = _exact_and_fixed(
        w, topk, W, False, True, 34)
    assert dropped == int(np.maximum(ne - W, 0).sum())
    for d in range(w.P):
        b, k = int(lay.window_row_base[d]), min(int(ne[d]), W)
        np.testing.assert_array_equal(fmeta[d * W:d * W + k], emeta[b:b + k])
        np.testing.assert_array_equal(frx[d * W:d * W + k], erx[b:b + k])
        np.testing.assert_array_equal(frw[d * W:d * W + k], erw[b:b + k])
        assert np.all(fmeta[d * W + k:(d + 1) * W] == -1)
    # every published slot appears once; the others are the slots whose row index reached W
    kept = fmeta[fmeta[:, 0] >= 0]
    trunc = np.zeros((w.T, w.K), bool)
    for u in range(w.T):
        for j in range(w.K):
            if topk[u, j] >= 0 and lay.dst_slot[u, j] >= W:
                trunc[u, j] = True
    assert len(kept) == int((topk >= 0).sum() - trunc.sum())
    wt0 = wt.copy()
    wt0[trunc] = 0.0
    np.testing.assert_array_equal(oracle.combine_fixed(lay, w.H, W, frx, wt),
                                  oracle.combine(lay, w.H, erx, wt0))


# ---------------------------------------------------------------------------
# API variants: column-major scales, pre-quantised input, combine bias
# (TileLang tutorial ch. 38, sections 3.3 and 3.6)
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("capacity", [0, 150])
def test_scales_col_major_is_the_transpose_of_row_major(capacity):
    """The column-major scale layout holds scale b of row r at b * rows + r: the transpose of
    the row-major [rows, H/128] layout, with no padding of the row dimension.  Six blocks
    per row, so that a swapped index cannot hide behind a square or a short block count."""
    w = small_workload(P=4, S=40, E=16, K=3, H=768, A=8, seed=41)
    topk = synth.gen_routing(w)
    x = synth.gen_bf16_rows(42, 1, w.T, w.H)
    wt = synth.gen_weights(w)
    lay = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk)
    rm = oracle.dispatch_general(lay, w.H, fp8=True, zero_padding=True, topk_weights=wt, x=x, capacity=capacity)
    cm = oracle.dispatch_general(lay, w.H, fp8=True, zero_padding=True, topk_weights=wt, x=x, capacity=capacity,
                                 scales_col_major=True)
    n = rm[0].shape[0]
    assert rm[1].shape == (n, 6) and cm[1].shape == (6, n)
    np.testing.assert_array_equal(cm[1], rm[1].T)
    np.testing.assert_array_equal(cm[0], rm[0])
    flat = cm[1].ravel()
    meta = rm[3]
    for r in np.flatnonzero(meta[:, 0] >= 0)[::17]:
        u = meta[r, 0]
        xf = bf16_bits_to_f64(x[u]).astype(np.float32).reshape(6, 128)
        amax = np.abs(xf).max(axis=1)
        for b in range(6):
            assert flat[b * n + r] == np.float32(amax[b]) / np.float32(448.0)


def test_prequantised_input_is_copied_and_matches_fused_quantisation():
    """Dispatching (E4M3 data, fp32 scales) moves those bytes unchanged to every row of the
    token; fed with the per-token quantisation of x it equals the fused fp8 dispatch."""
    w = small_workload(P=4, S=48, E=16, K=3, H=512, A=4, seed=43)
    topk = synth.gen_routing(w).copy()
    topk[::9, 2] = -1
    x = synth.gen_bf16_rows(44, 1, w.T, w.H)
    wt = synth.gen_weights(w)
    lay = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk)
    codes = np.empty((w.T, w.H), np.uint8)
    scales = np.empty((w.T, w.H // 128), np.float32)
    for u in range(w.T):
        codes[u], scales[u] = oracle.quantize_row(x[u])
    fused = oracle.dispatch_general(lay, w.H, fp8=True, zero_padding=True, topk_weights=wt, x=x)
    pre = oracle.dispatch_general(lay, w.H, fp8=True, zero_padding=True, topk_weights=wt, x_codes=codes,
                                  x_scales=scales)
    for a, b in zip(fused[:4], pre[:4]):
        np.testing.assert_array_equal(a, b)
    # arbitrary bytes (NaN codes included) and scales travel bit for bit
    rng = np.random.default_rng(45)
    rc = rng.integers(0, 256, (w.T, w.H), dtype=np.uint8)
    rs = rng.standard_normal((w.T, w.H // 128)).astype(np.float32)
    got = oracle.dispatch_general(lay, w.H, fp8=True, zero_padding=False, topk_weights=wt, x_codes=rc,
                                  x_scales=rs, fill=0xEE)
    meta = got[3]
    valid = meta[:, 0] >= 0
    np.testing.assert_array_equal(got[0][valid], rc[meta[valid, 0]])
    np.testing.assert_array_equal(got[1][valid].view(np.uint32), rs[meta[valid, 0]].view(np.uint32))
    assert np.all(got[0][~valid] == 0xEE)  # padding untouched without zero padding


def test_combine_bias_closed_forms():
    """Bias is added after the K slots, before the single rounding.  With y rows = x and unit
    weights the result is exactly bf16((k + 1) x) for a bias equal to x (k valid slots), and
    +0 for a bias equal to -x when a token has one valid slot."""
    w = small_workload(P=4, S=64, E=16, K=4, H=256, A=4, seed=46)
    topk = synth.gen_routing(w).copy()
    topk[::5, 1:] = -1  # tokens with a single valid slot
    x = synth.gen_bf16_rows(47, 1, w.T, w.H)
    lay = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk)
    y, _, _, _ = oracle.dispatch(lay, w.H, x, np.ones((w.T, w.K), np.float32), False, True)
    kv = (topk >= 0).sum(1).astype(np.float64)
    out = oracle.combine_general(lay, w.H, y, None, bias=x)
    expect = torch_bf16_bits((bf16_bits_to_f64(x) * (kv + 1)[:, None]).astype(np.float32))
    np.testing.assert_array_equal(out, expect)
    neg = x ^ np.uint16(0x8000)
    out = oracle.combine_general(lay, w.H, y, None, bias=neg)
    one = kv == 1
    assert np.all(out[one] == 0)  # x + (-x) = +0 in round-to-nearest
    np.testing.assert_array_equal(oracle.combine_identity(w.K, w.H, False, topk, x, None, 0, w.T, bias=x),
                                  oracle.combine_general(lay, w.H, y, None, bias=x))


def test_combine_bias_general_within_one_ulp():
    w = small_workload(P=4, S=64, E=32, K=8, H=256, A=8, seed=48)
    topk = synth.gen_routing(w)
    wt = synth.gen_weights(w)
    lay = oracle.layout(w.P, w.S, w.E, w.K, w.A, topk)
    y = synth.gen_bf16_rows(49, 1, lay.total_rows, w.H)
    bias = synth.gen_bf16_rows(50, 1, w.T, w.H)
    out = oracle.combine_general(lay, w.H, y, wt, bias=bias)
    El = w.E // w.P
    rows = lay.window_row_base[topk // El] + lay.dst_slot
    exact = (bf16_bits_to_f64(y)[rows] * wt[:, :, None].astype(np.float64)).sum(1) + bf16_bits_to_f64(bias)
    ref = torch_bf16_bits(exact.astype(np.float32))
    d = bf16_ulp_diff(out, ref)
    assert d.max() <= 1 and (d == 0).mean() > 0.99
    # a dropped bias term is caught
    assert (bf16_ulp_diff(out, oracle.combine_general(lay, w.H, y, wt)) > 1).mean() > 0.5


# --------------------------------------------------------------------------
# Combine arithmetic order, pinned by values chosen so that another order
# (or a fused multiply-add) changes the bf16 result, not just the last fp32 bit.
# --------------------------------------------------------------------------

_B = float(np.float32(2.0**25 + 2.0**17))  # exactly halfway between bf16 2^25 and 2^25 + 2^18


def _one_token_combine(weights, y_rows=None, bias=None):
    """One token whose K slots go to K distinct experts (P = 1, A = 1, so expert k owns row k);
    y row k is y_rows[k] (bf16 bits, default 1.0) across 8 channels; returns out[0][0]."""
    K = len(weights)
    topk = np.arange(K, dtype=np.int64)[None, :]
    lay = oracle.layout(1, 1, K, K, 1, topk)
    H = 8
    rows = [0x3F80] * K if y_rows is None else list(y_rows)
    y = np.repeat(np.asarray(rows, np.uint16)[:, None], H, 1)
    w = np.asarray(weights, np.float32)[None, :]
    b = None if bias is None else np.full((1, H), bias, np.uint16)
    return int(oracle.combine_general(lay, H, y, w, bias=b)[0, 0])


def test_combine_slot_order_is_ascending():
    """From acc = +0 the slots are added in order j = 0..K-1.  With w = (B, 1, 1, 1) on unit
    rows each +1 is lost against B (fp32 spacing 4 there, B even), so the sum stays at B, a
    bf16 tie, which rounds to even: 2^25 (0x4C00).  The same terms in the order (1, 1, 1, B)
    reach 3 + B -> B + 4 and round up to 2^25 + 2^18 (0x4C01)."""
    assert _one_token_combine([_B, 1.0, 1.0, 1.0]) == 0x4C00
    assert _one_token_combine([1.0, 1.0, 1.0, _B]) == 0x4C01


def test_combine_multiplies_and_adds_separately():
    """acc = fl(acc + fl(w * y)), no fused multiply-add.  w0 = -(1 + 2^-7 + 2^-23) on y0 = 1,
    then w1 = 1 + 2^-23 on y1 = 1 + 2^-7: the product 1 + 2^-7 + 2^-23 + 2^-30 rounds to
    1 + 2^-7 + 2^-23 and cancels acc exactly, giving +0.  A fused multiply-add would keep
    2^-30 (bf16 0x3080)."""
    w0 = -(1.0 + 2.0**-7 + 2.0**-23)
    w1 = 1.0 + 2.0**-23
    assert np.float32(w0) == w0 and np.float32(w1) == w1
    assert _one_token_combine([w0, w1], y_rows=[0x3F80, 0x3F81]) == 0x0000


def test_combine_bias_is_added_after_the_slots():
    """With w = (1, 1, B) on unit rows and a bias of 1: (1 + 1) + B = B + 2 -> B (ties to even),
    then + 1 -> B, the bf16 tie that rounds to 2^25 (0x4C00).  Adding the bias before the slots
    would give 1 + 1 + 1 + B -> B + 4, which rounds up (0x4C01)."""
    assert _one_token_combine([1.0, 1.0, _B], bias=0x3F80) == 0x4C00
    assert _one_token_combine([1.0, 1.0, 1.0, _B]) == 0x4C01  # the bias-first sum, for contrast
