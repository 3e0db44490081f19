"""Workload shapes and seeded generators for MoE dispatch/combine inputs.

Shapes follow the workloads the two source pages talk about (hidden 7168,
256 experts, top-6/top-8, 8-way and 128-way expert parallelism); see the
tutorial chapter "DeepEP-Ascend" (TileLang tutorial, ch. 38), section 1.2 and
section 3.1, and "Ascend DeepEP MoE Dispatch Optimization", section "A token's
journey through MoE".

Every array is drawn from numpy PCG64 streams keyed by
``SeedSequence(seed, spawn_key=(stream, block))`` so that any block of rows can
be regenerated on its own and blocks can be drawn in parallel threads.

Nothing here computes any part of dispatch or combine.  The only arithmetic is
in drawing the inputs: the softmax that turns N(0,1) logits into routing
weights, the Zipf/Gumbel scores that pick experts, and torch's float32 ->
bfloat16 cast of N(0,1) activations.
"""

from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# Stream ids for SeedSequence spawn keys.
STREAM_ROUTING = 0
STREAM_X = 1
STREAM_WEIGHTS = 2
STREAM_GRAD_OUT = 3
STREAM_EXPERT_OUT = 4
STREAM_PERM = 5
STREAM_CACHED_X = 100  # + iteration index

ROWS_PER_BLOCK = 1024  # rows per independently seeded block of activations


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: P virtual ranks x S tokens per rank."""

    name: str
    P: int  # virtual EP ranks
    S: int  # tokens per rank
    E: int  # experts (E_l = E / P per rank)
    K: int  # top-k
    H: int  # hidden size
    A: int  # expert_alignment
    zero_padding: bool
    routing: str  # "uniform" | "zipf" | "group"
    fp8: bool = False
    cached_iters: int = 0
    backward: bool = False
    seed: int = 0
    zipf_s: float = 1.0
    num_groups: int = 8  # group-limited routing: groups of consecutive ranks
    groups_per_token: int = 4

    @property
    def T(self) -> int:
        return self.P * self.S

    @property
    def E_l(self) -> int:
        return self.E // self.P

    def describe(self) -> dict:
        d = dataclasses.asdict(self)
        d["T"] = self.T
        return d


CONFIGS: dict[str, Workload] = {
    w.name: w
    for w in [
        # P=4 x S=64, E=16, K=2 uniform, H=512, alignment 16, zero padding, seed 0.
        Workload("tiny-p4-s64-e16-k2-h512", 4, 64, 16, 2, 512, 16, True, "uniform"),
        # DeepSeek-V3-like: P=8 x S=4096, E=256, K=8 uniform, H=7168, alignment 128.
        Workload("dsv3-bf16-p8-s4096-e256-k8-h7168", 8, 4096, 256, 8, 7168, 128, True, "uniform"),
        # Same routing, FP8 dispatch, plus 20 cached-handle dispatches of new x.
        Workload("dsv3-fp8-p8-s4096-e256-k8-h7168", 8, 4096, 256, 8, 7168, 128, True, "uniform",
                 fp8=True, cached_iters=20),
        # 128 ranks x 1024 tokens, E=256 (2 per rank), K=6, Zipf(1.0) popularity, no zero padding.
        Workload("ep128-zipf-p128-s1024-e256-k6-h7168", 128, 1024, 256, 6, 7168, 128, False, "zipf"),
        # 32 ranks x 8192 tokens, E=256, K=8 within 4 of 8 rank groups, H=4096, fwd + bwd.
        Workload("ep32-group-fwdbwd-p32-s8192-e256-k8-h4096", 32, 8192, 256, 8, 4096, 128, True,
                 "group", backward=True),
    ]
}
CONFIG_ORDER = list(CONFIGS)


def by_index(i: int) -> Workload:
    """Workload i (1-based) in the order above."""
    return CONFIGS[CONFIG_ORDER[i - 1]]


def scaled(w: Workload, P: int | None = None, S: int | None = None, H: int | None = None,
           E: int | None = None, K: int | None = None, A: int | None = None, seed: int | None = None,
           name: str | None = None, **kw) -> Workload:
    """A smaller (or otherwise varied) copy of a workload for full element-wise parity."""
    ch = {k: v for k, v in dict(P=P, S=S, H=H, E=E, K=K, A=A, seed=seed).items() if v is not None}
    ch.update(kw)
    nw = dataclasses.replace(w, **ch)
    if name is None:
        name = f"{w.name.split('-p')[0]}-p{nw.P}-s{nw.S}-e{nw.E}-k{nw.K}-h{nw.H}-a{nw.A}"
    return dataclasses.replace(nw, name=name)


def _gen(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _topk_desc(scores: np.ndarray, K: int) -> np.ndarray:
    """Indices of the K largest scores per row, in descending score order."""
    part = np.argpartition(-scores, K - 1, axis=1)[:, :K]
    sc = np.take_along_axis(scores, part, 1)
    order = np.argsort(-sc, axis=1, kind="stable")
    return np.take_along_axis(part, order, 1)


def gen_routing(w: Workload, block_rows: int = 16384) -> np.ndarray:
    """topk_idx [T, K] int64 for the workload's routing recipe.

    uniform: K distinct experts per token, uniform without replacement
             (top-K of i.i.d. uniform scores).
    zipf:    expert popularity p(e) proportional to 1/(pi(e)+1)^s over a seeded
             permutation pi; K distinct experts by Gumbel-top-K on log p
             (Plackett-Luce sampling without replacement).
    group:   the P ranks form num_groups groups of consecutive ranks; each token
             picks groups_per_token groups uniformly without replacement, then K
             distinct experts uniformly among those groups' experts.
    """
    T, E, K = w.T, w.E, w.K
    out = np.empty((T, K), dtype=np.int64)
    rng = _gen(w.seed, STREAM_ROUTING)
    if w.routing == "zipf":
        perm = _gen(w.seed, STREAM_PERM).permutation(E)
        logp = -w.zipf_s * np.log(perm.astype(np.float64) + 1.0)
    if w.routing == "group":
        assert w.P % w.num_groups == 0
        experts_per_group = E // w.num_groups
    for r0 in range(0, T, block_rows):
        n = min(block_rows, T - r0)
        if w.routing == "uniform":
            out[r0:r0 + n] = _topk_desc(rng.random((n, E)), K)
        elif w.routing == "zipf":
            g = rng.gumbel(size=(n, E))
            out[r0:r0 + n] = _topk_desc(logp[None, :] + g, K)
        elif w.routing == "group":
            groups = _topk_desc(rng.random((n, w.num_groups)), w.groups_per_token)
            cand = (groups[:, :, None] * experts_per_group
                    + np.arange(experts_per_group)[None, None, :]).reshape(n, -1)
            pick = _topk_desc(rng.random(cand.shape), K)
            out[r0:r0 + n] = np.take_along_axis(cand, pick, 1)
        else:
            raise ValueError(w.routing)
    return out


def gen_weights(w: Workload) -> np.ndarray:
    """topk_weights [T, K] float32: softmax over the K slots of N(0,1) logits."""
    rng = _gen(w.seed, STREAM_WEIGHTS)
    logits = rng.standard_normal((w.T, w.K), dtype=np.float32)
    z = logits - logits.max(axis=1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def gen_bf16_rows(seed: int, stream: int, rows: int, cols: int, row0: int = 0,
                  n: int | None = None) -> np.ndarray:
    """bf16 bit patterns (uint16) of N(0,1) draws, rows [row0, row0+n) of a rows x cols matrix.

    Block b (ROWS_PER_BLOCK rows) is drawn from its own generator, so any row
    range can be produced without the rest.  The float32 -> bfloat16 cast is
    torch's round-to-nearest-even conversion.
    """
    import torch

    if n is None:
        n = rows - row0
    assert 0 <= row0 and row0 + n <= rows
    out = np.empty((n, cols), dtype=np.uint16)
    if n == 0:
        return out
    b0, b1 = row0 // ROWS_PER_BLOCK, (row0 + n - 1) // ROWS_PER_BLOCK

    def fill(b: int) -> None:
        lo, hi = b * ROWS_PER_BLOCK, min((b + 1) * ROWS_PER_BLOCK, rows)
        f = _gen(seed, stream, b).standard_normal((hi - lo, cols), dtype=np.float32)
        s0, s1 = max(lo, row0), min(hi, row0 + n)
        part = torch.from_numpy(f[s0 - lo:s1 - lo]).to(torch.bfloat16)
        out[s0 - row0:s1 - row0] = part.view(torch.int16).numpy().view(np.uint16)

    blocks = range(b0, b1 + 1)
    if len(blocks) == 1:
        fill(b0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, blocks))
    return out


def gen_x(w: Workload) -> np.ndarray:
    """Activations x [T, H] as bf16 bit patterns."""
    return gen_bf16_rows(w.seed, STREAM_X, w.T, w.H)


def gen_cached_x(w: Workload, it: int) -> np.ndarray:
    """New activations for cached-handle dispatch iteration ``it`` (1-based)."""
    return gen_bf16_rows(w.seed, STREAM_CACHED_X + it, w.T, w.H)


def gen_grad_out(w: Workload) -> np.ndarray:
    """Upstream gradient of the combine output, [T, H] bf16 bit patterns."""
    return gen_bf16_rows(w.seed, STREAM_GRAD_OUT, w.T, w.H)


def gen_expert_out(w: Workload, total_rows: int) -> np.ndarray:
    """Arbitrary expert outputs [total_rows, H] bf16 bit patterns (combine input)."""
    return gen_bf16_rows(w.seed, STREAM_EXPERT_OUT, total_rows, w.H)
