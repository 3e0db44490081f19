// ep_layout.hpp -- layout kernels: routing table -> handle arrays.
//
// What is computed ("Ascend DeepEP MoE Dispatch Optimization", sections
// "What the six handle entries store" and "Notify exchanges counts and
// prefixes first"; TileLang tutorial ch. 38, sections 2.2, 2.4, 3.5):
// per-rank deduplicated destinations, per-expert / per-rank histograms, their
// prefix sums, and the deterministic position of every slot and every
// (token, destination) pair.
//
// How (no atomics anywhere, so the result is the same on every run):
//  1. layout_count  -- one 4-wave workgroup per chunk of 64 tokens of one
//     source rank; wave w owns the chunk's tokens [16w, 16w + 16).  Expert
//     and rank histograms by wavefront ballots: lanes holding the same key
//     are found with ballots and the lowest of them adds their popcount to
//     its wave's counters; the chunk's histogram is the sum of its waves'.
//     Each token's destination-rank bits are set by one lane; then the
//     is_token_in_rank rows.
//  2. layout_scan   -- one workgroup per histogram column (E experts + P
//     ranks): exclusive scan over chunks in order, per-source-rank sums.
//  3. layout_finalize -- one workgroup: aligned expert sizes, window offsets,
//     window bases, receive-list bases, where each expert's padding rows go
//     in the padding list, host summary (fixed windows: clipped padding,
//     tail bases, dropped rows).
//  4. layout_rank   -- one 4-wave workgroup per chunk again; wave w owns the
//     chunk's tokens [16w, 16w + 16).  Each wave counts its slots per key
//     (expert, first-seen destination rank); a prefix over the waves, seeded
//     with the chunk's scanned offsets, gives every wave its starting
//     position per key.  Each wave then walks its (u, j) slots 64 at a time
//     in memory order; lanes holding the same key are found with ballots,
//     their order within the step is their lane order, and the wave's
//     running counter per key carries the order across steps.  This yields
//     the global stable order by (u, j).  The same kernel writes the
//     padding-row list and send_head.
//
// Small batches (at most kSmallChunks chunks, none holding more than
// kSmallMaxChunkSlots slots) run all four steps in one 16-wave workgroup
// instead (layout_small_kernel): wave c counts and ranks chunk c, the scans
// and the finalize step run between workgroup barriers on LDS-resident
// histograms, and the handle arrays come out identical.
#pragma once

#include "ep_device.hpp"

namespace ep {

constexpr int kChunk = 64;          // tokens per layout chunk
constexpr int kLayoutThreads = 256;  // workgroup of the count and rank kernels: 4 waves per chunk
constexpr int kLayoutWaves = kLayoutThreads / kWave;
constexpr int kTokensPerWave = kChunk / kLayoutWaves;

struct LayoutDims {
  int P, S, E, K, A, El;
  int cpr;         // chunks per source rank, ceil(S / kChunk)
  int num_chunks;  // P * cpr
  int ncols;       // E + P + 1 histogram columns (experts, ranks, bad ids)
  int ebits;       // bits for expert keys 0..E (E = "no expert")
  int pbits;       // bits for rank keys 0..P (P = "not a new destination")
  int symmetric;   // window policy
  int cap;         // fixed rows per window (0: exact windows)
};

struct ChunkPos {
  int c, s, t0, n;
  int64_t u0;
};

__device__ __forceinline__ ChunkPos chunk_pos(const LayoutDims& d, int c) {
  ChunkPos p;
  p.c = c;
  p.s = p.c / d.cpr;
  p.t0 = (p.c % d.cpr) * kChunk;
  p.n = min(kChunk, d.S - p.t0);
  p.u0 = (int64_t)p.s * d.S + p.t0;
  return p;
}

// Stage the chunk's routing into LDS as int32: expert id, -1 for an unused
// slot, -2 for an out-of-range id.  Coalesced: the chunk's n*K entries are
// contiguous in topk_idx.
__device__ __forceinline__ void stage_chunk_experts(const LayoutDims& d, const ChunkPos& p,
                                                    const int64_t* __restrict__ topk_idx,
                                                    int32_t* ex, int first, int stride) {
  const int total = p.n * d.K;
  const int64_t* src = topk_idx + p.u0 * d.K;
  for (int i = first; i < total; i += stride) {
    const int64_t e = src[i];
    ex[i] = (e >= 0 && e < d.E) ? (int32_t)e : (e == -1 ? -1 : -2);
  }
}

// Barrier over the NT threads that run a step: the workgroup, or, for NT =
// 64, the one wave that runs it alone (its LDS accesses are ordered; the
// builtin keeps the compiler from moving them across).
template <int NT>
__device__ __forceinline__ void group_sync() {
  if constexpr (NT == kWave)
    __builtin_amdgcn_wave_barrier();
  else
    __syncthreads();
}

// Exclusive scan over NT threads (NT multiple of 64; NT = 64: one wave).
template <int NT>
__device__ __forceinline__ int64_t block_excl_scan(int64_t v, int64_t* wsum, int64_t* total) {
  const int lane = threadIdx.x & 63, wid = NT == kWave ? 0 : threadIdx.x >> 6;
  int64_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if constexpr (NT == kWave) {
    *total = __shfl(x, 63, 64);
    return x - v;
  }
  if (lane == 63) wsum[wid] = x;
  __syncthreads();
  int64_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int64_t s = wsum[w];
    before += (w < wid) ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

// --------------------------------------------------------------------------
// 1. counts
// --------------------------------------------------------------------------
// A slot is its token's first on rank r if no earlier slot of the token maps
// to r; that test only reads the staged row, so every slot is one lane.
__device__ __forceinline__ bool first_on_rank(const LayoutDims& d, const int32_t* ex, int t, int j, int r) {
  for (int jj = 0; jj < j; ++jj) {
    const int e2 = ex[t * d.K + jj];
    if (e2 >= 0 && e2 / d.El == r) return false;
  }
  return true;
}

// Adds one to counter `col` of this wave for every lane whose col >= 0.
// Lanes holding the same column are found with ballots (match_any), and the
// lowest of them adds their popcount; only this wave writes `cnt`, so no
// atomics are needed.  Every lane of the wave must call this (uniform
// control flow); `none` is a key no live column takes.
__device__ __forceinline__ void wave_count(int32_t* cnt, int col, int none, int bits, int lane) {
  const uint32_t key = col >= 0 ? (uint32_t)col : (uint32_t)none;
  const uint64_t peers = match_any(key, bits);
  if (col >= 0 && lane == (int)__builtin_ctzll(peers)) cnt[col] += __builtin_popcountll(peers);
  __builtin_amdgcn_wave_barrier();
}

// One wave's share of a chunk: tokens [t0, t0 + nt) of the chunk whose
// experts are staged in ex.  Histogram columns (hist[ncols], this wave's
// own counters): expert e, the destination rank E + r of each token's first
// slot on r, and E + P for an out-of-range id.  rmask_rows: the chunk's
// destination-rank bit rows ([64][words]); lane t sets token t0 + t's bits.
__device__ __forceinline__ void count_wave_tokens(const LayoutDims& d, const int32_t* ex, int t0, int nt, int lane,
                                                  int32_t* hist, uint32_t* rmask_rows, int words) {
  const int first = t0 * d.K, total = max(nt, 0) * d.K;
  for (int base = 0; base < total; base += kWave) {  // uniform trip count per wave
    const int i = base + lane;
    const int s = first + i;
    const int e = i < total ? ex[s] : -1;
    int col_r = -1;
    if (e >= 0) {
      const int t = s / d.K, j = s - t * d.K, r = e / d.El;
      if (first_on_rank(d, ex, t, j, r)) col_r = r;
    }
    wave_count(hist, e >= 0 ? e : -1, d.E, d.ebits, lane);  // experts: columns [0, E)
    wave_count(hist + d.E, col_r, d.P, d.pbits, lane);      // ranks: columns [E, E + P)
    const uint64_t bad = ballot(e == -2);                   // out-of-range ids: column E + P
    if (bad != 0 && lane == 0) hist[d.E + d.P] += __builtin_popcountll(bad);
    __builtin_amdgcn_wave_barrier();
  }
  if (lane < nt) {
    const int t = t0 + lane;
    for (int j = 0; j < d.K; ++j) {
      const int e = ex[t * d.K + j];
      if (e >= 0) {
        const int r = e / d.El;
        rmask_rows[t * words + (r >> 5)] |= 1u << (r & 31);
      }
    }
  }
}

// is_token_in_rank rows of n tokens (one contiguous byte range) from their
// bit rows; threads first, first + stride, ...
__device__ __forceinline__ void write_itr_rows(const LayoutDims& d, const uint32_t* rmask_rows, int words, int n,
                                               uint8_t* itr, int first, int stride) {
  const int nbytes = n * d.P;
  if ((d.P & 3) == 0) {
    uint32_t* itr4 = (uint32_t*)itr;  // the first token's row starts at a multiple of 4 bytes
    for (int wi = first; wi < (nbytes >> 2); wi += stride) {
      const int t = (wi << 2) / d.P, r0 = (wi << 2) - t * d.P;
      const uint32_t* m = rmask_rows + t * words;
      uint32_t v = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) v |= ((m[(r0 + q) >> 5] >> ((r0 + q) & 31)) & 1u) << (8 * q);
      itr4[wi] = v;
    }
  } else {
    for (int bi = first; bi < nbytes; bi += stride) {
      const int t = bi / d.P, r = bi - t * d.P;
      itr[bi] = (uint8_t)((rmask_rows[t * words + (r >> 5)] >> (r & 31)) & 1u);
    }
  }
}

// LDS: per-wave histograms [kLayoutWaves][ncols] | rank bit rows [64][ceil(P/32)] |
//      staged experts [64*K]
__global__ __launch_bounds__(kLayoutThreads) void layout_count_kernel(LayoutDims d,
                                                                      const int64_t* __restrict__ topk_idx,
                                                                      uint8_t* __restrict__ is_token_in_rank,
                                                                      int32_t* __restrict__ chunk_hist) {
  extern __shared__ int32_t lds[];
  const int words = (d.P + 31) >> 5;
  int32_t* hist = lds;
  uint32_t* rmask = (uint32_t*)(lds + kLayoutWaves * d.ncols);
  int32_t* ex = (int32_t*)(rmask + kChunk * words);
  const ChunkPos p = chunk_pos(d, blockIdx.x);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid >> 6;
  EP_TIMING_MARK(EP_TK_COUNT, 0);

  for (int i = tid; i < kLayoutWaves * d.ncols; i += kLayoutThreads) hist[i] = 0;
  for (int i = tid; i < kChunk * words; i += kLayoutThreads) rmask[i] = 0;
  stage_chunk_experts(d, p, topk_idx, ex, tid, kLayoutThreads);
  __syncthreads();

  const int t0 = wv * kTokensPerWave;
  count_wave_tokens(d, ex, t0, min(kTokensPerWave, p.n - t0), lane, hist + wv * d.ncols, rmask, words);
  __syncthreads();
  EP_TIMING_MARK(EP_TK_COUNT, 1);

  write_itr_rows(d, rmask, words, p.n, is_token_in_rank + p.u0 * d.P, tid, kLayoutThreads);
  for (int col = tid; col < d.ncols; col += kLayoutThreads) {
    int32_t sum = 0;
#pragma unroll
    for (int w = 0; w < kLayoutWaves; ++w) sum += hist[w * d.ncols + col];
    chunk_hist[(int64_t)col * d.num_chunks + p.c] = sum;
  }
  EP_TIMING_MARK(EP_TK_COUNT, 7);
}

// --------------------------------------------------------------------------
// 2. column scans
// --------------------------------------------------------------------------
// One workgroup (256 threads) per column: exclusive prefix over chunks of
// chunk_hist[col][chunk].  Per-source-rank sums give
// num_tokens_per_expert[s][e], num_tokens_per_rank[s][d] and
// rank_prefix_matrix[s][d] (inclusive over s).
// LDS: rank_start[P+1] | wave sums (int64) [4]
constexpr int kScanThreads = 256;

// chunk_excl_t[chunk][col] receives the same offsets chunk-major, so that the
// rank kernel reads its chunk's E + P offsets contiguously.
__global__ __launch_bounds__(kScanThreads) void layout_scan_kernel(
    LayoutDims d, int32_t* __restrict__ chunk_hist, int32_t* __restrict__ chunk_excl_t,
    int32_t* __restrict__ col_total, int32_t* __restrict__ num_tokens_per_expert,
    int32_t* __restrict__ num_tokens_per_rank, int32_t* __restrict__ rank_prefix_matrix) {
  EP_TIMING_MARK(EP_TK_SCAN, 0);
  extern __shared__ int32_t lds[];
  int32_t* rank_start = lds;  // [P+1]: the column's prefix at each source rank's first chunk
  int64_t* wsum = (int64_t*)(lds + ((d.P + 2) & ~1));
  const int col = blockIdx.x;
  const int tid = threadIdx.x;
  const int nc = d.num_chunks;
  int32_t* v = chunk_hist + (int64_t)col * nc;

  for (int i = tid; i <= d.P; i += kScanThreads) rank_start[i] = 0;
  __syncthreads();

  int64_t carry = 0;
  for (int base = 0; base < nc; base += kScanThreads * 4) {
    int32_t x[4];
    int64_t tsum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = base + tid * 4 + q;
      x[q] = i < nc ? v[i] : 0;
      tsum += x[q];
    }
    int64_t tile_total;
    int64_t run = carry + block_excl_scan<kScanThreads>(tsum, wsum, &tile_total);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = base + tid * 4 + q;
      if (i < nc) {
        chunk_excl_t[(int64_t)i * d.ncols + col] = (int32_t)run;
        if (i % d.cpr == 0) rank_start[i / d.cpr] = (int32_t)run;  // chunks of a rank are consecutive
      }
      run += x[q];
    }
    carry += tile_total;
  }
  if (tid == 0) {
    col_total[col] = (int32_t)carry;
    rank_start[d.P] = (int32_t)carry;
  }
  __syncthreads();
  // per-source-rank sums of the column
  const auto rank_sum = [&](int s) { return rank_start[s + 1] - rank_start[s]; };

  if (col < d.E) {
    for (int s = tid; s < d.P; s += kScanThreads)
      num_tokens_per_expert[(int64_t)s * d.E + col] = rank_sum(s);
  } else if (col < d.E + d.P) {
    const int r = col - d.E;
    int64_t run = 0;
    for (int base = 0; base < d.P; base += kScanThreads) {
      const int s = base + tid;
      const int64_t val = s < d.P ? rank_sum(s) : 0;
      int64_t tile_total;
      const int64_t excl = run + block_excl_scan<kScanThreads>(val, wsum, &tile_total);
      if (s < d.P) {
        num_tokens_per_rank[s * d.P + r] = (int32_t)val;
        rank_prefix_matrix[s * d.P + r] = (int32_t)(excl + val);
      }
      run += tile_total;
    }
  }
}

// --------------------------------------------------------------------------
// 3. finalize
// --------------------------------------------------------------------------
// Host summary (int64): [0] total_rows  [1] total_pad (padding rows inside the
// windows)  [2] number of out-of-range ids  [3] sum of num_recv_tokens
// [4] tail rows of fixed windows  [5] rows dropped past fixed windows' ends
// [6, 6+P) num_expanded  [6+P, 6+2P) num_recv_tokens  [6+2P, 7+3P) window_row_base.
constexpr int kSummaryHeader = 6;
constexpr int kFinalizeThreads = 256;

struct FinalizeOut {
  int32_t* n_e;             // [E]
  int64_t* expert_offset;   // [P][El+1] window-local
  int64_t* num_expanded;    // [P]
  int64_t* window_row_base; // [P+1]
  int32_t* num_recv;        // [P]
  int64_t* recv_src_base;   // [P+1]
  int32_t* pad_base;        // [E+1]
  int32_t* pad_rows;        // [E*(A-1)] capacity
  int64_t* packed_base;     // [P+1] windows laid end to end (row_slot index space)
  int32_t* row_slot;        // [sum num_expanded] source slot u*K+j of each row, -1 padding
  int64_t* tail_base;       // [P+1] fixed windows: prefix of the tail row counts
  int64_t* summary;         // summary, see above (device copy, read by later kernels)
  int64_t* summary_host;    // the same, written straight into pinned host memory,
                            // followed by [7+3P] = seq, written last
  int64_t seq;              // the layout's sequence number (the host waits for it)
};

__device__ __forceinline__ void put_summary(const FinalizeOut& o, int i, int64_t v) {
  o.summary[i] = v;
  o.summary_host[i] = v;
}

// int64 words of LDS that finalize_body needs besides the column totals:
// g[E+1] int64 (global prefix of aligned sizes) | pad_base[E+1] int32 | wave sums [NT/64]
__host__ __device__ inline int finalize_lds_words(const LayoutDims& d, int nt) {
  return d.E + 1 + ((d.E + 2) >> 1) + 1 + nt / 64;
}

// The finalize step for a workgroup of NT threads (all of them call it), from
// the column totals col_total[E+P+1] (in LDS); lds64 holds
// finalize_lds_words(d, NT) int64 words.
template <int NT>
__device__ void finalize_body(const LayoutDims& d, const int32_t* col_total, const FinalizeOut& o, int64_t* lds64) {
  int64_t* g = lds64;
  int32_t* pb = (int32_t*)(lds64 + d.E + 1);
  int64_t* wsum = lds64 + d.E + 1 + ((d.E + 2) >> 1) + 1;
  const int tid = threadIdx.x;

  // aligned sizes p_e = ceil(n_e / A) * A and padding p_e - n_e, scanned over e
  int64_t carry_g = 0, carry_p = 0;
  for (int base = 0; base < d.E; base += NT) {
    const int e = base + tid;
    const int64_t n = e < d.E ? col_total[e] : 0;
    const int64_t pe = ((n + d.A - 1) / d.A) * d.A;
    int64_t tg, tp;
    const int64_t xg = block_excl_scan<NT>(pe, wsum, &tg);
    const int64_t xp = block_excl_scan<NT>(pe - n, wsum, &tp);
    if (e < d.E) {
      g[e] = carry_g + xg;
      pb[e] = (int32_t)(carry_p + xp);
      o.n_e[e] = (int32_t)n;
    }
    carry_g += tg;
    carry_p += tp;
  }
  if (tid == 0) {
    g[d.E] = carry_g;
    pb[d.E] = (int32_t)carry_p;
  }
  group_sync<NT>();

  // Fixed windows keep only window-local rows < cap: the padding rows of an
  // expert are [off + n, off + p) clipped to the window.
  if (d.cap > 0) {
    int64_t carry = 0;
    for (int base = 0; base < d.E; base += NT) {
      const int e = base + tid;
      int64_t pad = 0;
      if (e < d.E) {
        const int r = e / d.El;
        const int64_t off = g[e] - g[r * d.El];
        const int64_t n = col_total[e];
        const int64_t pe = ((n + d.A - 1) / d.A) * d.A;
        pad = min(off + pe, (int64_t)d.cap) - min(off + n, (int64_t)d.cap);
      }
      int64_t tp;
      const int64_t xp = block_excl_scan<NT>(pad, wsum, &tp);
      if (e < d.E) pb[e] = (int32_t)(carry + xp);
      carry += tp;
    }
    if (tid == 0) pb[d.E] = (int32_t)carry;
    group_sync<NT>();
  }

  // window sizes; packed bases are the global prefix at each window's first expert
  int64_t my_max = 0;
  for (int r = tid; r < d.P; r += NT) {
    const int64_t ne = g[(r + 1) * d.El] - g[r * d.El];
    o.num_expanded[r] = ne;
    put_summary(o, kSummaryHeader + r, ne);
    my_max = ne > my_max ? ne : my_max;
  }
  for (int e = tid; e <= d.E; e += NT) o.pad_base[e] = pb[e];
  // max over the workgroup (symmetric windows)
  for (int off = 32; off > 0; off >>= 1) {
    const int64_t y = __shfl_xor(my_max, off, 64);
    my_max = y > my_max ? y : my_max;
  }
  if ((tid & 63) == 0) wsum[tid >> 6] = my_max;
  group_sync<NT>();
  int64_t wmax = 0;
  for (int w = 0; w < NT / 64; ++w) wmax = wsum[w] > wmax ? wsum[w] : wmax;
  group_sync<NT>();

  for (int r = tid; r <= d.P; r += NT) {
    const int64_t base = d.cap > 0 ? (int64_t)r * d.cap : d.symmetric ? (int64_t)r * wmax : g[min(r, d.P) * d.El];
    o.window_row_base[r] = base;
    o.packed_base[r] = g[r * d.El];
    put_summary(o, kSummaryHeader + 2 * d.P + r, base);
  }
  for (int x = tid; x < d.P * (d.El + 1); x += NT) {
    const int r = x / (d.El + 1), l = x - r * (d.El + 1);
    o.expert_offset[x] = g[r * d.El + l] - g[r * d.El];
  }

  // receive-list bases
  int64_t carry_r = 0;
  for (int base = 0; base < d.P; base += NT) {
    const int r = base + tid;
    const int64_t nr = r < d.P ? col_total[d.E + r] : 0;
    int64_t tr;
    const int64_t xr = block_excl_scan<NT>(nr, wsum, &tr);
    if (r < d.P) {
      o.num_recv[r] = (int32_t)nr;
      o.recv_src_base[r] = carry_r + xr;
      put_summary(o, kSummaryHeader + d.P + r, nr);
    }
    carry_r += tr;
  }
  if (tid == 0) {
    o.recv_src_base[d.P] = carry_r;
    put_summary(o, 0, d.cap > 0 ? (int64_t)d.P * d.cap : d.symmetric ? (int64_t)d.P * wmax : g[d.E]);
    put_summary(o, 1, pb[d.E]);
    put_summary(o, 2, col_total[d.E + d.P]);
    put_summary(o, 3, carry_r);
  }

  // fixed windows: tail rows [min(ne, cap), cap) of each window, and the rows
  // past cap that are dropped
  int64_t carry_t = 0, carry_d = 0;
  if (d.cap > 0) {
    for (int base = 0; base < d.P; base += NT) {
      const int r = base + tid;
      const int64_t ne = r < d.P ? g[(r + 1) * d.El] - g[r * d.El] : 0;
      const int64_t tail = r < d.P ? d.cap - min(ne, (int64_t)d.cap) : 0;
      const int64_t drop = r < d.P ? max(ne - (int64_t)d.cap, (int64_t)0) : 0;
      int64_t tt, td;
      const int64_t xt = block_excl_scan<NT>(tail, wsum, &tt);
      (void)block_excl_scan<NT>(drop, wsum, &td);
      if (r < d.P) o.tail_base[r] = carry_t + xt;
      carry_t += tt;
      carry_d += td;
    }
  }
  if (tid == 0) {
    o.tail_base[d.P] = carry_t;
    put_summary(o, 4, carry_t);
    put_summary(o, 5, carry_d);
  }
  // Publish: every thread's summary writes reach the host before the sequence
  // number that the host spins on.
  __threadfence_system();
  group_sync<NT>();
  if (tid == 0) {
    o.summary_host[kSummaryHeader + 3 * d.P + 1] = o.seq;
    __threadfence_system();
  }
}

// LDS: finalize_body's words | column totals [E+P+1] int32
__global__ __launch_bounds__(kFinalizeThreads) void layout_finalize_kernel(
    LayoutDims d, const int32_t* __restrict__ col_total_g, FinalizeOut o) {
  extern __shared__ int64_t lds64[];
  int32_t* col_total = (int32_t*)(lds64 + finalize_lds_words(d, kFinalizeThreads));
  EP_TIMING_MARK(EP_TK_FINALIZE, 0);
  for (int i = threadIdx.x; i < d.ncols; i += kFinalizeThreads) col_total[i] = col_total_g[i];
  __syncthreads();
  finalize_body<kFinalizeThreads>(d, col_total, o, lds64);
  EP_TIMING_MARK(EP_TK_FINALIZE, 7);
}

// --------------------------------------------------------------------------
// 4. stable ranks
// --------------------------------------------------------------------------
struct RankOut {
  int32_t* dst_slot;      // [T][K]
  int32_t* dst_row;       // [T][K]
  int32_t* row_slot;      // [sum num_expanded], packed window order
  int32_t* send_head;     // [T][P]
  int32_t* recv_src_idx;  // [sum num_recv]
  int32_t* pad_rows;      // [total padding] global rows, expert-major
};

struct RankIn {
  const int32_t* chunk_excl_t;     // [chunk][E + P + 1]
  const int32_t* n_e;              // [E]
  const int32_t* pad_base;         // [E + 1]
  const int64_t* expert_offset;    // [P][El + 1]
  const int64_t* window_row_base;  // [P + 1]
  const int64_t* packed_base;      // [P + 1]
  const int64_t* recv_src_base;    // [P + 1]
};

// Per-wave counts of the keys of tokens [t0, t0 + nt) of a chunk: cnt_e[e]
// per expert, cnt_r[r] per destination rank of each token's first slot on
// r (ballot-counted, see wave_count).
__device__ __forceinline__ void count_wave_keys(const LayoutDims& d, const int32_t* ex, int t0, int nt, int lane,
                                                int32_t* cnt_e, int32_t* cnt_r) {
  const int first = t0 * d.K, total = max(nt, 0) * d.K;
  for (int base = 0; base < total; base += kWave) {  // uniform trip count per wave
    const int i = base + lane;
    const int s = first + i;
    const int e = i < total ? ex[s] : -1;
    int col_r = -1;
    if (e >= 0) {
      const int t = s / d.K, j = s - t * d.K, r = e / d.El;
      if (first_on_rank(d, ex, t, j, r)) col_r = r;
    }
    wave_count(cnt_e, e >= 0 ? e : -1, d.E, d.ebits, lane);
    wave_count(cnt_r, col_r, d.P, d.pbits, lane);
  }
}

// Stable positions of tokens [t0, t0 + nt) of chunk p, walked by one wave 64
// slots at a time in (u, j) order.  cnt_e[e] / cnt_r[r] hold the wave's next
// position per expert / destination rank (its starting offsets on entry; they
// advance as slots are ranked; the "none" keys E and P are never written).
// Writes dst_slot, dst_row, row_slot, recv_src_idx; pos[s] gets each slot's
// receive-list position, -1 where the slot is not its token's first on its
// rank.
__device__ __forceinline__ void rank_wave_tokens(const LayoutDims& d, const ChunkPos& p, const int32_t* ex, int t0,
                                                 int nt, int lane, int32_t* cnt_e, int32_t* cnt_r, int32_t* pos,
                                                 const RankIn& in, const RankOut& o) {
  const int first_slot = t0 * d.K, total = max(nt, 0) * d.K;
  for (int base = 0; base < total; base += kWave) {  // uniform trip count per wave
    const int i = base + lane;
    const bool live = i < total;
    const int s = first_slot + i;
    const int e = live ? ex[s] : -1;
    const int t = s / d.K, j = s - t * d.K;
    const int r = e >= 0 ? e / d.El : d.P;
    const bool first = e >= 0 && first_on_rank(d, ex, t, j, r);
    const uint32_t key_e = e >= 0 ? (uint32_t)e : (uint32_t)d.E;
    const uint32_t key_r = first ? (uint32_t)r : (uint32_t)d.P;
    const uint64_t pe = match_any(key_e, d.ebits);
    const uint64_t pr = match_any(key_r, d.pbits);
    const int be = e >= 0 ? cnt_e[key_e] : 0, br = first ? cnt_r[key_r] : 0;
    __builtin_amdgcn_wave_barrier();
    if (e >= 0 && lane == 63 - __builtin_clzll(pe)) cnt_e[key_e] = be + __builtin_popcountll(pe);
    if (first && lane == 63 - __builtin_clzll(pr)) cnt_r[key_r] = br + __builtin_popcountll(pr);
    __builtin_amdgcn_wave_barrier();
    if (live) {
      const int64_t u = p.u0 + t;
      if (e >= 0) {
        const int64_t slot = in.expert_offset[(int64_t)r * (d.El + 1) + (e - r * d.El)] + be + count_below(pe);
        o.dst_slot[u * d.K + j] = (int32_t)slot;
        // a row past a fixed window's end is dropped
        o.dst_row[u * d.K + j] = (d.cap > 0 && slot >= d.cap) ? -1 : (int32_t)(in.window_row_base[r] + slot);
        o.row_slot[in.packed_base[r] + slot] = (int32_t)(u * d.K + j);
      } else {
        o.dst_slot[u * d.K + j] = -1;
        o.dst_row[u * d.K + j] = -1;
      }
      int32_t sh = -1;
      if (first) {
        sh = br + count_below(pr);
        o.recv_src_idx[in.recv_src_base[r] + sh] = p.t0 + t;
      }
      pos[s] = sh;
    }
  }
}

// Padding rows [first + n_e, first + ceil(n_e / A) * A) of experts e_begin,
// e_begin + e_stride, ... (clipped to fixed windows by pad_base): pad_rows
// (global row) and row_slot = -1; threads first, first + stride, ...
__device__ __forceinline__ void padding_rows(const LayoutDims& d, int e_begin, int e_stride, int first, int stride,
                                             const RankIn& in, const RankOut& o) {
  for (int e = e_begin; e < d.E; e += e_stride) {
    const int r = e / d.El, l = e - r * d.El;
    const int n = in.n_e[e];
    const int b0 = in.pad_base[e], npad = in.pad_base[e + 1] - b0;
    const int64_t local = in.expert_offset[(int64_t)r * (d.El + 1) + l] + n;
    for (int i = first; i < npad; i += stride) {
      o.pad_rows[b0 + i] = (int32_t)(in.window_row_base[r] + local + i);
      o.row_slot[in.packed_base[r] + local + i] = -1;
    }
  }
}

// Also writes the padding rows of its share of the experts (wave by wave, see below).
// LDS: per-wave counters [W][E+P+1] (experts, then ranks) | staged experts
//      [64*K] | send positions [64*K]
__global__ __launch_bounds__(kLayoutThreads) void layout_rank_kernel(LayoutDims d,
                                                                     const int64_t* __restrict__ topk_idx,
                                                                     RankIn in, RankOut o) {
  extern __shared__ int32_t lds[];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid >> 6;
  int32_t* cnt_all = lds;  // [W][ncols]
  int32_t* ex = cnt_all + kLayoutWaves * d.ncols;
  int32_t* pos = ex + kChunk * d.K;
  EP_TIMING_MARK(EP_TK_RANK, 0);

  if (blockIdx.x < d.num_chunks) {  // token part: one chunk per workgroup
    const ChunkPos p = chunk_pos(d, blockIdx.x);
    for (int i = tid; i < kLayoutWaves * d.ncols; i += kLayoutThreads) cnt_all[i] = 0;
    stage_chunk_experts(d, p, topk_idx, ex, tid, kLayoutThreads);
    __syncthreads();

    // this wave's slots: tokens [t0, t0 + nt) of the chunk
    const int t0 = wv * kTokensPerWave;
    const int nt = max(0, min(kTokensPerWave, p.n - t0));
    int32_t* cnt_e = cnt_all + wv * d.ncols;
    int32_t* cnt_r = cnt_e + d.E;

    // 1. per-wave counts per key
    count_wave_keys(d, ex, t0, nt, lane, cnt_e, cnt_r);
    __syncthreads();

    // 2. starting position of every wave per key: the chunk's scanned offset
    //    plus the counts of the earlier waves
    const int32_t* my_excl = in.chunk_excl_t + (int64_t)p.c * d.ncols;
    for (int k = tid; k < d.E + d.P; k += kLayoutThreads) {
      int32_t run = my_excl[k];
#pragma unroll
      for (int w = 0; w < kLayoutWaves; ++w) {
        const int32_t n = cnt_all[w * d.ncols + k];
        cnt_all[w * d.ncols + k] = run;
        run += n;
      }
    }
    __syncthreads();

    // 3. stable ranks inside the wave
    rank_wave_tokens(d, p, ex, t0, nt, lane, cnt_e, cnt_r, pos, in, o);
    __syncthreads();

    // send_head rows of the chunk: one contiguous int32 range, -1 where not
    // sent; then each token's first slot on a rank writes its position (the
    // barrier orders the two writes of the same element)
    int32_t* out = o.send_head + p.u0 * d.P;
    for (int q = tid; q < p.n * d.P; q += kLayoutThreads) out[q] = -1;
    __syncthreads();
    for (int i = tid; i < p.n * d.K; i += kLayoutThreads) {
      const int sh = pos[i];
      if (sh >= 0) out[(i / d.K) * d.P + ex[i] / d.El] = sh;
    }
  }
  // wave w of workgroup b: experts b * W + w, then every grid * W further; its lanes the rows
  padding_rows(d, blockIdx.x * kLayoutWaves + wv, gridDim.x * kLayoutWaves, lane, kWave, in, o);
  EP_TIMING_MARK(EP_TK_RANK, 7);
}

// --------------------------------------------------------------------------
// small batches: the whole layout in one workgroup
// --------------------------------------------------------------------------
constexpr int kSmallThreads = 1024;
constexpr int kSmallChunks = kSmallThreads / kWave;  // one wave per chunk
constexpr size_t kSmallLdsMax = 64 * 1024;           // bytes: beyond this the four-kernel path runs
// Slots (tokens x top-k) of the fullest chunk up to which the one-workgroup
// layout runs: one wave counts and ranks a whole chunk there, where the
// four-kernel path spreads a chunk over four waves.  Measured on MI355X at
// 8 chunks: 128 slots a chunk is 6-12 us faster in one workgroup, 256 is even
// and 384 or more is slower.
constexpr int kSmallMaxChunkSlots = 256;

// LDS of layout_small_kernel, in bytes:
//   int32: histograms [C][ncols] | column totals [ncols] | staged experts
//          [C][64*K] | send positions [C][64*K] | rank bit rows [T][ceil(P/32)]
//   int64 (8-byte aligned): finalize_body's words
__host__ __device__ inline size_t small_lds_int32_words(const LayoutDims& d) {
  const size_t C = (size_t)d.num_chunks;
  const size_t T = (size_t)d.P * (size_t)d.S;
  return C * d.ncols + d.ncols + 2 * C * kChunk * d.K + T * ((d.P + 31) / 32);
}
__host__ __device__ inline size_t small_lds_bytes(const LayoutDims& d) {
  return ((small_lds_int32_words(d) + 1) / 2) * 8 + (size_t)finalize_lds_words(d, kWave) * 8;
}

// The four steps in order, with workgroup barriers between them: wave c
// counts chunk c (its histogram is one LDS row), thread `col` scans column col
// over the chunks in order (source ranks' chunks are consecutive), the
// finalize step runs on the column totals, and wave c ranks chunk c from its
// scanned offsets.  Launched with one workgroup when num_chunks <= 16.
__global__ __launch_bounds__(kSmallThreads) void layout_small_kernel(
    LayoutDims d, const int64_t* __restrict__ topk_idx, uint8_t* __restrict__ is_token_in_rank,
    int32_t* __restrict__ num_tokens_per_expert, int32_t* __restrict__ num_tokens_per_rank,
    int32_t* __restrict__ rank_prefix_matrix, FinalizeOut fo, RankIn in, RankOut o) {
  extern __shared__ int64_t lds_small[];
  const int C = d.num_chunks;
  const int words = (d.P + 31) >> 5;
  const int T = d.P * d.S;
  const int slots = kChunk * d.K;
  int32_t* hist = (int32_t*)lds_small;                 // [C][ncols]
  int32_t* col_total = hist + C * d.ncols;             // [ncols]
  int32_t* ex_all = col_total + d.ncols;               // [C][64*K]
  int32_t* pos_all = ex_all + C * slots;               // [C][64*K]
  uint32_t* rmask = (uint32_t*)(pos_all + C * slots);  // [T][words]
  int64_t* fin = lds_small + (small_lds_int32_words(d) + 1) / 2;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid >> 6;
  EP_TIMING_MARK(EP_TK_SMALL, 0);

  for (int i = tid; i < C * d.ncols; i += kSmallThreads) hist[i] = 0;
  for (int i = tid; i < T * words; i += kSmallThreads) rmask[i] = 0;
  for (int q = tid; q < T * d.P; q += kSmallThreads) o.send_head[q] = -1;  // positions come in step 4
  for (int c = 0; c < C; ++c) stage_chunk_experts(d, chunk_pos(d, c), topk_idx, ex_all + c * slots, tid, kSmallThreads);
  __syncthreads();
  EP_TIMING_MARK(EP_TK_SMALL, 1);

  // 1. counts, one wave per chunk
  if (wv < C) {
    const ChunkPos p = chunk_pos(d, wv);
    count_wave_tokens(d, ex_all + wv * slots, 0, p.n, lane, hist + wv * d.ncols, rmask + p.u0 * words, words);
  }
  __syncthreads();
  EP_TIMING_MARK(EP_TK_SMALL, 2);
  write_itr_rows(d, rmask, words, T, is_token_in_rank, tid, kSmallThreads);

  // 2. column scans over the chunks, in place; per-source-rank sums
  for (int col = tid; col < d.ncols; col += kSmallThreads) {
    int32_t run = 0;
    for (int s = 0; s < d.P; ++s) {
      int32_t rank_sum = 0;
      for (int cc = 0; cc < d.cpr; ++cc) {
        int32_t* h = hist + (s * d.cpr + cc) * d.ncols + col;
        const int32_t v = *h;
        *h = run;
        run += v;
        rank_sum += v;
      }
      if (col < d.E) {
        num_tokens_per_expert[(int64_t)s * d.E + col] = rank_sum;
      } else if (col < d.E + d.P) {
        num_tokens_per_rank[s * d.P + (col - d.E)] = rank_sum;
        rank_prefix_matrix[s * d.P + (col - d.E)] = run;  // inclusive over source ranks
      }
    }
    col_total[col] = run;
  }
  __syncthreads();
  EP_TIMING_MARK(EP_TK_SMALL, 3);

  // 3. finalize (publishes the host summary before the ranks are written), on
  //    one wave: its scans need no workgroup barriers
  if (wv == 0) finalize_body<kWave>(d, col_total, fo, fin);
  __syncthreads();
  EP_TIMING_MARK(EP_TK_SMALL, 4);

  // 4. stable ranks, one wave per chunk, starting from the chunk's scanned offsets
  if (wv < C) {
    const ChunkPos p = chunk_pos(d, wv);
    int32_t* cnt = hist + wv * d.ncols;
    rank_wave_tokens(d, p, ex_all + wv * slots, 0, p.n, lane, cnt, cnt + d.E, pos_all + wv * slots, in, o);
  }
  __syncthreads();
  EP_TIMING_MARK(EP_TK_SMALL, 5);
  for (int c = 0; c < C; ++c) {
    const ChunkPos p = chunk_pos(d, c);
    const int32_t* pos = pos_all + c * slots;
    const int32_t* ex = ex_all + c * slots;
    for (int i = tid; i < p.n * d.K; i += kSmallThreads) {
      const int sh = pos[i];
      if (sh >= 0) o.send_head[(p.u0 + i / d.K) * d.P + ex[i] / d.El] = sh;
    }
  }
  padding_rows(d, wv, kSmallThreads / kWave, lane, kWave, in, o);  // wave w: experts w, w + 16, ...
  EP_TIMING_MARK(EP_TK_SMALL, 7);
}

}  // namespace ep
