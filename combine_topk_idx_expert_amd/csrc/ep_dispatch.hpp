// ep_dispatch.hpp -- dispatch (pack/expand) and combine kernels.
//
// Dispatch: every token row of x is read from HBM once and written to each of
// its K expanded rows (TileLang tutorial ch. 38, sections 2.2 and 4.3: the
// local copy into the receive buffer; here every virtual rank is local).  With
// FP8 the row is quantised once per token -- amax per 128 channels, scale =
// amax / 448, E4M3 codes of x / scale (section 3.6) -- and the codes are
// written K times.
//
// Combine: every token gathers its K expert rows and reduces them in a fixed
// slot order in fp32, adds the optional bias (section 3.3), then rounds to
// bf16 (section 4.5).
//
// Work split: one wave per (source token, column part).  Partitioning by source
// token keeps skewed routing balanced: a hot expert means more rows written,
// not a longer wave.  A lane moves 16-byte vectors; 64 lanes cover 1 KiB of a
// bf16 row per vector.
#pragma once

#include "ep_device.hpp"

namespace ep {

// Rows are split into column parts of NC 16-byte chunks per lane (NC KiB of
// bf16 per wave); a wave handles one (row, part).  Short-lived waves that
// each move a few KiB keep more of HBM's write bandwidth than long-lived
// waves that move whole rows (measured on MI355X).
//
// Row metadata (weight, source slot) is written in row order by waves that
// each own 64 consecutive expanded rows, so every store is coalesced; that
// measured faster than letting the token waves scatter it.  The fp8 scales of
// a row, by contrast, are written by the token waves next to its codes, which
// measured faster than a separate row-order pass.
struct DispatchArgs {
  const uint16_t* x;             // [T][H] bf16
  const float* w;                // [T][K]           (fresh only)
  const int32_t* dst_row;        // [T][K] global row, -1 unused
  const int32_t* pad_rows;       // [total_pad] global rows
  const int32_t* row_slot;       // [sum_expanded] source slot u*K+j, -1 padding (packed order)
  const int64_t* packed_base;    // [P+1] packed start of each window
  const int64_t* window_row_base;  // [P+1] global start of each window
  void* recv_x;                  // [rows][H] bf16 | u8
  float* recv_scales;            // [rows][H/128]    (fp8)
  float* tok_scales;             // [T][H/128]       (fp8 scratch: scales per token)
  float* recv_weights;           // [rows]           (fresh only)
  int32_t* recv_meta;            // [rows][2]        (fresh only)
  int T, K, H, P;
  int total_pad, sum_expanded;
  int split;                     // parts per row = ceil((H / 8) / (64 * NC))
  int zero_pad, symmetric;
  // fixed windows of cap rows (cap > 0); the row counts are known on the device only
  int cap;
  int zero_waves;                // waves that share the padding / tail rows
  const int64_t* counts;         // layout summary: [1] padding rows, [4] tail rows
  const int64_t* tail_base;      // [P+1]
  const int64_t* num_expanded;   // [P]
  const uint8_t* x_codes;        // [T][H] pre-quantised E4M3 input (tok_scales then holds its scales)
  int scales_cm;                 // fp8 scales column-major: [H/128][scale_rows]
  int64_t scale_rows;            // rows of the expanded tensors (the column-major stride)
};

// Wave-uniform global wave index of the calling lane.
__device__ __forceinline__ int wave_index() {
  return uniform((int)(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)));
}

// Global row of the p-th row when the windows are laid end to end.
__device__ __forceinline__ int64_t packed_to_row(const DispatchArgs& a, int64_t p) {
  if (!a.symmetric) return p;  // packed windows: the same numbering
  int lo = 0, hi = a.P;        // last window with packed_base <= p
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.packed_base[mid] <= p) lo = mid; else hi = mid;
  }
  return a.window_row_base[lo] + (p - a.packed_base[lo]);
}

// E4M3 codes of 8 bf16 values (packed in v) for one 128-channel block with
// scale `scale`: code = E4M3FN_RNE(x / scale) with IEEE fp32 division; a block
// whose amax is 0 has scale 0 and gets the signed zero of each input.
// Little-endian bytes in two words.
__device__ __forceinline__ u32x2 quantize8(u32x4 v, float scale, bool zero_block) {
  u32x2 out;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t p0 = v[2 * h], p1 = v[2 * h + 1];
    if (!zero_block) {
      out[h] = e4m3x4_hw(bf16_lo(p0) / scale, bf16_hi(p0) / scale, bf16_lo(p1) / scale, bf16_hi(p1) / scale);
    } else {
      out[h] = ((p0 >> 8) & 0x80u) | ((p0 >> 16) & 0x8000u) | (((p1 >> 8) & 0x80u) << 16) |
               ((p1 & 0x80000000u));
    }
  }
  return out;
}

// UE8M0 exponent byte of a 32-channel block from m, the largest |x| bf16
// bit pattern of the block: the smallest k in [-127, 127] with
// 448 * 2^k >= amax, biased by 127.  With amax = M * 2^E (M in [1, 2)) and
// 448 = 1.75 * 2^8, that is k = E - 8, or E - 7 when M > 1.75 (bf16 mantissa
// above 0x60); zero and subnormal maxima give k = -127 (byte 0), a
// non-finite maximum the UE8M0 NaN 0xFF.
__device__ __forceinline__ uint32_t ue8m0_exponent(uint32_t m) {
  if (m >= 0x7F80u) return 0xFFu;
  const int ef = (int)(m >> 7);
  if (ef == 0) return 0u;
  const int t = ef - 8 + ((m & 0x7Fu) > 0x60u ? 1 : 0);
  return t < 0 ? 0u : (uint32_t)t;
}

// E4M3 codes of 8 bf16 values for a power-of-two scale 2^k, given inv =
// 2^-k (an exact normal float): x * 2^-k is the correctly rounded x / 2^k.
__device__ __forceinline__ u32x2 quantize8_pow2(u32x4 v, float inv, bool zero_block) {
  u32x2 out;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t p0 = v[2 * h], p1 = v[2 * h + 1];
    if (!zero_block) {
      out[h] = e4m3x4_hw(bf16_lo(p0) * inv, bf16_hi(p0) * inv, bf16_lo(p1) * inv, bf16_hi(p1) * inv);
    } else {
      out[h] = ((p0 >> 8) & 0x80u) | ((p0 >> 16) & 0x8000u) | (((p1 >> 8) & 0x80u) << 16) |
               ((p1 & 0x80000000u));
    }
  }
  return out;
}

// Codes of 8 bf16 values (packed in v) of a block whose maximum is not
// finite, byte order as in quantize8.  A NaN block (some |x| is NaN) codes
// every value 0x7F; an Inf block codes its infinities 0x7F (Inf / Inf is NaN)
// and every finite value as the signed zero of x / Inf.  NaN codes carry a
// clear sign bit, so the result does not depend on which NaN a division makes.
__device__ __forceinline__ u32x2 nonfinite_codes8(u32x4 v, bool nan_block) {
  u32x2 out;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t w = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t word = v[2 * h + (k >> 1)];
      const uint32_t b = (k & 1) ? (word >> 16) : (word & 0xFFFFu);
      const uint32_t code = (nan_block || (b & 0x7FFFu) >= 0x7F80u) ? 0x7Fu : ((b >> 8) & 0x80u);
      w |= code << (8 * k);
    }
    out[h] = w;
  }
  return out;
}

// Row of the k-th tail row of fixed windows: tail rows are the last
// tail_base[r+1] - tail_base[r] rows of window r.
__device__ __forceinline__ int64_t tail_row(const DispatchArgs& a, int64_t k) {
  int lo = 0, hi = a.P;  // last window with tail_base <= k
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.tail_base[mid] <= k) lo = mid; else hi = mid;
  }
  const int64_t len = a.tail_base[lo + 1] - a.tail_base[lo];
  return (int64_t)lo * a.cap + (a.cap - len) + (k - a.tail_base[lo]);
}

// Source slot of output row g of fixed windows: -1 for padding and tail rows.
__device__ __forceinline__ int fixed_row_slot(const DispatchArgs& a, int64_t g) {
  const int r = (int)(g / a.cap);
  const int64_t l = g - (int64_t)r * a.cap;
  return l < a.num_expanded[r] ? a.row_slot[a.packed_base[r] + l] : -1;
}

// Work items, in grid order:
//   [0, T*split)                      payload of (token, part)
//   exact windows:
//   [.., + total_pad*split)           zero payload of (padding row, part)   if zero_pad
//   [.., + ceil(sum_expanded / 64))   row metadata of 64 rows               if META
//   fixed windows (cap > 0), counts read on the device:
//   [.., + zero_waves)                waves striding over whole padding rows (if zero_pad)
//                                     and tail rows
//   [.., + ceil(P * cap / 64))        row metadata of 64 rows               if META
// NC: 16-byte chunks per lane per wave (the column part is 64 * NC chunks).
// Store pacing: after each destination row, wait until at most
// EP_DISPATCH_ROWS_IN_FLIGHT - 1 earlier rows' stores of this wave are still
// outstanding.  Fewer scattered writes in flight keep HBM more efficient than
// letting every wave burst all K rows (measured on MI355X); 0 disables.
// Payload stores of dispatch are nontemporal: the expanded rows are consumed by
// a later kernel, and streaming them past the caches measured slightly faster.
template <typename V>
__device__ __forceinline__ void stream_store(V* p, V v) {
  __builtin_nontemporal_store(v, p);
}

#ifndef EP_DISPATCH_ROWS_IN_FLIGHT
#define EP_DISPATCH_ROWS_IN_FLIGHT 1
#endif
template <int NC>
__device__ __forceinline__ void store_pacing() {
  if constexpr (EP_DISPATCH_ROWS_IN_FLIGHT > 0) {
    constexpr int want = NC * (EP_DISPATCH_ROWS_IN_FLIGHT - 1);
    constexpr int allow = want < 15 ? want : 15;  // the vmcnt field holds 0..15 here
    __builtin_amdgcn_s_waitcnt(0x0F70 | allow);  // vmcnt(allow), expcnt/lgkmcnt unchanged
  }
}

// fp8 rows with row-major scales: each 16-byte chunk position issues its code
// store, then (lanes 0..3) its scale store, so a row is 2 * NC stores.  Stores
// complete in issue order; this pacing waits for the row's code stores only,
// leaving the last scale store in flight.  Used for pre-quantised input, where
// it measured 2-5% faster on MI355X than waiting for every store; with the
// quantisation in the wave it ranged from 1% faster to 2% slower at the
// DeepSeek-V3 shape (1-2% faster under Zipf routing), so those waves keep the
// plain pacing.
template <int NC>
__device__ __forceinline__ void store_pacing_fp8() {
  if constexpr (EP_DISPATCH_ROWS_IN_FLIGHT > 0) {
    constexpr int want = 2 * NC * (EP_DISPATCH_ROWS_IN_FLIGHT - 1) + 1;
    constexpr int allow = want < 15 ? want : 15;
    __builtin_amdgcn_s_waitcnt(0x0F70 | allow);
  }
}

// scales: fp8 row-major scales to zero with the row (null: none); with UE8M0
// they are the row's H/32 exponent bytes, zeroed four per lane (lanes 0..3).
template <int NC, bool FP8, bool UE8M0 = false>
__device__ __forceinline__ void zero_row_part(uint8_t* recv, int64_t row, int part, int64_t out_row_bytes,
                                              int nchunk, int lane, float* scales) {
  if constexpr (FP8 && UE8M0) {
    if (scales) {
      const int nw = nchunk >> 4;  // 32-bit words of exponent bytes per row
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int wd = ((part * NC * kWave + c * kWave) >> 4) + lane;
        if (lane < 4 && wd < nw) ((uint32_t*)scales)[row * nw + wd] = 0u;
      }
    }
  } else if constexpr (FP8) {
    if (scales) {
      const int nblk = nchunk >> 4;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int blk = (part * NC * kWave + c * kWave) / 16 + lane;
        if (lane < 4 && blk < nblk) scales[row * nblk + blk] = 0.0f;
      }
    }
  }
  uint8_t* dst = recv + row * out_row_bytes;
  const int tile = part * NC * kWave;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int q = tile + c * kWave + lane;  // 16-byte bf16 chunk index
    if (q < nchunk) {
      if constexpr (FP8)
        stream_store((u32x2*)dst + q, u32x2{0, 0});
      else
        stream_store((u32x4*)dst + q, u32x4{0, 0, 0, 0});
    }
  }
}

// PREQ: the input is already E4M3 codes (x_codes) with their scales; rows get
// the bytes unchanged (FP8 only).  FIXED: fixed windows (a.cap > 0); exact
// windows get kernels without the fixed-window paths (measured: carrying them
// slowed the exact fp8 dispatch by ~15%).
// UE8M0: fp8 scales as one exponent byte per 32 channels (row-major bytes
// [rows][H/32]) instead of one fp32 per 128 channels; fused quantisation only.
template <int NC, bool FP8, bool META, bool PREQ, bool FIXED, bool UE8M0 = false>
__global__ __launch_bounds__(1024) void dispatch_kernel(DispatchArgs a) {
  static_assert(!PREQ || FP8, "pre-quantised input is fp8");
  static_assert(!UE8M0 || (FP8 && !PREQ), "UE8M0 scales come from the fused quantisation");
  const int gw = wave_index();
  const int lane = lane_id();
  const int nchunk = a.H >> 3;  // 16-byte bf16 chunks per row
  const int64_t out_row_bytes = FP8 ? (int64_t)a.H : (int64_t)a.H * 2;
  uint8_t* recv = (uint8_t*)a.recv_x;
  const int token_items = a.T * a.split;
  const int pad_items = FIXED ? a.zero_waves : a.zero_pad ? a.total_pad * a.split : 0;
  EP_TIMING_MARK(EP_TK_DISPATCH, 0);

  if (gw < token_items) {
    const int u = gw / a.split;
    const int part = gw - u * a.split;
    const int tile = part * NC * kWave;
    const u32x4* src = (const u32x4*)(a.x + (int64_t)u * a.H);
    // All K destination rows in one vector load (lane j holds row j), issued
    // before any store: the stores could alias the table as far as the compiler
    // knows, so per-slot loads inside the store loop would each wait for memory.
    const int my_row = lane < a.K ? a.dst_row[(int64_t)u * a.K + lane] : -1;
    u32x4 v[NC];
    u32x2 codes[NC];
    float pq_sc[NC];  // pre-quantised: lanes 0..3 load the part's four block scales up front
    if constexpr (PREQ) {
      const int nb = a.H >> 7;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int blk = (tile + c * kWave) / 16 + lane;
        pq_sc[c] = (!a.scales_cm && lane < 4 && blk < nb) ? a.tok_scales[(int64_t)u * nb + blk] : 0.0f;
      }
    }
    if constexpr (PREQ) {  // 8 code bytes per 16-byte bf16 chunk position
      const u32x2* csrc = (const u32x2*)(a.x_codes + (int64_t)u * a.H);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int q = tile + c * kWave + lane;
        codes[c] = q < nchunk ? __builtin_nontemporal_load(csrc + q) : u32x2{0, 0};
      }
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int q = tile + c * kWave + lane;
        v[c] = q < nchunk ? __builtin_nontemporal_load(src + q) : u32x4{0, 0, 0, 0};
      }
    }
    if constexpr (!FP8) {
      for (int j = 0; j < a.K; ++j) {
        const int row = __builtin_amdgcn_readlane(my_row, j);
        if (row < 0) continue;
        u32x4* dst = (u32x4*)(recv + (int64_t)row * out_row_bytes);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int q = tile + c * kWave + lane;
          if (q < nchunk) stream_store(dst + q, v[c]);
        }
        store_pacing<NC>();
      }
    } else {
      const int nblk = a.H >> 7;
      // Row-major scales: the waves also write each row's scales, lanes 0..3
      // holding the scales of the part's four 128-channel blocks (computed
      // here, or the caller's, loaded up front).  Column-major scales are
      // written afterwards by dispatch_scales_cm_kernel from tok_scales.
      const bool fused_scales = !a.scales_cm;
      float sc[NC];
      uint32_t ew[NC];  // UE8M0: lanes 0..3 hold four exponent bytes each
#pragma unroll
      for (int c = 0; c < NC && PREQ; ++c) sc[c] = pq_sc[c];
#pragma unroll
      for (int c = 0; c < NC && UE8M0; ++c) {
        uint32_t m = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) m = max(m, max(v[c][k] & 0x7FFFu, (v[c][k] >> 16) & 0x7FFFu));
        m = quad_max_u32(m);  // 4 lanes = one 32-channel block
        const uint32_t eb = ue8m0_exponent(m);
        const float inv = __uint_as_float((254u - min(eb, 247u)) << 23);  // 2^(127 - eb)
        codes[c] = quantize8_pow2(v[c], inv, m == 0);
        if (__builtin_expect(m >= 0x7F80u, 0)) codes[c] = nonfinite_codes8(v[c], m > 0x7F80u);
        // word w of the part's 16 blocks holds blocks 4w..4w+3, i.e. the bytes of lanes 16w + 4i
        const int w16 = (lane & 3) * 16;
        ew[c] = (uint32_t)__shfl((int)eb, w16) | ((uint32_t)__shfl((int)eb, w16 + 4) << 8) |
                ((uint32_t)__shfl((int)eb, w16 + 8) << 16) | ((uint32_t)__shfl((int)eb, w16 + 12) << 24);
      }
#pragma unroll
      for (int c = 0; c < NC && !PREQ && !UE8M0; ++c) {
        uint32_t m = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) m = max(m, max(v[c][k] & 0x7FFFu, (v[c][k] >> 16) & 0x7FFFu));
        m = row16_max_u32(m);  // one DPP row = 16 lanes = one 128-channel block
        // |x| patterns order like the magnitudes, NaN above +Inf, so m is the
        // block maximum with NaN propagated; a non-finite maximum gives the
        // scale 0x7FC00000 (NaN) or +Inf and the codes of nonfinite_codes8
        const bool nonfinite = m >= 0x7F80u;
        float scale = __uint_as_float(m << 16) / 448.0f;
        if (nonfinite) scale = __uint_as_float(m > 0x7F80u ? 0x7FC00000u : 0x7F800000u);
        codes[c] = quantize8(v[c], scale, m == 0);
        if (__builtin_expect(nonfinite, 0)) codes[c] = nonfinite_codes8(v[c], m > 0x7F80u);
        const int q = tile + c * kWave + lane;
        if (!fused_scales && (lane & 15) == 0 && q < nchunk) a.tok_scales[(int64_t)u * nblk + (q >> 4)] = scale;
        sc[c] = __shfl(scale, (lane & 3) * 16, kWave);
      }
      for (int j = 0; j < a.K; ++j) {
        const int row = __builtin_amdgcn_readlane(my_row, j);
        if (row < 0) continue;
        u32x2* dst = (u32x2*)(recv + (int64_t)row * out_row_bytes);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int q = tile + c * kWave + lane;
          if (q < nchunk) stream_store(dst + q, codes[c]);
          if constexpr (UE8M0) {
            const int wd = ((tile + c * kWave) >> 4) + lane;  // 32-bit word of exponent bytes
            if (lane < 4 && wd < (nchunk >> 4)) ((uint32_t*)a.recv_scales)[(int64_t)row * (nchunk >> 4) + wd] = ew[c];
          } else {
            const int blk = (tile + c * kWave) / 16 + lane;
            if (fused_scales && lane < 4 && blk < nblk) a.recv_scales[(int64_t)row * nblk + blk] = sc[c];
          }
        }
        if (PREQ && fused_scales)
          store_pacing_fp8<NC>();
        else
          store_pacing<NC>();
      }
    }
  } else if (gw < token_items + pad_items) {
    float* zero_scales = (FP8 && !a.scales_cm) ? a.recv_scales : nullptr;  // fused scales only
    if constexpr (!FIXED) {
      const int p = (gw - token_items) / a.split;
      const int part = (gw - token_items) - p * a.split;
      zero_row_part<NC, FP8, UE8M0>(recv, a.pad_rows[p], part, out_row_bytes, nchunk, lane, zero_scales);
    } else {
      // Fixed windows: padding rows (if asked) then tail rows (always),
      // counted on the device.  Wave w zeroes whole rows z = z0 + w, z0 + w +
      // zero_waves, ...: the waves together sweep the list front to back.
      // Tail rows are found by one search, then followed window by window.
      const int64_t npad = a.counts[1], ntail = a.counts[4];
      const int64_t z0 = a.zero_pad ? 0 : npad;
      int win = -1;
      for (int64_t z = z0 + (gw - token_items); z < npad + ntail; z += a.zero_waves) {
        int64_t row;
        if (z < npad) {
          row = a.pad_rows[z];
        } else {
          const int64_t k = z - npad;
          if (win < 0) {
            row = tail_row(a, k);
            win = (int)(row / a.cap);
          }
          while (a.tail_base[win + 1] <= k) ++win;
          row = (int64_t)win * a.cap + a.cap - (a.tail_base[win + 1] - a.tail_base[win]) + (k - a.tail_base[win]);
        }
        for (int part = 0; part < a.split; ++part)
          zero_row_part<NC, FP8, UE8M0>(recv, row, part, out_row_bytes, nchunk, lane, zero_scales);
      }
    }
  } else if (META) {
    const int64_t pr = (int64_t)(gw - token_items - pad_items) * kWave + lane;
    int slot;
    int64_t row;
    if constexpr (!FIXED) {
      if (pr >= a.sum_expanded) return;
      slot = a.row_slot[pr];
      row = packed_to_row(a, pr);
    } else {
      if (pr >= (int64_t)a.P * a.cap) return;
      slot = fixed_row_slot(a, pr);
      row = pr;
    }
    const int u = slot >= 0 ? slot / a.K : -1;
    a.recv_weights[row] = slot >= 0 ? a.w[slot] : 0.0f;
    ((int2*)a.recv_meta)[row] = make_int2(u, slot >= 0 ? slot - u * a.K : -1);
  }
}

// Column-major fp8 scales: recv_scales[b][row] = scale b of the row's source
// token (0 for padding rows with zero padding, otherwise untouched; 0 for the
// tail rows of fixed windows).  Row-major scales are written by the dispatch
// kernel's own waves; this runs after it for column-major scales only.
__device__ __forceinline__ void row_source(const DispatchArgs& a, int64_t pr, int& slot, int64_t& row,
                                           bool& tail) {
  tail = false;
  if (a.cap == 0) {
    slot = a.row_slot[pr];
    row = packed_to_row(a, pr);
  } else {
    row = pr;
    const int r = (int)(pr / a.cap);
    const int64_t l = pr - (int64_t)r * a.cap;
    tail = l >= a.num_expanded[r];
    slot = tail ? -1 : a.row_slot[a.packed_base[r] + l];
  }
}

// One workgroup per 64 consecutive rows, transposing through LDS 64 blocks at
// a time: the loads read each row's scales contiguously (a row's token scales
// are 4 * H/128 contiguous bytes), the stores write each block's 64 rows
// contiguously.
constexpr int kCmRows = 64;
__global__ __launch_bounds__(256) void dispatch_scales_cm_kernel(DispatchArgs a) {
  __shared__ float tile[kCmRows][kCmRows + 1];
  __shared__ int64_t src_tok[kCmRows];  // source token, -1: zero, -2: untouched
  __shared__ int64_t dst_row[kCmRows];
  const int nblk = a.H >> 7;
  const int tid = threadIdx.x;
  const int64_t rows = a.cap > 0 ? (int64_t)a.P * a.cap : (int64_t)a.sum_expanded;
  const int64_t pr0 = (int64_t)blockIdx.x * kCmRows;
  if (tid < kCmRows) {
    const int64_t pr = pr0 + tid;
    int64_t tok = -2, row = 0;
    if (pr < rows) {
      int slot;
      bool tail;
      row_source(a, pr, slot, row, tail);
      tok = slot >= 0 ? (int64_t)(slot / a.K) : (a.zero_pad || tail) ? -1 : -2;
    }
    src_tok[tid] = tok;
    dst_row[tid] = row;
  }
  __syncthreads();
  for (int b0 = 0; b0 < nblk; b0 += kCmRows) {
    // load: element (i, k) = scale b0 + k of row i; consecutive threads take consecutive k
    for (int e = tid; e < kCmRows * kCmRows; e += 256) {
      const int i = e / kCmRows, k = e - i * kCmRows;
      const int64_t tok = src_tok[i];
      float v = 0.0f;
      if (tok >= 0 && b0 + k < nblk) v = a.tok_scales[tok * nblk + b0 + k];
      tile[i][k] = v;
    }
    __syncthreads();
    // store: element (k, i); consecutive threads take consecutive rows i
    for (int e = tid; e < kCmRows * kCmRows; e += 256) {
      const int k = e / kCmRows, i = e - k * kCmRows;
      if (b0 + k < nblk && src_tok[i] != -2)
        a.recv_scales[(int64_t)(b0 + k) * a.scale_rows + dst_row[i]] = tile[i][k];
    }
    __syncthreads();
  }
}

// Test hook: the dispatch kernel's float -> E4M3 conversion applied to an
// array (four values per thread, the tail padded with zeros).
__global__ __launch_bounds__(256) void e4m3_encode_kernel(const float* __restrict__ in, uint8_t* __restrict__ out,
                                                          int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  float f[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) f[k] = i + k < n ? in[i + k] : 0.0f;
  const uint32_t w = e4m3x4_hw(f[0], f[1], f[2], f[3]);
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (i + k < n) out[i + k] = (uint8_t)(w >> (8 * k));
}

// --------------------------------------------------------------------------
// combine
// --------------------------------------------------------------------------
struct CombineArgs {
  const uint16_t* y;       // [rows][H] bf16
  const float* w;          // [T][K] or null (unit weights)
  const int32_t* dst_row;  // [T][K]
  const uint16_t* bias;    // [T][H] bf16 or null, added after the K slots
  uint16_t* out;           // [T][H] bf16
  int T, K, H;
  int split;               // parts per row = ceil((H / 8) / (64 * NCT))
};

// NCT: 16-byte chunks per lane (the wave's column part is 64 * NCT chunks);
// G: slots whose loads are in flight together.  Accumulation order is always
// j = 0..K-1.
template <int NCT, int G>
__global__ __launch_bounds__(1024) void combine_kernel(CombineArgs a) {
#pragma clang fp contract(off)
  const int gw = wave_index();
  EP_TIMING_MARK(EP_TK_COMBINE, 0);
  if (gw >= a.T * a.split) return;
  const int u = gw / a.split;  // ascending tokens: measured faster than descending
  const int part = gw % a.split;
  const int tile = part * NCT * kWave;
  const int lane = lane_id();
  const int nchunk = a.H >> 3;
  // the token's K rows and weights, one vector load each (lane j holds slot j)
  const int my_row = lane < a.K ? a.dst_row[(int64_t)u * a.K + lane] : -1;
  const float my_w = (lane < a.K && a.w) ? a.w[(int64_t)u * a.K + lane] : 1.0f;
  u32x4* dst = (u32x4*)(a.out + (int64_t)u * a.H);
  u32x4 bv[NCT];
  if (a.bias) {
    const u32x4* bsrc = (const u32x4*)(a.bias + (int64_t)u * a.H);
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      const int q = tile + c * kWave + lane;
      bv[c] = q < nchunk ? __builtin_nontemporal_load(bsrc + q) : u32x4{0, 0, 0, 0};
    }
  }

  float acc[NCT][8];
#pragma unroll
  for (int c = 0; c < NCT; ++c)
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[c][k] = 0.0f;

  for (int j0 = 0; j0 < a.K; j0 += G) {
    u32x4 v[G][NCT];
    int row[G];
    float wj[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int j = j0 + g;
      row[g] = j < a.K ? __builtin_amdgcn_readlane(my_row, j) : -1;
      wj[g] = j < a.K ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j)) : 1.0f;
      if (row[g] >= 0) {
        const u32x4* src = (const u32x4*)(a.y + (int64_t)row[g] * a.H);
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
          const int q = tile + c * kWave + lane;
          v[g][c] = q < nchunk ? __builtin_nontemporal_load(src + q) : u32x4{0, 0, 0, 0};
        }
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (row[g] < 0) continue;
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float p0 = wj[g] * bf16_lo(v[g][c][k]);
          const float p1 = wj[g] * bf16_hi(v[g][c][k]);
          acc[c][2 * k] = acc[c][2 * k] + p0;
          acc[c][2 * k + 1] = acc[c][2 * k + 1] + p1;
        }
    }
  }
  if (a.bias) {
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[c][2 * k] = acc[c][2 * k] + bf16_lo(bv[c][k]);
        acc[c][2 * k + 1] = acc[c][2 * k + 1] + bf16_hi(bv[c][k]);
      }
  }
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    const int q = tile + c * kWave + lane;
    if (q < nchunk) {
      u32x4 o;
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = pack_bf16x2(acc[c][2 * k], acc[c][2 * k + 1]);
      stream_store(dst + q, o);  // nontemporal: measured 3-4% faster
    }
  }
}

// Combine through LDS: one workgroup of 8 waves per (token, column part of
// 64 * NCF chunks); wave j loads slot j's part of the row (all NCF chunks per
// lane in flight) into LDS, then the workgroup reduces each chunk over the
// slots in order.  K <= 8.
template <int NCF>
__global__ __launch_bounds__(512) void combine_lds_kernel(CombineArgs a) {
#pragma clang fp contract(off)
  extern __shared__ u32x4 stage[];  // [K][64 * NCF]
  constexpr int W = NCF * kWave;
  const int u = blockIdx.x / a.split;
  const int tile = (blockIdx.x - u * a.split) * W;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int nchunk = a.H >> 3;
  const int my_row = lane < a.K ? a.dst_row[(int64_t)u * a.K + lane] : -1;
  const float my_w = (lane < a.K && a.w) ? a.w[(int64_t)u * a.K + lane] : 1.0f;
  if (wv < a.K) {
    const int row = __builtin_amdgcn_readlane(my_row, wv);
    if (row >= 0) {
      const u32x4* src = (const u32x4*)(a.y + (int64_t)row * a.H);
      u32x4 v[NCF];
#pragma unroll
      for (int c = 0; c < NCF; ++c) {
        const int q = tile + c * kWave + lane;
        v[c] = q < nchunk ? __builtin_nontemporal_load(src + q) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int c = 0; c < NCF; ++c) stage[wv * W + c * kWave + lane] = v[c];
    }
  }
  __syncthreads();
  u32x4* dst = (u32x4*)(a.out + (int64_t)u * a.H);
  for (int i = threadIdx.x; i < W; i += 512) {
    const int q = tile + i;
    if (q >= nchunk) break;
    float acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = 0.0f;
    for (int j = 0; j < a.K; ++j) {
      const int row = __builtin_amdgcn_readlane(my_row, j);
      if (row < 0) continue;
      const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j));
      const u32x4 v = stage[j * W + i];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float p0 = wj * bf16_lo(v[k]);
        const float p1 = wj * bf16_hi(v[k]);
        acc[2 * k] = acc[2 * k] + p0;
        acc[2 * k + 1] = acc[2 * k + 1] + p1;
      }
    }
    if (a.bias) {
      const u32x4 bv = __builtin_nontemporal_load((const u32x4*)(a.bias + (int64_t)u * a.H) + q);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[2 * k] = acc[2 * k] + bf16_lo(bv[k]);
        acc[2 * k + 1] = acc[2 * k + 1] + bf16_hi(bv[k]);
      }
    }
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = pack_bf16x2(acc[2 * k], acc[2 * k + 1]);
    stream_store(dst + q, o);  // nontemporal: measured 3-4% faster
  }
}

}  // namespace ep
