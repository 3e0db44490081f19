/*
 * oracle.c -- plain, slow, single-threaded CPU oracle of the MoE dispatch /
 * combine path (layout, dispatch in bf16 or fp8, combine).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may call this; the product path never does.
 * It shares no code, header, table or helper with the HIP library.
 *
 * Sources (the two pages this method is described on):
 *   [BLOG]  "Ascend DeepEP MoE Dispatch Optimization"
 *   [TUT]   TileLang tutorial, chapter 38 "DeepEP-Ascend"
 *
 * Every step below is the plain definition, in plain loops.  "#{u' < u : ...}"
 * style counts are kept as running counters scanned in index order, which is
 * the same count written the obvious way.
 *
 * Readings where the pages are silent (all listed in the design notes):
 *  - expert e lives on rank e / E_l (contiguous blocks); E_l = E / P
 *  - topk_idx == -1 marks an unused slot; any other value outside [0, E) is a
 *    routing error
 *  - global token index u = s * S + t (source rank s, local token t)
 *  - the receive list of a destination rank is ordered by source rank, then
 *    by token; expanded rows of one expert are ordered by (u, j)
 *  - fp8 scale = amax / 448 in fp32; a block with amax == 0 has scale +0 and
 *    signed-zero codes
 *  - combine: acc = +0; for j = 0..K-1: acc = fl(acc + fl(w_j * y_j)) in fp32;
 *    out = bf16 round-to-nearest-even(acc)
 *  - fixed output length: the fixed row count applies to each rank's window of
 *    expanded rows; the tail is zeroed whatever the zero-padding flag says;
 *    rows past the fixed length are dropped and counted, and combine skips the
 *    slots whose rows were dropped
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off -fno-fast-math
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

/* ------------------------------------------------------------------------ */
/* Scalar encodings                                                          */
/* ------------------------------------------------------------------------ */

static float f32_from_bits(uint32_t b) {
  float f;
  memcpy(&f, &b, 4);
  return f;
}
static uint32_t bits_from_f32(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  return b;
}

/* bfloat16 -> float: the bf16 pattern is the upper half of an fp32 pattern. */
float oracle_bf16_to_float(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* float -> bfloat16, round to nearest, ties to even (the conversion the tutorial's
 * combine ends with, [TUT] section 4.5).  Keep the upper 16 bits of the fp32
 * pattern, rounding on the lower 16: add 0x7FFF plus the kept LSB, so an exact
 * half rounds up only when that LSB is odd.  NaN maps to a quiet NaN. */
uint16_t oracle_bf16_round(float f) {
  uint32_t b = bits_from_f32(f);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((b >> 16) | 0x0040u);
  uint32_t lsb = (b >> 16) & 1u;
  return (uint16_t)((b + 0x7FFFu + lsb) >> 16);
}

/* OCP FP8 E4M3FN ("float8_e4m3fn"): 1 sign, 4 exponent (bias 7), 3 mantissa
 * bits; no infinities; 0x7F / 0xFF are NaN; largest finite 448 (0x7E);
 * subnormals m * 2^-9.  [TUT] section 3.6 names torch.float8_e4m3fn. */
float oracle_e4m3_decode(uint8_t c) {
  int sign = (c >> 7) & 1;
  int e = (c >> 3) & 15;
  int m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return (float)(sign ? -v : v);
}

/* float -> E4M3FN, round to nearest, ties to even mantissa.
 * |q| beyond the rounding range of 448 (> 464), infinities and NaN give NaN
 * (the format has no infinity). */
uint8_t oracle_e4m3_encode(float q) {
  uint8_t sign = signbit(q) ? 0x80 : 0x00;
  double a = fabs((double)q);
  if (isnan(q) || isinf(q)) return (uint8_t)(sign | 0x7F);
  if (a < ldexp(1.0, -6)) {
    /* subnormal range: value = r * 2^-9, r in 0..8 (8 is the smallest normal,
     * whose code is also 8) */
    double r = nearbyint(a * 512.0); /* default rounding mode: ties to even */
    return (uint8_t)(sign | (uint8_t)r);
  }
  int ex;
  double f = frexp(a, &ex); /* a = f * 2^ex, f in [0.5, 1) */
  int e = ex - 1;            /* a = (1 + m) * 2^e, m in [0, 1) */
  double m = 2.0 * f - 1.0;
  double r = nearbyint(m * 8.0); /* 3 mantissa bits, ties to even */
  if (r == 8.0) {
    r = 0.0;
    e += 1;
  }
  if (e > 8 || (e == 8 && r == 7.0)) return (uint8_t)(sign | 0x7F);
  return (uint8_t)(sign | (uint8_t)(((e + 7) << 3) | (int)r));
}

/* ------------------------------------------------------------------------ */
/* Layout                                                                    */
/* ------------------------------------------------------------------------ */

/* Size of the packed recv_src_idx output is sum_d num_recv_tokens[d], at most
 * T * min(K, P).
 *
 * Outputs (all caller-allocated, row-major):
 *  is_token_in_rank     [T*P]  u8   1 iff some valid slot of token u has rank(e) == d
 *                                    ([BLOG] "what the six handle entries store")
 *  num_tokens_per_rank  [P*P]  i32  [s][d] = sum over tokens t of rank s of itr
 *  num_tokens_per_expert[P*E]  i32  [s][e] = number of slots of rank s's tokens routed to e
 *  rank_prefix_matrix   [P*P]  i32  [s][d] = sum_{s' <= s} num_tokens_per_rank[s'][d]
 *                                    (segment of s in d's receive list starts at [s-1][d];
 *                                    [BLOG] "how the device side turns a channel into a remote Put")
 *  num_recv_tokens      [P]    i32  rank-deduplicated tokens received by d
 *  num_tokens_per_expert_total [E] i32  n_e over all source ranks
 *  expert_offset        [P*(E_l+1)] i64  window-local start of each local expert's rows:
 *                                    sum of ceil(n/A)*A over earlier local experts ([TUT] 2.2)
 *  num_expanded         [P]    i64  rows of window d = sum_e ceil(n_e/A)*A ([TUT] 2.2)
 *  window_row_base      [P+1]  i64  first global row of each window (packed: prefix sum of
 *                                    num_expanded; symmetric: d * max_d num_expanded)
 *  dst_slot             [T*K]  i32  window-local row of slot (u, j), -1 if unused
 *  send_head            [T*P]  i32  position of u in d's receive list, -1 if not sent
 *                                    ([BLOG] handle entries: "-1 = not sent to that rank")
 *  recv_src_idx         [sum]  i32  for each destination d (packed, d-major), for each
 *                                    receive-list position i: the local token index t of the
 *                                    i-th token received ([BLOG] handle entries)
 *  recv_src_base        [P+1]  i64  start of d's list inside recv_src_idx
 */
int oracle_layout(int P, int S, int E, int K, int A, int symmetric, const int64_t *topk_idx,
                  uint8_t *is_token_in_rank, int32_t *num_tokens_per_rank,
                  int32_t *num_tokens_per_expert, int32_t *rank_prefix_matrix,
                  int32_t *num_recv_tokens, int32_t *num_tokens_per_expert_total,
                  int64_t *expert_offset, int64_t *num_expanded, int64_t *window_row_base,
                  int32_t *dst_slot, int32_t *send_head, int32_t *recv_src_idx,
                  int64_t *recv_src_base) {
  if (P < 1 || S < 0 || E < 1 || K < 1 || A < 1 || E % P != 0) return ORACLE_ERR_SHAPE;
  const int64_t T = (int64_t)P * S;
  const int El = E / P;

  /* Unused slots are -1; anything else outside [0, E) is an error. */
  for (int64_t i = 0; i < T * K; i++) {
    int64_t e = topk_idx[i];
    if (e != -1 && (e < 0 || e >= E)) return ORACLE_ERR_ROUTING;
  }

  /* is_token_in_rank: rank(e) = e / E_l ([BLOG] "a token's journey"; [TUT] 7.2:
   * 256 experts over 8 ranks leaves 32 local experts per rank). */
  memset(is_token_in_rank, 0, (size_t)(T * P));
  for (int64_t u = 0; u < T; u++)
    for (int j = 0; j < K; j++) {
      int64_t e = topk_idx[u * K + j];
      if (e >= 0) is_token_in_rank[u * P + e / El] = 1;
    }

  /* Per-source-rank histograms. */
  memset(num_tokens_per_rank, 0, sizeof(int32_t) * (size_t)P * P);
  memset(num_tokens_per_expert, 0, sizeof(int32_t) * (size_t)P * E);
  for (int s = 0; s < P; s++)
    for (int t = 0; t < S; t++) {
      int64_t u = (int64_t)s * S + t;
      for (int d = 0; d < P; d++) num_tokens_per_rank[s * P + d] += is_token_in_rank[u * P + d];
      for (int j = 0; j < K; j++) {
        int64_t e = topk_idx[u * K + j];
        if (e >= 0) num_tokens_per_expert[(int64_t)s * E + e] += 1;
      }
    }

  /* rank_prefix_matrix: cumulative over source ranks, per destination. */
  for (int d = 0; d < P; d++) {
    int32_t acc = 0;
    for (int s = 0; s < P; s++) {
      acc += num_tokens_per_rank[s * P + d];
      rank_prefix_matrix[s * P + d] = acc;
    }
    num_recv_tokens[d] = acc;
  }

  /* Expert totals, aligned sizes and window-local offsets ([TUT] 2.2). */
  for (int e = 0; e < E; e++) {
    int32_t n = 0;
    for (int s = 0; s < P; s++) n += num_tokens_per_expert[(int64_t)s * E + e];
    num_tokens_per_expert_total[e] = n;
  }
  int64_t max_expanded = 0;
  for (int d = 0; d < P; d++) {
    int64_t off = 0;
    for (int l = 0; l < El; l++) {
      expert_offset[(int64_t)d * (El + 1) + l] = off;
      int64_t n = num_tokens_per_expert_total[d * El + l];
      int64_t padded = ((n + A - 1) / A) * A;
      off += padded;
    }
    expert_offset[(int64_t)d * (El + 1) + El] = off;
    num_expanded[d] = off;
    if (off > max_expanded) max_expanded = off;
  }
  window_row_base[0] = 0;
  for (int d = 0; d < P; d++)
    window_row_base[d + 1] = symmetric ? (int64_t)(d + 1) * max_expanded
                                       : window_row_base[d] + num_expanded[d];

  /* dst_slot: the rows of expert e are the slots (u, j) routed to e in
   * increasing (u, j) order -- the order the tutorial's deterministic mode
   * sorts by (key expert * 1e10 + source token global index, [TUT] 3.5). */
  int32_t *seen_e = (int32_t *)calloc((size_t)E, sizeof(int32_t));
  if (!seen_e) return ORACLE_ERR_SHAPE;
  for (int64_t u = 0; u < T; u++)
    for (int j = 0; j < K; j++) {
      int64_t e = topk_idx[u * K + j];
      if (e < 0) {
        dst_slot[u * K + j] = -1;
        continue;
      }
      int d = (int)(e / El), l = (int)(e % El);
      dst_slot[u * K + j] = (int32_t)(expert_offset[(int64_t)d * (El + 1) + l] + seen_e[e]);
      seen_e[e] += 1;
    }
  free(seen_e);

  /* send_head / recv_src_idx: d's receive list holds the tokens u with
   * is_token_in_rank[u][d] in increasing u (source rank, then token). */
  recv_src_base[0] = 0;
  for (int d = 0; d < P; d++) recv_src_base[d + 1] = recv_src_base[d] + num_recv_tokens[d];
  int32_t *seen_d = (int32_t *)calloc((size_t)P, sizeof(int32_t));
  if (!seen_d) return ORACLE_ERR_SHAPE;
  for (int64_t u = 0; u < T; u++)
    for (int d = 0; d < P; d++) {
      if (!is_token_in_rank[u * P + d]) {
        send_head[u * P + d] = -1;
        continue;
      }
      send_head[u * P + d] = seen_d[d];
      recv_src_idx[recv_src_base[d] + seen_d[d]] = (int32_t)(u % S);
      seen_d[d] += 1;
    }
  free(seen_d);
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Dispatch                                                                  */
/* ------------------------------------------------------------------------ */

/* Per-token FP8 quantisation ([TUT] 3.6): one fp32 scale per 128 channels,
 * scale = amax / 448, code = E4M3(x / scale), both divisions IEEE fp32.
 * codes [H] u8, scales [H/128] f32.
 *
 * Non-finite inputs (the pages say nothing; this is the stated reading): the
 * block maximum is NaN as soon as one |x| is NaN, else the largest |x|, +Inf
 * included.  A NaN maximum gives the scale 0x7FC00000 (the quiet NaN with a
 * clear sign and payload), an infinite one the scale +Inf.  Codes are still
 * E4M3(x / scale), except that a NaN quotient (x / NaN, or +-Inf / +Inf) is
 * written as 0x7F, the E4M3FN NaN with a clear sign bit.  A finite x over an
 * infinite scale is the signed zero of the quotient. */
void oracle_quantize_row(const uint16_t *x, int H, uint8_t *codes, float *scales) {
  for (int b = 0; b < H / 128; b++) {
    float amax = 0.0f;
    int has_nan = 0;
    for (int h = 128 * b; h < 128 * b + 128; h++) {
      float v = fabsf(oracle_bf16_to_float(x[h]));
      if (isnan(v))
        has_nan = 1;
      else if (v > amax)
        amax = v;
    }
    float scale = has_nan ? f32_from_bits(0x7FC00000u) : amax / 448.0f;
    scales[b] = scale;
    for (int h = 128 * b; h < 128 * b + 128; h++) {
      float xf = oracle_bf16_to_float(x[h]);
      if (amax == 0.0f && !has_nan) {
        codes[h] = signbit(xf) ? 0x80 : 0x00;
      } else {
        float q = xf / scale;
        codes[h] = isnan(q) ? 0x7F : oracle_e4m3_encode(q);
      }
    }
  }
}

/* FP8 quantisation with UE8M0 scales.  The tutorial's size-hint passage
 * ([TUT] 3.2) counts ceil(H/64) int16 scale packs per token, each holding two
 * UE8M0 values: one unsigned 8-bit exponent per 32 channels.  (Its FP8 section,
 * [TUT] 3.6, describes the same byte count as fp32 scales per 128 channels;
 * that is the default format, this is the alternative.)  Reading, per block of
 * 32 channels:
 *   amax as in oracle_quantize_row;
 *   k = the smallest integer in [-127, 127] with 448 * 2^k >= amax (a power of
 *       two at or above amax / 448, so no |x| / 2^k exceeds 448 and no code
 *       saturates), found by counting up from -127; amax = 0 gives -127;
 *   exps[b] = k + 127 (the biased exponent byte), codes = E4M3(x / 2^k) with
 *       the IEEE fp32 division;
 *   a non-finite maximum (NaN or Inf in the block) gives exps[b] = 0xFF, the
 *       UE8M0 NaN, and the codes of oracle_quantize_row's non-finite rule.
 * codes [H] u8, exps [H/32] u8 (byte b of the row is block b; as int16 packs,
 * pack i holds block 2i in its low byte and block 2i + 1 in its high byte). */
void oracle_quantize_row_ue8m0(const uint16_t *x, int H, uint8_t *codes, uint8_t *exps) {
  for (int b = 0; b < H / 32; b++) {
    float amax = 0.0f;
    int has_nan = 0;
    for (int h = 32 * b; h < 32 * b + 32; h++) {
      float v = fabsf(oracle_bf16_to_float(x[h]));
      if (isnan(v))
        has_nan = 1;
      else if (v > amax)
        amax = v;
    }
    if (has_nan || isinf(amax)) {
      exps[b] = 0xFF;
      for (int h = 32 * b; h < 32 * b + 32; h++) {
        float xf = oracle_bf16_to_float(x[h]);
        codes[h] = (has_nan || isinf(xf)) ? 0x7F : (signbit(xf) ? 0x80 : 0x00);
      }
      continue;
    }
    int k = -127;
    while (k < 127 && ldexp(448.0, k) < (double)amax) k++;
    exps[b] = (uint8_t)(k + 127);
    float scale = ldexpf(1.0f, k);
    for (int h = 32 * b; h < 32 * b + 32; h++)
      codes[h] = oracle_e4m3_encode(oracle_bf16_to_float(x[h]) / scale);
  }
}

/* oracle_quantize_row_ue8m0 applied to rows [row_begin, row_end) of x [T][H];
 * the outputs hold only those rows. */
void oracle_quantize_rows_ue8m0(const uint16_t *x, int H, int64_t row_begin, int64_t row_end,
                                uint8_t *codes, uint8_t *exps) {
  for (int64_t u = row_begin; u < row_end; u++)
    oracle_quantize_row_ue8m0(x + u * H, H, codes + (u - row_begin) * H,
                              exps + (u - row_begin) * (H / 32));
}

/* oracle_quantize_row applied to rows [row_begin, row_end) of x [T][H]; the
 * outputs hold only those rows. */
void oracle_quantize_rows(const uint16_t *x, int H, int64_t row_begin, int64_t row_end,
                          uint8_t *codes, float *scales) {
  for (int64_t u = row_begin; u < row_end; u++)
    oracle_quantize_row(x + u * H, H, codes + (u - row_begin) * H,
                        scales + (u - row_begin) * (H / 128));
}

/* Dispatch rows [row_begin, row_end) of the expanded output ([TUT] 2.2).
 *
 * Row r = window_row_base[rank(e)] + dst_slot[u][j] of slot (u, j) gets
 *   recv_x[r]        = x[u]                (bf16 bit copy), or
 *   recv_x[r]        = E4M3 codes of x[u], recv_scales[r] = its H/128 scales (fp8)
 *   recv_weights[r]  = topk_weights[u][j]
 *   recv_src_meta[r] = (u, j)
 * Alignment padding rows of expert e ([off + n_e, off + ceil(n_e/A)*A) in its
 * window) get recv_src_meta = (-1, -1), recv_weights = 0 and, with
 * zero_padding, an all-zero payload and zero scales ([BLOG] "output length":
 * padding carries x / scales / weights 0 and index -1; [TUT] 2.2:
 * do_zero_padding).  Without zero_padding their payload is left untouched.
 * Rows not covered (symmetric-window tails) are left untouched.
 *
 * Options (oracle_dispatch_general):
 *  capacity > 0      the fixed output length of every window (see
 *                    oracle_dispatch_fixed): window d starts at d * capacity,
 *                    window-local rows >= capacity are not written, and the rows
 *                    [num_expanded[d], capacity) of a window are its tail.
 *  scales_col_major  1: recv_scales is laid out [H/128][n] (n = row_end - row_begin:
 *                    one scale position contiguous across rows) instead of
 *                    [n][H/128] ([TUT] 3.6 (3): the column-major scale layout is
 *                    the transpose of the row-major one, with no padding of the
 *                    row dimension).
 *                    2: UE8M0 scales (oracle_quantize_row_ue8m0): recv_scales
 *                    holds bytes [n][H/32] (cast to uint8_t *), zero bytes
 *                    where fp32 scales would be zero.  Not with x_codes.
 *  x_codes, x_scales pre-quantised input ([TUT] 3.6 (2): x may be the pair of
 *                    E4M3 data [T][H] and one fp32 scale per 128 channels
 *                    [T][H/128]); rows then carry these bytes and scales as
 *                    they are, and x is not read.  fp8 only.
 *
 * Output arrays hold only rows [row_begin, row_end): element (r, h) is at
 * (r - row_begin) * H + h.  recv_weights / recv_src_meta may be NULL (cached
 * dispatch moves payload only); recv_x may be NULL (metadata only).
 * recv_scales is used only when fp8. */
static void put_scales(float *recv_scales, int col_major, int64_t n, int64_t rr, int nb,
                       const float *src) {
  for (int b = 0; b < nb; b++) {
    float v = src ? src[b] : 0.0f;
    if (col_major)
      recv_scales[(int64_t)b * n + rr] = v;
    else
      recv_scales[rr * nb + b] = v;
  }
}

static int dispatch_rows(int P, int S, int E, int K, int H, int A, int fp8, int zero_padding,
                         int scales_col_major, const int64_t *topk_idx, const int32_t *dst_slot,
                         const int32_t *num_tokens_per_expert_total, const int64_t *expert_offset,
                         const int64_t *window_row_base, int64_t capacity, const uint16_t *x,
                         const uint8_t *x_codes, const float *x_scales,
                         const float *topk_weights, int64_t row_begin, int64_t row_end,
                         void *recv_x, float *recv_scales, float *recv_weights,
                         int32_t *recv_src_meta) {
  if (P < 1 || E % P != 0 || H < 1 || (fp8 && H % 128 != 0)) return ORACLE_ERR_SHAPE;
  if (x_codes && !fp8) return ORACLE_ERR_SHAPE;
  const int ue8m0 = scales_col_major == 2;
  if (ue8m0 && (x_codes || !fp8)) return ORACLE_ERR_SHAPE;
  const int64_t T = (int64_t)P * S;
  const int El = E / P;
  const int nb = H / 128;
  const int nb32 = H / 32;
  const int64_t n_out = row_end - row_begin;
  uint8_t *codes = NULL;
  float *scales = NULL;
  uint8_t *exps = NULL;
  if (fp8) {
    codes = (uint8_t *)malloc((size_t)H);
    scales = (float *)malloc(sizeof(float) * (size_t)(nb > 0 ? nb : 1));
    exps = (uint8_t *)malloc((size_t)(nb32 > 0 ? nb32 : 1));
    if (!codes || !scales || !exps) {
      free(codes);
      free(scales);
      free(exps);
      return ORACLE_ERR_SHAPE;
    }
  }
  for (int64_t u = 0; u < T; u++) {
    for (int j = 0; j < K; j++) {
      int64_t e = topk_idx[u * K + j];
      if (e < 0) continue;
      int64_t local = dst_slot[u * K + j];
      if (capacity > 0 && local >= capacity) continue; /* truncated */
      int64_t r = (capacity > 0 ? (e / El) * capacity : window_row_base[e / El]) + local;
      if (r < row_begin || r >= row_end) continue;
      int64_t rr = r - row_begin;
      if (!recv_x) {
        /* metadata only */
      } else if (fp8 && ue8m0) {
        oracle_quantize_row_ue8m0(x + u * H, H, codes, exps);
        memcpy((uint8_t *)recv_x + rr * H, codes, (size_t)H);
        memcpy((uint8_t *)recv_scales + rr * nb32, exps, (size_t)nb32);
      } else if (fp8) {
        if (x_codes) {
          memcpy(codes, x_codes + u * H, (size_t)H);
          memcpy(scales, x_scales + u * nb, sizeof(float) * (size_t)nb);
        } else {
          oracle_quantize_row(x + u * H, H, codes, scales);
        }
        memcpy((uint8_t *)recv_x + rr * H, codes, (size_t)H);
        put_scales(recv_scales, scales_col_major, n_out, rr, nb, scales);
      } else {
        memcpy((uint16_t *)recv_x + rr * H, x + u * H, sizeof(uint16_t) * (size_t)H);
      }
      if (recv_weights) recv_weights[rr] = topk_weights[u * K + j];
      if (recv_src_meta) {
        recv_src_meta[2 * rr] = (int32_t)u;
        recv_src_meta[2 * rr + 1] = j;
      }
    }
  }
  /* Alignment padding rows. */
  for (int e = 0; e < E; e++) {
    int d = e / El, l = e % El;
    int64_t n = num_tokens_per_expert_total[e];
    int64_t padded = ((n + A - 1) / A) * A;
    int64_t local0 = expert_offset[(int64_t)d * (El + 1) + l];
    for (int64_t local = local0 + n; local < local0 + padded; local++) {
      if (capacity > 0 && local >= capacity) break; /* truncated */
      int64_t r = (capacity > 0 ? d * capacity : window_row_base[d]) + local;
      if (r < row_begin || r >= row_end) continue;
      int64_t rr = r - row_begin;
      if (recv_weights) recv_weights[rr] = 0.0f;
      if (recv_src_meta) {
        recv_src_meta[2 * rr] = -1;
        recv_src_meta[2 * rr + 1] = -1;
      }
      if (zero_padding && recv_x) {
        if (fp8) {
          memset((uint8_t *)recv_x + rr * H, 0, (size_t)H);
          if (ue8m0)
            memset((uint8_t *)recv_scales + rr * nb32, 0, (size_t)nb32);
          else
            put_scales(recv_scales, scales_col_major, n_out, rr, nb, NULL);
        } else {
          for (int h = 0; h < H; h++) ((uint16_t *)recv_x)[rr * H + h] = 0;
        }
      }
    }
  }
  /* Tail rows of a fixed-length window: always x / scales / weights 0 and
   * index -1 ([BLOG] "output length"). */
  if (capacity > 0) {
    for (int d = 0; d < P; d++) {
      int64_t used = expert_offset[(int64_t)d * (El + 1) + El]; /* num_expanded[d] */
      for (int64_t local = used; local < capacity; local++) {
        int64_t r = d * capacity + local;
        if (r < row_begin || r >= row_end) continue;
        int64_t rr = r - row_begin;
        if (recv_weights) recv_weights[rr] = 0.0f;
        if (recv_src_meta) {
          recv_src_meta[2 * rr] = -1;
          recv_src_meta[2 * rr + 1] = -1;
        }
        if (recv_x) {
          if (fp8) {
            memset((uint8_t *)recv_x + rr * H, 0, (size_t)H);
            if (ue8m0)
              memset((uint8_t *)recv_scales + rr * nb32, 0, (size_t)nb32);
            else
              put_scales(recv_scales, scales_col_major, n_out, rr, nb, NULL);
          } else {
            for (int h = 0; h < H; h++) ((uint16_t *)recv_x)[rr * H + h] = 0;
          }
        }
      }
    }
  }
  free(codes);
  free(scales);
  free(exps);
  return ORACLE_OK;
}

int oracle_dispatch(int P, int S, int E, int K, int H, int A, int fp8, int zero_padding,
                    const int64_t *topk_idx, const int32_t *dst_slot,
                    const int32_t *num_tokens_per_expert_total, const int64_t *expert_offset,
                    const int64_t *window_row_base, const uint16_t *x, const float *topk_weights,
                    int64_t row_begin, int64_t row_end, void *recv_x, float *recv_scales,
                    float *recv_weights, int32_t *recv_src_meta) {
  return dispatch_rows(P, S, E, K, H, A, fp8, zero_padding, 0, topk_idx, dst_slot,
                       num_tokens_per_expert_total, expert_offset, window_row_base, 0, x, NULL,
                       NULL, topk_weights, row_begin, row_end, recv_x, recv_scales, recv_weights,
                       recv_src_meta);
}

/* Rows past the fixed length of each window, sum_d max(0, num_expanded[d] - capacity). */
static int64_t dropped_rows(int P, int El, const int64_t *expert_offset, int64_t capacity) {
  int64_t drop = 0;
  for (int d = 0; d < P; d++) {
    int64_t used = expert_offset[(int64_t)d * (El + 1) + El];
    if (used > capacity) drop += used - capacity;
  }
  return drop;
}

/* Fixed output length ([BLOG] "the output length has a dynamic and a fixed
 * mode"): the caller fixes in advance how many rows every rank's output holds
 * (num_worst_tokens there; here `capacity` expanded rows per window), so no
 * count has to be read back before the output is sized.  Window d is rows
 * [d * capacity, (d + 1) * capacity) and holds the first min(num_expanded[d],
 * capacity) rows of the exact window, at the same window-local index.
 *  - num_expanded[d] < capacity: the rest is the tail, with payload, scales
 *    and weights 0 and index (-1, -1), whatever zero_padding says.
 *  - num_expanded[d] > capacity: the rows from capacity on are not published.
 *    The page's implementation drops them silently; here *dropped receives
 *    sum_d max(0, num_expanded[d] - capacity), the rows left out.
 * Rows [row_begin, row_end) of the P * capacity output, as oracle_dispatch. */
int oracle_dispatch_fixed(int P, int S, int E, int K, int H, int A, int fp8, int zero_padding,
                          const int64_t *topk_idx, const int32_t *dst_slot,
                          const int32_t *num_tokens_per_expert_total,
                          const int64_t *expert_offset, int64_t capacity, const uint16_t *x,
                          const float *topk_weights, int64_t row_begin, int64_t row_end,
                          void *recv_x, float *recv_scales, float *recv_weights,
                          int32_t *recv_src_meta, int64_t *dropped) {
  if (capacity < 1 || P < 1 || E % P != 0) return ORACLE_ERR_SHAPE;
  if (dropped) *dropped = dropped_rows(P, E / P, expert_offset, capacity);
  return dispatch_rows(P, S, E, K, H, A, fp8, zero_padding, 0, topk_idx, dst_slot,
                       num_tokens_per_expert_total, expert_offset, NULL, capacity, x, NULL, NULL,
                       topk_weights, row_begin, row_end, recv_x, recv_scales, recv_weights,
                       recv_src_meta);
}

/* Every option at once (see dispatch_rows): exact (capacity 0) or fixed
 * windows, row- or column-major scales, quantised here or pre-quantised
 * input.  *dropped (may be NULL) as in oracle_dispatch_fixed. */
int oracle_dispatch_general(int P, int S, int E, int K, int H, int A, int fp8, int zero_padding,
                            int scales_col_major, int64_t capacity, const int64_t *topk_idx,
                            const int32_t *dst_slot, const int32_t *num_tokens_per_expert_total,
                            const int64_t *expert_offset, const int64_t *window_row_base,
                            const uint16_t *x, const uint8_t *x_codes, const float *x_scales,
                            const float *topk_weights, int64_t row_begin, int64_t row_end,
                            void *recv_x, float *recv_scales, float *recv_weights,
                            int32_t *recv_src_meta, int64_t *dropped) {
  if (capacity < 0 || P < 1 || E % P != 0) return ORACLE_ERR_SHAPE;
  if (dropped) *dropped = capacity > 0 ? dropped_rows(P, E / P, expert_offset, capacity) : 0;
  return dispatch_rows(P, S, E, K, H, A, fp8, zero_padding, scales_col_major, topk_idx,
                       dst_slot, num_tokens_per_expert_total, expert_offset, window_row_base,
                       capacity, x, x_codes, x_scales, topk_weights, row_begin, row_end, recv_x,
                       recv_scales, recv_weights, recv_src_meta);
}

/* ------------------------------------------------------------------------ */
/* Combine                                                                   */
/* ------------------------------------------------------------------------ */

/* Combine tokens [tok_begin, tok_end) ([BLOG] "a token's journey": the K
 * results are sent back and reduced with the top-k weights; [TUT] 4.5: bf16
 * inputs, fp32 accumulation, round-to-nearest-even back to bf16):
 *   acc = +0
 *   for j = 0..K-1 with a valid slot:
 *     acc = fl(acc + fl(w[u][j] * float(y[window_row_base[rank(e)] + dst_slot[u][j]][h])))
 *   with a bias ([TUT] 3.3: combine's optional bias, the fused residual or
 *   shared-expert output, bf16 [T][H]):  acc = fl(acc + float(bias[u][h]))
 *   out[u][h] = bf16(acc)
 * topk_weights == NULL means every weight is 1; bias == NULL means none.
 * capacity > 0: fixed-length windows (oracle_dispatch_fixed): row
 * rank(e) * capacity + dst_slot, and a slot whose row was not published
 * (dst_slot >= capacity) is skipped like an unused one.
 * out holds only tokens [tok_begin, tok_end). */
static int combine_rows(int P, int E, int K, int H, const int64_t *topk_idx,
                        const int32_t *dst_slot, const int64_t *window_row_base,
                        int64_t capacity, const uint16_t *y, const float *topk_weights,
                        const uint16_t *bias, int64_t tok_begin, int64_t tok_end, uint16_t *out) {
  if (P < 1 || E % P != 0) return ORACLE_ERR_SHAPE;
  const int El = E / P;
  for (int64_t u = tok_begin; u < tok_end; u++) {
    for (int h = 0; h < H; h++) {
      float acc = 0.0f;
      for (int j = 0; j < K; j++) {
        int64_t e = topk_idx[u * K + j];
        if (e < 0) continue;
        int64_t local = dst_slot[u * K + j];
        if (capacity > 0 && local >= capacity) continue;
        int64_t r = (capacity > 0 ? (e / El) * capacity : window_row_base[e / El]) + local;
        float w = topk_weights ? topk_weights[u * K + j] : 1.0f;
        float prod = w * oracle_bf16_to_float(y[r * H + h]);
        acc = acc + prod;
      }
      if (bias) acc = acc + oracle_bf16_to_float(bias[u * H + h]);
      out[(u - tok_begin) * H + h] = oracle_bf16_round(acc);
    }
  }
  return ORACLE_OK;
}

int oracle_combine(int P, int S, int E, int K, int H, const int64_t *topk_idx,
                   const int32_t *dst_slot, const int64_t *window_row_base, const uint16_t *y,
                   const float *topk_weights, int64_t tok_begin, int64_t tok_end,
                   uint16_t *out) {
  (void)S;
  return combine_rows(P, E, K, H, topk_idx, dst_slot, window_row_base, 0, y, topk_weights, NULL,
                      tok_begin, tok_end, out);
}

int oracle_combine_fixed(int P, int S, int E, int K, int H, const int64_t *topk_idx,
                         const int32_t *dst_slot, int64_t capacity, const uint16_t *y,
                         const float *topk_weights, int64_t tok_begin, int64_t tok_end,
                         uint16_t *out) {
  (void)S;
  if (capacity < 1) return ORACLE_ERR_SHAPE;
  return combine_rows(P, E, K, H, topk_idx, dst_slot, NULL, capacity, y, topk_weights, NULL,
                      tok_begin, tok_end, out);
}

/* Every option at once: exact (capacity 0, rows at window_row_base) or fixed
 * windows, with or without a bias. */
int oracle_combine_general(int P, int S, int E, int K, int H, int64_t capacity,
                           const int64_t *topk_idx, const int32_t *dst_slot,
                           const int64_t *window_row_base, const uint16_t *y,
                           const float *topk_weights, const uint16_t *bias, int64_t tok_begin,
                           int64_t tok_end, uint16_t *out) {
  (void)S;
  if (capacity < 0) return ORACLE_ERR_SHAPE;
  return combine_rows(P, E, K, H, topk_idx, dst_slot, window_row_base, capacity, y, topk_weights,
                      bias, tok_begin, tok_end, out);
}

/* combine(identity_expert(dispatch(x))) for tokens [tok_begin, tok_end),
 * without materialising the expanded tensor: every valid slot of u carries the
 * same dispatched row, so the expert output of each of u's rows is
 *   bf16:  x[u]
 *   fp8:   bf16(fl(decode(code) * scale))  (the identity expert dequantises)
 * and the combine of those rows follows oracle_combine's order.  [TUT] 2.3
 * (combine is the inverse of dispatch). */
static int combine_identity_rows(int K, int H, int fp8, const int64_t *topk_idx,
                                 const uint16_t *x, const float *topk_weights,
                                 const uint16_t *bias, int64_t tok_begin, int64_t tok_end,
                                 uint16_t *out) {
  if (fp8 && H % 128 != 0) return ORACLE_ERR_SHAPE;
  uint16_t *row = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)H);
  uint8_t *codes = (uint8_t *)malloc((size_t)H);
  float *scales = (float *)malloc(sizeof(float) * (size_t)(H / 128 + 1));
  if (!row || !codes || !scales) {
    free(row);
    free(codes);
    free(scales);
    return ORACLE_ERR_SHAPE;
  }
  for (int64_t u = tok_begin; u < tok_end; u++) {
    if (fp8) {
      oracle_quantize_row(x + u * H, H, codes, scales);
      for (int h = 0; h < H; h++)
        row[h] = oracle_bf16_round(oracle_e4m3_decode(codes[h]) * scales[h / 128]);
    } else {
      memcpy(row, x + u * H, sizeof(uint16_t) * (size_t)H);
    }
    for (int h = 0; h < H; h++) {
      float acc = 0.0f;
      for (int j = 0; j < K; j++) {
        if (topk_idx[u * K + j] < 0) continue;
        float w = topk_weights ? topk_weights[u * K + j] : 1.0f;
        float prod = w * oracle_bf16_to_float(row[h]);
        acc = acc + prod;
      }
      if (bias) acc = acc + oracle_bf16_to_float(bias[u * H + h]);
      out[(u - tok_begin) * H + h] = oracle_bf16_round(acc);
    }
  }
  free(row);
  free(codes);
  free(scales);
  return ORACLE_OK;
}

int oracle_combine_identity(int K, int H, int fp8, const int64_t *topk_idx, const uint16_t *x,
                            const float *topk_weights, int64_t tok_begin, int64_t tok_end,
                            uint16_t *out) {
  return combine_identity_rows(K, H, fp8, topk_idx, x, topk_weights, NULL, tok_begin, tok_end, out);
}

/* As oracle_combine_identity, plus combine's optional bias (oracle_combine_general). */
int oracle_combine_identity_bias(int K, int H, int fp8, const int64_t *topk_idx,
                                 const uint16_t *x, const float *topk_weights,
                                 const uint16_t *bias, int64_t tok_begin, int64_t tok_end,
                                 uint16_t *out) {
  return combine_identity_rows(K, H, fp8, topk_idx, x, topk_weights, bias, tok_begin, tok_end,
                               out);
}

/* Array forms of the scalar encoders, for the self-tests. */
void oracle_e4m3_encode_array(const float *q, int64_t n, uint8_t *out) {
  for (int64_t i = 0; i < n; i++) out[i] = oracle_e4m3_encode(q[i]);
}
void oracle_e4m3_decode_array(const uint8_t *c, int64_t n, float *out) {
  for (int64_t i = 0; i < n; i++) out[i] = oracle_e4m3_decode(c[i]);
}
void oracle_bf16_round_array(const float *f, int64_t n, uint16_t *out) {
  for (int64_t i = 0; i < n; i++) out[i] = oracle_bf16_round(f[i]);
}
