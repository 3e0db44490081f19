/*
 * ep_mi355x.h -- C ABI of the single-GPU MoE dispatch / combine path for
 * AMD Instinct MI355X (gfx950).
 *
 * The method: dispatch is a routing-driven All-to-AllV that copies each token
 * row to every expert-parallel (EP) rank holding one of its top-k experts and
 * lays the rows out grouped by expert; combine is its inverse, gathering the
 * k expert outputs of each token and reducing them with the top-k weights.
 * ("Ascend DeepEP MoE Dispatch Optimization", section "A token's journey
 * through MoE"; TileLang tutorial ch. 38 "DeepEP-Ascend", sections 2.1-2.2.)
 *
 * Here the P expert-parallel ranks are *virtual*: each rank's receive buffer
 * is a window (a range of rows) of one expanded tensor in one GPU's HBM, and
 * the remote Put of the multi-device method becomes a coalesced HBM store,
 * ordered by the HIP stream.  No flags, no collectives.
 *
 * Conventions shared by every call
 *  - Every tensor argument is a DEVICE pointer to row-major, contiguous memory
 *    that the caller allocated and owns; the library never allocates a tensor
 *    that the caller sees and never keeps a caller pointer after returning.
 *    bf16 / fp8 row tensors (x, x_codes, recv_x, y, bias, out) must be 16-byte aligned, other
 *    arrays aligned to their element size (else EP_ERR_SHAPE).
 *  - `stream` is a hipStream_t (0 = the null stream).  All device work of a
 *    call is enqueued on it; calls return without waiting for it, except that
 *    ep_get_layout / ep_relayout in exact mode wait for the row counts.
 *  - Token u = s * S + t is token t of virtual rank s (the tutorial's source
 *    token global index, section 2.1); T = P * S.
 *  - Expert e lives on rank e / E_l, E_l = E / P (contiguous blocks; the
 *    tutorial's EP8 example, section 7.2: 256 experts / 8 ranks = 32 local).
 *  - topk_idx[u][j] == -1 marks an unused slot: it is skipped everywhere.  Any
 *    other value outside [0, E) is a routing error.
 *  - A non-OK status leaves outputs unspecified; validation errors return
 *    before anything is enqueued.  ep_last_error() gives a message.
 *  - One handle may be used by any number of ep_dispatch_cached / ep_combine
 *    calls; ep_handle_free and ep_relayout require that none is in flight.
 *    fp8 dispatch with EP_DISPATCH_SCALES_COL_MAJOR (not the pre-quantised
 *    form) stages per-token scales in the handle; the library orders such
 *    calls on one handle itself, on whatever streams, with an event the handle
 *    owns.  Inside a graph capture it neither waits nor records, so the
 *    captured graph must order its own such calls, and a replay must not
 *    overlap such a call made outside the graph.
 *  - A handle belongs to the device that was current at ep_get_layout; calls
 *    that launch work with another device current return
 *    EP_ERR_HANDLE_MISMATCH.
 *  - Two output-length modes ("Ascend DeepEP MoE Dispatch Optimization",
 *    section "Output length has a dynamic and a fixed mode"):
 *      exact  (num_worst_rows == 0): ep_get_layout reads the per-window row
 *             counts back once and sizes the expanded tensors exactly;
 *      fixed  (num_worst_rows == W > 0): every window is W rows, window d is
 *             rows [d*W, (d+1)*W), and nothing is read back: ep_get_layout /
 *             ep_relayout only enqueue.  Rows past a window's num_expanded
 *             (its tail) get payload 0, scales 0, weight 0, meta (-1, -1) on
 *             every dispatch.  A window that needs more than W rows keeps its
 *             first W; the rest are dropped (not written, and skipped by
 *             combine) and ep_handle_status reports EP_STATUS_TRUNCATED.
 */
#ifndef EP_MI355X_H
#define EP_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EP_ABI_VERSION 4

/* Limits of the library. */
#define EP_MAX_RANKS 1024
#define EP_MAX_EXPERTS 4096
#define EP_MAX_TOPK 32

typedef enum {
  EP_OK = 0,
  EP_ERR_NULL = -1,            /* a required pointer is NULL                              */
  EP_ERR_SHAPE = -2,           /* bad sizes: H % 8, (fp8) H % 128, E % P, K, A, limits    */
  EP_ERR_ROUTING = -3,         /* topk_idx outside {-1} U [0, E) (detected on the device) */
  EP_ERR_OVERFLOW = -4,        /* T*K, T*P or the expanded row count reach 2^31           */
  EP_ERR_HANDLE_MISMATCH = -5, /* config differs from the one the handle was built for    */
  EP_ERR_HIP = -6,             /* a HIP runtime call or kernel launch failed              */
  EP_ERR_NOMEM = -7            /* device or pinned host allocation failed                 */
} ep_status;

/* Layout-level flags (ep_config.flags). */
#define EP_LAYOUT_SYMMETRIC_WINDOWS 1u /* every window gets max_d num_expanded rows     */

/* Per-call dispatch flags. */
#define EP_DISPATCH_FP8 1u          /* emit E4M3 codes + fp32 scales per 128 channels  */
#define EP_DISPATCH_ZERO_PADDING 2u /* zero the alignment padding rows' payload         */
#define EP_DISPATCH_SCALES_COL_MAJOR 4u /* fp8: recv_scales as [H/128, total_rows]       */
#define EP_DISPATCH_SCALES_UE8M0 8u /* fp8 with one UE8M0 exponent byte per 32 channels  */
                                    /* (implies EP_DISPATCH_FP8; see ep_dispatch)        */

/* Shape of one dispatch/combine problem.  The tutorial's EPBuffer is built for
 * a token capacity, hidden size and top-k, and dispatch takes num_experts and
 * expert_alignment (TileLang tutorial ch. 38, sections 3.1 and 3.3). */
typedef struct {
  int32_t num_ranks;        /* P, virtual EP ranks, 1..EP_MAX_RANKS                     */
  int32_t num_tokens;       /* S, tokens per rank, >= 0                                  */
  int32_t hidden;           /* H, multiple of 8 (16-byte bf16 vectors)                   */
  int32_t num_topk;         /* K, 1..EP_MAX_TOPK                                         */
  int32_t num_experts;      /* E, multiple of P, <= EP_MAX_EXPERTS                       */
  int32_t expert_alignment; /* A >= 1: every expert's row count is padded to a multiple  */
  uint32_t flags;           /* EP_LAYOUT_* bits                                          */
  int32_t num_worst_rows;   /* 0: exact output length; W > 0: fixed length of W expanded */
                            /* rows per window (the pages' num_worst_tokens); P*W < 2^31 */
                            /* and EP_LAYOUT_SYMMETRIC_WINDOWS unset                      */
} ep_config;

typedef struct ep_handle ep_handle; /* opaque; owns its device arrays */

/* --------------------------------------------------------------------------
 * ep_get_layout -- plan a fresh dispatch ("Ascend DeepEP MoE Dispatch
 * Optimization", sections "Notify exchanges counts and prefixes first" and
 * "What the six handle entries store"; TileLang tutorial ch. 38, sections 2.2,
 * 2.4 and 3.5).
 *
 *   topk_idx  device, int64 [T, K]; read by the work this call enqueues on
 *             `stream` (the handle keeps what it needs, so writes to topk_idx
 *             ordered after that work are harmless).
 *   out       receives a new handle (NULL on error); free with ep_handle_free.
 *   total_rows  host, receives the row count the caller must allocate for the
 *             expanded tensors (recv_x, recv_scales, recv_weights,
 *             recv_src_meta, and the combine input y).  May be NULL.
 *
 * Computes on the device, deterministically (no global atomics):
 *   is_token_in_rank [T,P] u8, num_tokens_per_rank [P,P], num_tokens_per_expert
 *   [P,E], rank_prefix_matrix [P,P] (inclusive over source ranks),
 *   num_recv_tokens [P], aligned per-expert row offsets, num_expanded [P]
 *   (= sum_e ceil(n_e/A)*A over the rank's experts), window row bases,
 *   dst_slot [T,K] (window-local row of each slot, -1 if unused), send_head
 *   [T,P] (position in the destination's receive list, -1 if not sent) and
 *   recv_src_idx (per destination, the local token index of each received
 *   token).  Receive lists are ordered by source rank then token; the rows of
 *   one expert are ordered by (u, j) -- the tutorial's deterministic order.
 * Allocates the handle's device memory (hipMalloc).  Exact mode: waits once
 * for the per-window row counts to reach the host (the pages' do_cpu_sync
 * mode); the last layout kernel may still be running on `stream` when the call
 * returns, and later work on `stream` is ordered after it.  Fixed mode: returns as soon as the work is enqueued, with
 * total_rows = P * num_worst_rows; a routing error does not fail the call
 * (the bad slots are treated as unused) and is reported by ep_handle_status.
 * Before the host uses the counts it checks identities between them (window
 * bases from 0 to total_rows, each window holding its rows, the receive
 * total); counts that still disagree once the layout has finished are
 * EP_ERR_HIP, never a wrong total_rows.
 * Errors: EP_ERR_NULL, EP_ERR_SHAPE, EP_ERR_OVERFLOW, EP_ERR_ROUTING (exact
 * mode), EP_ERR_NOMEM, EP_ERR_HIP.
 */
ep_status ep_get_layout(const ep_config *cfg, const int64_t *topk_idx, void *stream,
                        ep_handle **out, int64_t *total_rows);

/* --------------------------------------------------------------------------
 * ep_buffer_size_hint -- device memory a config needs, computed on the host
 * without allocating or launching anything (TileLang tutorial ch. 38, section
 * 3.2: the size hint that lays the buffers out once and returns the byte
 * count, rounded to 2 MB).
 *   cfg             as for ep_get_layout (validated the same way).
 *   dispatch_flags  EP_DISPATCH_* bits of the dispatches that will run (fp8
 *                   output halves recv_x and adds scales).
 *   out             host, receives:
 *     handle_bytes        the device arena ep_get_layout allocates for the handle;
 *     max_rows            the expanded tensors' row count: P * num_worst_rows in
 *                         fixed mode, else the largest total_rows any routing can
 *                         give, T*K + E*(A-1) (packed windows) or
 *                         P * (T*K + E_l*(A-1)) (symmetric windows);
 *     recv_x_bytes, recv_scales_bytes, recv_weights_bytes, recv_src_meta_bytes
 *                         of max_rows rows (fp8 scales: H/32 bytes a row, fp32
 *                         per 128 channels or UE8M0 per 32);
 *     combine_out_bytes   T * H * 2;
 *     total_bytes         the sum, rounded up to a multiple of 2 MiB.
 * Errors: EP_ERR_NULL, EP_ERR_SHAPE, EP_ERR_OVERFLOW (as ep_get_layout). */
typedef struct {
  int64_t handle_bytes;
  int64_t max_rows;
  int64_t recv_x_bytes;
  int64_t recv_scales_bytes;
  int64_t recv_weights_bytes;
  int64_t recv_src_meta_bytes;
  int64_t combine_out_bytes;
  int64_t total_bytes;
} ep_size_hint;
ep_status ep_buffer_size_hint(const ep_config *cfg, uint32_t dispatch_flags, ep_size_hint *out);

/* ep_relayout -- ep_get_layout into an existing handle for a new topk_idx of
 * the same config, without allocating (one long-lived buffer reused across
 * layers, TileLang tutorial ch. 38, section 2.6).  No call using `h` may be
 * in flight.  On error the handle's layout is invalid until a successful
 * ep_relayout.  Errors: EP_ERR_NULL, EP_ERR_SHAPE (misaligned topk_idx),
 * EP_ERR_HANDLE_MISMATCH (another device is current), EP_ERR_ROUTING (exact
 * mode), EP_ERR_OVERFLOW (symmetric windows reaching 2^31 rows), EP_ERR_HIP
 * (also: exact mode on a stream that is capturing a graph, since the counts
 * must reach the host; fixed mode can be captured). */
ep_status ep_relayout(ep_handle *h, const int64_t *topk_idx, void *stream, int64_t *total_rows);

/* --------------------------------------------------------------------------
 * ep_dispatch -- fresh dispatch into the expanded, expert-grouped layout
 * (TileLang tutorial ch. 38, sections 2.1, 2.2, 3.6 and 4.3).
 *
 *   x             device, bf16 [T, H].
 *   topk_weights  device, fp32 [T, K].
 *   recv_x        device, [total_rows, H]: bf16, or E4M3 bytes with EP_DISPATCH_FP8.
 *   recv_scales   device, fp32 [total_rows, H/128] row-major, or [H/128,
 *                 total_rows] with EP_DISPATCH_SCALES_COL_MAJOR (scale b of row
 *                 r at b * total_rows + r: one scale position contiguous across
 *                 rows, no row padding; TileLang tutorial ch. 38, section 3.6);
 *                 with EP_DISPATCH_SCALES_UE8M0 it holds bytes, uint8
 *                 [total_rows, H/32]: one UE8M0 exponent per 32 channels, so
 *                 that viewed as int16 it is the ceil(H/64) packs of two UE8M0
 *                 per token of the tutorial's size-hint passage (section 3.2);
 *                 required with EP_DISPATCH_FP8 (H % 128 == 0), ignored
 *                 otherwise.
 *   recv_weights  device, fp32 [total_rows].
 *   recv_src_meta device, int32 [total_rows, 2]: (u, j) of the slot a row came
 *                 from ((-1, -1) for padding rows).
 * Row r = window_row_base[rank(e)] + dst_slot[u][j] of every valid slot gets
 * x[u] (bf16 copy, or its E4M3 codes: scale = amax/448 per 128-channel block
 * in fp32, code = E4M3FN round-to-nearest-even of x/scale; a block with amax 0
 * has scale 0 and signed-zero codes; a block holding NaN gets scale 0x7FC00000
 * and codes 0x7F, one holding +-Inf (no NaN) scale +Inf, codes 0x7F for the
 * infinities and signed zeros for finite values; with EP_DISPATCH_SCALES_UE8M0
 * the scale of each 32-channel block is 2^k for the smallest k in [-127, 127]
 * with 448 * 2^k >= amax, stored as the byte k + 127, code = E4M3FN of
 * x / 2^k, and a non-finite block gets the byte 0xFF and the codes above;
 * UE8M0 is row-major, for this call and ep_dispatch_cached only, and not with
 * EP_DISPATCH_SCALES_COL_MAJOR), recv_weights = topk_weights[u][j] and
 * recv_src_meta = (u, j).  Padding rows get weight 0, meta (-1, -1) and, with
 * EP_DISPATCH_ZERO_PADDING, a zero payload (and zero scales); otherwise their
 * payload is left as it was ("Ascend DeepEP MoE Dispatch Optimization",
 * section "Output length has a dynamic and a fixed mode"; tutorial 2.2).
 * Rows past num_expanded in symmetric windows are not touched; in fixed mode
 * they are the tail (zero payload and scales, weight 0, meta (-1, -1)) and
 * slots whose row would lie past the window are not written.
 * Errors: EP_ERR_NULL, EP_ERR_SHAPE (flags, alignment, fp8 with H % 128 != 0),
 * EP_ERR_HANDLE_MISMATCH (no valid layout, or another device is current),
 * EP_ERR_OVERFLOW (launch grid too large), EP_ERR_HIP.
 */
ep_status ep_dispatch(const ep_handle *h, uint32_t flags, const void *x, const float *topk_weights,
                      void *recv_x, float *recv_scales, float *recv_weights,
                      int32_t *recv_src_meta, void *stream);

/* ep_dispatch_noalloc -- ep_dispatch for callers that cannot allocate device
 * memory: code under graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, flags, outputs and errors as ep_dispatch, and
 * it calls no allocating routine.  The one difference is where the fp8
 * column-major path (EP_DISPATCH_FP8 | EP_DISPATCH_SCALES_COL_MAJOR) stages
 * its per-token scales: a fixed array of EP_NOALLOC_SCRATCH_BYTES that the
 * library keeps on every device it runs on until the process ends, instead
 * of the handle.  The first call on a device looks up that array's address.
 * Every call on one GPU shares the array, so two such calls that may overlap
 * on one GPU (other streams, other handles) race and must be ordered by the
 * caller; the handle's own ordering of ep_dispatch calls does not cover them.
 * Extra error: EP_ERR_OVERFLOW when T * (H/128) * 4 bytes exceed the array
 * (fp8 column-major only; other flags stage nothing). */
#define EP_NOALLOC_SCRATCH_BYTES ((int64_t)32 << 20)
ep_status ep_dispatch_noalloc(const ep_handle *h, uint32_t flags, const void *x, const float *topk_weights,
                              void *recv_x, float *recv_scales, float *recv_weights,
                              int32_t *recv_src_meta, void *stream);

/* ep_dispatch_cached -- dispatch with a cached handle: the same routing, new
 * x; only the payload (and fp8 scales) move, padding is re-zeroed when asked
 * ("Ascend DeepEP MoE Dispatch Optimization", section "Entering the real call
 * chain from the Python interface", cached dispatch; tutorial 2.4).  Its
 * payload equals ep_dispatch's for the same x and flags.  Errors as for
 * ep_dispatch. */
ep_status ep_dispatch_cached(const ep_handle *h, uint32_t flags, const void *x, void *recv_x,
                             float *recv_scales, void *stream);

/* ep_dispatch_prequant / ep_dispatch_prequant_cached -- dispatch of input that
 * the caller already quantised: the pair (E4M3 data, fp32 scale per 128
 * channels) that the tutorial's dispatch takes in fp8 mode (TileLang
 * tutorial ch. 38, section 3.6 (2)).
 *   x_codes   device, u8 [T, H] (E4M3FN bytes; copied unchanged, any pattern).
 *   x_scales  device, fp32 [T, H/128] row-major (copied unchanged).
 * The output is fp8 whatever EP_DISPATCH_FP8 says: every valid row gets its
 * token's bytes and scales; everything else is as in ep_dispatch /
 * ep_dispatch_cached (padding, tails, metadata, EP_DISPATCH_SCALES_COL_MAJOR).
 * H % 128 == 0.  Errors as for ep_dispatch. */
ep_status ep_dispatch_prequant(const ep_handle *h, uint32_t flags, const uint8_t *x_codes,
                               const float *x_scales, const float *topk_weights, void *recv_x,
                               float *recv_scales, float *recv_weights, int32_t *recv_src_meta,
                               void *stream);
ep_status ep_dispatch_prequant_cached(const ep_handle *h, uint32_t flags, const uint8_t *x_codes,
                                      const float *x_scales, void *recv_x, float *recv_scales,
                                      void *stream);

/* --------------------------------------------------------------------------
 * ep_combine -- weighted reduction of the K expert rows of every token back
 * to token order (TileLang tutorial ch. 38, sections 2.1, 3.6(5) and 4.5).
 *
 *   y             device, bf16 [total_rows, H] (expert outputs; padding rows
 *                 are never read).
 *   topk_weights  device, fp32 [T, K], or NULL for unit weights.
 *   bias          device, bf16 [T, H], or NULL: the tutorial's optional
 *                 combine bias (a residual or the shared experts' output,
 *                 section 3.3), added once per token.
 *   out           device, bf16 [T, H].
 * out[u][h] = bf16_rne(acc) with acc = +0 and, for j = 0..K-1 over valid
 * slots in order, acc = fl(acc + fl(w[u][j] * float(y[row(u,j)][h]))) in fp32
 * (no fused multiply-add); then, with a bias, acc = fl(acc + float(bias[u][h])).
 * A token without valid slots gets +0 (or its bias).  In fixed mode a slot
 * whose row was dropped counts as unused.
 * The backward of dispatch is this call and the backward of combine is
 * ep_dispatch_cached, with the same handle (tutorial 2.3).
 * Errors: EP_ERR_NULL, EP_ERR_SHAPE (alignment), EP_ERR_HANDLE_MISMATCH (no
 * valid layout, or another device is current), EP_ERR_OVERFLOW (launch grid
 * too large), EP_ERR_HIP.
 */
ep_status ep_combine(const ep_handle *h, const void *y, const float *topk_weights, const void *bias,
                     void *out, void *stream);

/* ep_handle_free -- waits for the handle's own layout work, then releases its
 * device and pinned host memory.  The caller guarantees no other call using
 * `h` is still in flight (tutorial 2.6).  NULL is a no-op. */
void ep_handle_free(ep_handle *h);

/* --------------------------------------------------------------------------
 * Introspection (host-side, no device work; in fixed mode some calls wait for
 * the last layout, as stated).
 */

/* Config the handle was built with. */
ep_status ep_handle_config(const ep_handle *h, ep_config *cfg);

/* EP_ERR_HANDLE_MISMATCH unless cfg's shape fields and flags equal the
 * handle's (the tutorial's cached-handle check of num_experts,
 * expert_alignment and token capacity, section 2.4). */
ep_status ep_handle_check(const ep_handle *h, const ep_config *cfg);

/* Host copies of the read-back counts: num_expanded [P], num_recv_tokens [P],
 * window_row_base [P+1] (int64).  Any pointer may be NULL.  In fixed mode
 * every call waits for the last layout enqueued outside a graph capture, then
 * reads the summary that the last layout to run published (after replaying a
 * graph that holds a layout, wait for the replay before calling). */
ep_status ep_handle_counts(const ep_handle *h, int64_t *num_expanded, int64_t *num_recv_tokens,
                           int64_t *window_row_base);

/* Outcome of the handle's last layout.  flags receives EP_STATUS_* bits;
 * dropped_rows (may be NULL) the number of rows past a fixed window's end,
 * sum_d max(0, num_expanded[d] - num_worst_rows).  Waits as ep_handle_counts
 * does and reads the summary afresh on every call, so a graph replay of the
 * layout is reported once the caller has waited for it (in exact mode the
 * layout has already finished, and both are always 0).
 * Errors: EP_ERR_NULL, EP_ERR_HANDLE_MISMATCH (no layout), EP_ERR_HIP. */
#define EP_STATUS_ROUTING 1u   /* ids outside {-1} U [0, E) were seen and treated as unused */
#define EP_STATUS_TRUNCATED 2u /* some window needed more than num_worst_rows rows            */
ep_status ep_handle_status(const ep_handle *h, uint32_t *flags, int64_t *dropped_rows);

/* Device arrays of the handle, for parity checks and for callers that want
 * the pages' handle tensors.  The pointer stays valid until ep_handle_free /
 * ep_relayout; the caller must not write through it. */
enum {
  EP_T_IS_TOKEN_IN_RANK = 0,      /* u8  [T, P]                                       */
  EP_T_NUM_TOKENS_PER_RANK = 1,   /* i32 [P, P]   [source][destination]               */
  EP_T_NUM_TOKENS_PER_EXPERT = 2, /* i32 [P, E]   [source][expert]                    */
  EP_T_RANK_PREFIX_MATRIX = 3,    /* i32 [P, P]   inclusive over source ranks         */
  EP_T_NUM_RECV_TOKENS = 4,       /* i32 [P]                                          */
  EP_T_NUM_TOKENS_PER_EXPERT_TOTAL = 5, /* i32 [E]                                    */
  EP_T_EXPERT_OFFSET = 6,         /* i64 [P, E_l + 1] window-local, multiples of A    */
  EP_T_NUM_EXPANDED = 7,          /* i64 [P]                                          */
  EP_T_WINDOW_ROW_BASE = 8,       /* i64 [P + 1]                                      */
  EP_T_DST_SLOT = 9,              /* i32 [T, K]   window-local row, -1 if unused      */
  EP_T_SEND_HEAD = 10,            /* i32 [T, P]   receive-list position, -1 if unsent */
  EP_T_RECV_SRC_IDX = 11,         /* i32 [sum num_recv_tokens], destination-major     */
  EP_T_RECV_SRC_BASE = 12,        /* i64 [P + 1]  start of each destination's list    */
  EP_T_DST_ROW = 13,              /* i32 [T, K]   global row (window base + dst_slot), */
                                  /*              -1 if unused or dropped (fixed mode) */
  EP_T_COUNT = 14
};
ep_status ep_handle_tensor(const ep_handle *h, int32_t which, const void **dev_ptr, int64_t *numel,
                           int32_t *elem_bytes);

/* Test hook, not part of the method: converts n floats (device) to OCP E4M3FN
 * bytes (device) with the same device conversion that fp8 dispatch applies to
 * x / scale, so that it can be compared with a reference encoder.  Async on
 * `stream`.  Errors: EP_ERR_NULL, EP_ERR_SHAPE, EP_ERR_OVERFLOW, EP_ERR_HIP. */
ep_status ep_debug_e4m3_encode(const float *in, uint8_t *out, int64_t n, void *stream);

/* Calibration hook, not part of the method: a plain streaming copy of nbytes
 * (a multiple of 1024) from src to dst (device, 16-byte aligned), one wave per
 * KiB with 16-byte nontemporal accesses, the access unit of the dispatch and
 * combine kernels.  Async on `stream`; gives the copy ceiling their bandwidth
 * is compared with.  Errors: EP_ERR_NULL, EP_ERR_SHAPE, EP_ERR_OVERFLOW, EP_ERR_HIP. */
ep_status ep_debug_copy(void *dst, const void *src, int64_t nbytes, void *stream);

/* Profiling hook, not part of the method: the device-side timing slots of a
 * library built with EP_DEVICE_TIMING=1 ("Ascend DeepEP MoE Dispatch
 * Optimization", section "Measure time and bytes correctly first", device-side
 * timing).  Every kernel then stamps the device's constant-rate clock
 * (100 MHz) at its phase boundaries: slot ((kernel * 8 + phase) * 1024 +
 * workgroup) for the first 1024 workgroups, kernel 0 count, 1 scan,
 * 2 finalize, 3 rank, 4 the one-workgroup layout, 5 dispatch, 6 combine.
 * Copies the first n slots (synchronously) into host memory `slots`.  A slot
 * keeps the last stamp written to it.  Built without the switch (the
 * default), the kernels stamp nothing and this returns EP_ERR_SHAPE.
 * Errors: EP_ERR_NULL, EP_ERR_SHAPE, EP_ERR_HIP. */
ep_status ep_debug_timing(uint64_t *slots, int64_t n);

/* Message for the last non-OK status returned on the calling thread. */
const char *ep_last_error(void);

/* EP_ABI_VERSION of the loaded library. */
int32_t ep_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EP_MI355X_H */
