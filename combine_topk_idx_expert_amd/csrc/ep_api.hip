// ep_api.hip -- host side of the C ABI declared in include/ep_mi355x.h.
//
// Validation and status codes follow the pages' host path: missing routing
// tensors are errors, capacities are computed with checked products, and a
// cached handle must match the config it is used with ("Ascend DeepEP MoE
// Dispatch Optimization", sections "Entering the real call chain from the
// Python interface" and "Host side: building a communication map"; TileLang
// tutorial ch. 38, section 2.4).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "ep_mi355x.h"
#include "ep_dispatch.hpp"
#include "ep_layout.hpp"

using namespace ep;

namespace {

thread_local std::string g_last_error;

ep_status fail(ep_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

#define EP_HIP(call)                                                                      \
  do {                                                                                    \
    hipError_t e_ = (call);                                                               \
    if (e_ != hipSuccess) return fail(EP_ERR_HIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

#define EP_LAUNCHED(name)                                                                     \
  do {                                                                                        \
    hipError_t e_ = hipGetLastError();                                                        \
    if (e_ != hipSuccess) return fail(EP_ERR_HIP, "launch of %s: %s", name, hipGetErrorString(e_)); \
  } while (0)

bool misaligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) != 0; }

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

}  // namespace

struct ep_handle {
  ep_config cfg;
  LayoutDims dims;
  int64_t T;
  int device;
  // read back by the layout (fixed windows: on every query, see ensure_counts)
  int64_t total_rows = 0, total_pad = 0, sum_recv = 0, sum_expanded = 0;
  int64_t dropped = 0;
  uint32_t status = 0;  // EP_STATUS_* of the last layout
  bool valid = false;
  bool fixed = false;          // num_worst_rows > 0
  bool counts_known = false;   // host fields above hold the last layout's summary
  // device arena and the arrays inside it
  void* arena = nullptr;
  size_t arena_bytes = 0;
  uint8_t* is_token_in_rank;
  int32_t *num_tokens_per_rank, *num_tokens_per_expert, *rank_prefix_matrix, *num_recv, *n_e;
  int64_t *expert_offset, *num_expanded, *window_row_base, *recv_src_base;
  int32_t *dst_slot, *dst_row, *send_head, *recv_src_idx;
  int32_t *pad_base, *pad_rows, *chunk_hist, *chunk_excl_t, *col_total, *row_slot;
  int64_t* packed_base;
  int64_t* tail_base;
  float* tok_scales = nullptr;  // fp8 per-token scales (H % 128 == 0 only)
  int64_t* summary_dev;
  int64_t* summary_host = nullptr;      // pinned; the finalize kernel writes it directly
  int64_t* summary_host_dev = nullptr;  // its device address
  int64_t layout_seq = 0;               // sequence number of the last enqueued layout
  bool done_recorded = false;       // done_ev marks an eager layout (not one captured in a graph)
  hipEvent_t done = nullptr;        // end of the last eager four-kernel layout's work
  hipEvent_t summary_ready = nullptr;  // the last exact layout's host summary has landed
  hipEvent_t done_ev = nullptr;     // the event that marks the end of the last eager layout's work
  hipEvent_t cm_done = nullptr;     // end of the last column-major fp8 dispatch (tok_scales free again)
  bool cm_recorded = false;
  size_t lds_count, lds_scan, lds_finalize, lds_rank, lds_small;
  bool small_layout = false;  // the whole layout in one workgroup (layout_small_kernel)
};

namespace {

ep_status validate_config(const ep_config* c) {
  if (!c) return fail(EP_ERR_NULL, "config is NULL");
  if (c->num_ranks < 1 || c->num_ranks > EP_MAX_RANKS)
    return fail(EP_ERR_SHAPE, "num_ranks %d outside [1, %d]", c->num_ranks, EP_MAX_RANKS);
  if (c->num_tokens < 0) return fail(EP_ERR_SHAPE, "num_tokens %d < 0", c->num_tokens);
  if (c->hidden < 8 || c->hidden % 8 != 0)
    return fail(EP_ERR_SHAPE, "hidden %d must be a positive multiple of 8", c->hidden);
  if (c->num_topk < 1 || c->num_topk > EP_MAX_TOPK)
    return fail(EP_ERR_SHAPE, "num_topk %d outside [1, %d]", c->num_topk, EP_MAX_TOPK);
  if (c->num_experts < c->num_ranks || c->num_experts % c->num_ranks != 0 ||
      c->num_experts > EP_MAX_EXPERTS)
    return fail(EP_ERR_SHAPE, "num_experts %d must be a multiple of num_ranks %d, <= %d",
                c->num_experts, c->num_ranks, EP_MAX_EXPERTS);
  if (c->expert_alignment < 1) return fail(EP_ERR_SHAPE, "expert_alignment %d < 1", c->expert_alignment);
  if (c->flags & ~EP_LAYOUT_SYMMETRIC_WINDOWS) return fail(EP_ERR_SHAPE, "unknown layout flags 0x%x", c->flags);
  if (c->num_worst_rows < 0) return fail(EP_ERR_SHAPE, "num_worst_rows %d < 0", c->num_worst_rows);
  if (c->num_worst_rows > 0 && (c->flags & EP_LAYOUT_SYMMETRIC_WINDOWS))
    return fail(EP_ERR_SHAPE, "num_worst_rows fixes the window size; EP_LAYOUT_SYMMETRIC_WINDOWS must be unset");
  const int64_t T = (int64_t)c->num_ranks * c->num_tokens;
  const int64_t lim = (int64_t)1 << 31;
  if ((int64_t)c->num_ranks * c->num_worst_rows >= lim)
    return fail(EP_ERR_OVERFLOW, "P * num_worst_rows = %lld reaches 2^31",
                (long long)((int64_t)c->num_ranks * c->num_worst_rows));
  if (T * c->num_topk >= lim) return fail(EP_ERR_OVERFLOW, "T*K = %lld reaches 2^31", (long long)(T * c->num_topk));
  if (T * c->num_ranks >= lim) return fail(EP_ERR_OVERFLOW, "T*P = %lld reaches 2^31", (long long)(T * c->num_ranks));
  const int64_t max_rows = T * c->num_topk + (int64_t)c->num_experts * (c->expert_alignment - 1);
  if (max_rows >= lim) return fail(EP_ERR_OVERFLOW, "expanded rows may reach 2^31 (bound %lld)", (long long)max_rows);
  return EP_OK;
}

LayoutDims make_dims(const ep_config& c) {
  LayoutDims d;
  d.P = c.num_ranks;
  d.S = c.num_tokens;
  d.E = c.num_experts;
  d.K = c.num_topk;
  d.A = c.expert_alignment;
  d.El = d.E / d.P;
  d.cpr = (d.S + kChunk - 1) / kChunk;
  d.num_chunks = d.P * d.cpr;
  d.ncols = d.E + d.P + 1;
  d.ebits = bits_for((uint32_t)d.E);
  d.pbits = bits_for((uint32_t)d.P);
  d.symmetric = (c.flags & EP_LAYOUT_SYMMETRIC_WINDOWS) ? 1 : 0;
  d.cap = c.num_worst_rows;
  return d;
}

// The handle's device arrays, laid end to end in one arena (each aligned to
// 256 bytes): returns the arena's size; with base != nullptr, also points the
// handle's members into it.  Uses only h->cfg, h->dims and h->T.
size_t arena_layout(ep_handle* h, uint8_t* base) {
  const LayoutDims& d = h->dims;
  const int64_t T = h->T, P = d.P, E = d.E, K = d.K;
  struct Item {
    void** ptr;
    size_t bytes;
  };
  const int64_t max_pad = E * (d.A - 1);
  Item items[] = {
      {(void**)&h->is_token_in_rank, (size_t)(T * P)},
      {(void**)&h->num_tokens_per_rank, (size_t)(P * P * 4)},
      {(void**)&h->num_tokens_per_expert, (size_t)(P * E * 4)},
      {(void**)&h->rank_prefix_matrix, (size_t)(P * P * 4)},
      {(void**)&h->num_recv, (size_t)(P * 4)},
      {(void**)&h->n_e, (size_t)(E * 4)},
      {(void**)&h->expert_offset, (size_t)(P * (d.El + 1) * 8)},
      {(void**)&h->num_expanded, (size_t)(P * 8)},
      {(void**)&h->window_row_base, (size_t)((P + 1) * 8)},
      {(void**)&h->recv_src_base, (size_t)((P + 1) * 8)},
      {(void**)&h->dst_slot, (size_t)(T * K * 4)},
      {(void**)&h->dst_row, (size_t)(T * K * 4)},
      {(void**)&h->send_head, (size_t)(T * P * 4)},
      {(void**)&h->recv_src_idx, (size_t)(T * std::min<int64_t>(K, P) * 4)},
      {(void**)&h->pad_base, (size_t)((E + 1) * 4)},
      {(void**)&h->pad_rows, (size_t)(std::max<int64_t>(max_pad, 1) * 4)},
      {(void**)&h->chunk_hist, (size_t)((int64_t)d.ncols * d.num_chunks * 4)},
      {(void**)&h->chunk_excl_t, (size_t)((int64_t)d.ncols * d.num_chunks * 4)},
      {(void**)&h->col_total, (size_t)(d.ncols * 4)},
      {(void**)&h->summary_dev, (size_t)((kSummaryHeader + 3 * P + 1) * 8)},
      {(void**)&h->row_slot, (size_t)((T * K + max_pad) * 4)},
      {(void**)&h->packed_base, (size_t)((P + 1) * 8)},
      {(void**)&h->tail_base, (size_t)((P + 1) * 8)},
      {(void**)&h->tok_scales, (size_t)(h->cfg.hidden % 128 == 0 ? T * (h->cfg.hidden / 128) * 4 : 0)},
  };
  size_t off = 0;
  for (const Item& it : items) {
    if (base) *it.ptr = base + off;
    off += align_up(std::max<size_t>(it.bytes, 1));
  }
  return off;
}

ep_status allocate(ep_handle* h) {
  const LayoutDims& d = h->dims;
  const int64_t P = d.P;
  const size_t total = arena_layout(h, nullptr);
  hipError_t e = hipMalloc(&h->arena, total);
  if (e != hipSuccess) return fail(EP_ERR_NOMEM, "hipMalloc(%zu): %s", total, hipGetErrorString(e));
  h->arena_bytes = total;
  arena_layout(h, (uint8_t*)h->arena);
  e = hipHostMalloc((void**)&h->summary_host, (size_t)((kSummaryHeader + 3 * P + 2) * 8),
                    hipHostMallocMapped | hipHostMallocCoherent);
  if (e != hipSuccess) return fail(EP_ERR_NOMEM, "hipHostMalloc: %s", hipGetErrorString(e));
  std::memset(h->summary_host, 0, (size_t)((kSummaryHeader + 3 * P + 2) * 8));
  e = hipHostGetDevicePointer((void**)&h->summary_host_dev, h->summary_host, 0);
  if (e != hipSuccess) return fail(EP_ERR_HIP, "hipHostGetDevicePointer: %s", hipGetErrorString(e));
  e = hipEventCreateWithFlags(&h->summary_ready, hipEventDisableTiming);
  if (e != hipSuccess) return fail(EP_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(e));
  e = hipEventCreateWithFlags(&h->done, hipEventDisableTiming);
  if (e != hipSuccess) return fail(EP_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(e));
  e = hipEventCreateWithFlags(&h->cm_done, hipEventDisableTiming);
  if (e != hipSuccess) return fail(EP_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(e));

  h->lds_count = (size_t)(kLayoutWaves * d.ncols + kChunk * ((d.P + 31) / 32) + kChunk * d.K) * 4;
  h->lds_scan = (size_t)(((d.P + 2) & ~1) * 4 + (kScanThreads / 64) * 8);
  h->lds_finalize = (size_t)finalize_lds_words(d, kFinalizeThreads) * 8 + (size_t)d.ncols * 4;
  h->lds_rank = (size_t)(kLayoutWaves * d.ncols + 2 * kChunk * d.K) * 4;
  h->lds_small = small_lds_bytes(d);
  int lds_max = 0;
  if (hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, h->device) != hipSuccess)
    return fail(EP_ERR_HIP, "hipDeviceGetAttribute(MaxSharedMemoryPerBlock) failed");
  const size_t lds_need = std::max({h->lds_count, h->lds_scan, h->lds_finalize, h->lds_rank});
  if (lds_need > (size_t)lds_max)
    return fail(EP_ERR_SHAPE, "layout needs %zu bytes of LDS per workgroup, the device has %d (E=%d P=%d K=%d)",
                lds_need, lds_max, d.E, d.P, d.K);
  // small batches: one launch for the whole layout when it fits one workgroup
  // and its chunks are light enough for one wave each
  const int64_t chunk_slots = (int64_t)std::min(d.S, kChunk) * d.K;
  h->small_layout = d.num_chunks <= kSmallChunks && chunk_slots <= kSmallMaxChunkSlots &&
                    h->lds_small <= kSmallLdsMax && h->lds_small <= (size_t)lds_max;
  return EP_OK;
}

void release(ep_handle* h) {
  if (!h) return;
  if (h->cm_done) {
    if (h->cm_recorded) (void)hipEventSynchronize(h->cm_done);
    (void)hipEventDestroy(h->cm_done);
  }
  if (h->done_recorded && h->done_ev) (void)hipEventSynchronize(h->done_ev);
  if (h->done) (void)hipEventDestroy(h->done);
  if (h->summary_ready) (void)hipEventDestroy(h->summary_ready);
  if (h->arena) (void)hipFree(h->arena);
  if (h->summary_host) (void)hipHostFree(h->summary_host);
  delete h;
}

// Wait until the last enqueued layout's finalize kernel has written the host
// summary: spin on the sequence number it writes last (coherent pinned
// memory), asking the event now and then, so that a stream that fails or has
// already passed the kernel also ends the wait.
ep_status wait_summary(ep_handle* h) {
  int64_t* flag = h->summary_host + kSummaryHeader + 3 * h->dims.P + 1;
  for (uint32_t i = 1;; ++i) {
    if (__atomic_load_n(flag, __ATOMIC_ACQUIRE) == h->layout_seq) return EP_OK;
    if ((i & 255) == 0) {
      const hipError_t e = hipEventQuery(h->summary_ready);
      if (e == hipSuccess) break;
      if (e != hipErrorNotReady) return fail(EP_ERR_HIP, "layout: %s", hipGetErrorString(e));
    }
  }
  if (__atomic_load_n(flag, __ATOMIC_ACQUIRE) != h->layout_seq)
    return fail(EP_ERR_HIP, "layout finished without publishing its summary");
  return EP_OK;
}

// Identities the finalize step guarantees between the words of the host
// summary: the windows start at 0 and end at the total row count, each holds
// its rows (exact windows; symmetric ones may hold more), and the receive
// total is the sum of the per-rank receive counts.  The words and the
// sequence number reach host memory as separate writes over the bus, so the
// host checks them before it trusts a row count that sizes the caller's
// buffers.
bool summary_consistent(const ep_handle* h) {
  const int64_t* sm = h->summary_host;
  const int P = h->dims.P;
  const int64_t* ne = sm + kSummaryHeader;
  const int64_t* nr = ne + P;
  const int64_t* wb = nr + P;
  if (wb[0] != 0 || wb[P] != sm[0]) return false;
  int64_t recv = 0;
  for (int r = 0; r < P; ++r) {
    recv += nr[r];
    if (!h->fixed && wb[r + 1] - wb[r] < ne[r]) return false;
  }
  return recv == sm[3];
}

// True when `s` is capturing into a graph.  A failing query (for instance of
// the null stream while another stream captures) counts as "not capturing"
// and its error is cleared so that the launch checks below do not see it.
bool stream_capturing(hipStream_t s) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return cs != hipStreamCaptureStatusNone;
}

// Enqueue the layout for the handle's config and read back the summary.
// Exact windows wait for the row counts on the host, so they cannot be
// captured; fixed windows only enqueue, so they can.  A captured layout
// records no events: the graph's replays publish their summaries into the
// pinned host buffer, which status queries read after the caller has waited
// for the replay.  An eager layout records as few events as it needs, since
// each record costs the GPU ~4.5 us (measured on MI355X): summary_ready only
// for exact windows (the host's wait for the counts ends on it), and one
// event for the end of all layout work -- the same event when one kernel does
// everything.
ep_status run_layout(ep_handle* h, const int64_t* topk_idx, hipStream_t s, int64_t* total_rows) {
  h->valid = false;
  const LayoutDims& d = h->dims;
  const bool capturing = stream_capturing(s);
  if (capturing && !h->fixed)
    return fail(EP_ERR_HIP, "exact windows read the row counts back to the host and cannot be captured in a "
                            "graph; use fixed windows (num_worst_rows > 0)");
  FinalizeOut fo{h->n_e, h->expert_offset, h->num_expanded, h->window_row_base, h->num_recv,
                 h->recv_src_base, h->pad_base, h->pad_rows, h->packed_base, h->row_slot, h->tail_base,
                 h->summary_dev, h->summary_host_dev, ++h->layout_seq};
  RankOut ro{h->dst_slot, h->dst_row, h->row_slot, h->send_head, h->recv_src_idx, h->pad_rows};
  RankIn ri{h->chunk_excl_t, h->n_e, h->pad_base, h->expert_offset, h->window_row_base, h->packed_base,
            h->recv_src_base};
  hipEvent_t end_ev = h->done;
  if (h->small_layout) {
    layout_small_kernel<<<1, kSmallThreads, h->lds_small, s>>>(d, topk_idx, h->is_token_in_rank,
                                                               h->num_tokens_per_expert, h->num_tokens_per_rank,
                                                               h->rank_prefix_matrix, fo, ri, ro);
    EP_LAUNCHED("layout_small_kernel");
    if (!h->fixed) end_ev = h->summary_ready;  // summary and ranks come from the one kernel
  } else {
    if (d.num_chunks > 0) {
      layout_count_kernel<<<d.num_chunks, kLayoutThreads, h->lds_count, s>>>(d, topk_idx, h->is_token_in_rank,
                                                                     h->chunk_hist);
      EP_LAUNCHED("layout_count_kernel");
    }
    layout_scan_kernel<<<d.ncols, kScanThreads, h->lds_scan, s>>>(
        d, h->chunk_hist, h->chunk_excl_t, h->col_total, h->num_tokens_per_expert, h->num_tokens_per_rank,
        h->rank_prefix_matrix);
    EP_LAUNCHED("layout_scan_kernel");
    layout_finalize_kernel<<<1, kFinalizeThreads, h->lds_finalize, s>>>(d, h->col_total, fo);
    EP_LAUNCHED("layout_finalize_kernel");
    if (!capturing && !h->fixed)
      EP_HIP(hipEventRecord(h->summary_ready, s));  // the finalize kernel wrote the host summary
    // at least one workgroup, so that the padding rows are written even when T = 0
    layout_rank_kernel<<<std::max(d.num_chunks, 1), kLayoutThreads, h->lds_rank, s>>>(d, topk_idx, ri, ro);
    EP_LAUNCHED("layout_rank_kernel");
  }
  if (!capturing) EP_HIP(hipEventRecord(end_ev, s));
  h->done_ev = end_ev;
  h->done_recorded = !capturing;
  h->counts_known = false;
  if (h->fixed) {  // fixed windows: nothing to wait for
    h->total_rows = (int64_t)d.P * d.cap;
    h->valid = true;
    if (total_rows) *total_rows = h->total_rows;
    return EP_OK;
  }
  // The host needs only the summary; the rank kernel keeps running meanwhile,
  // so the caller's next launches queue up behind it without a gap.
  if (ep_status st = wait_summary(h); st != EP_OK) return st;
  if (!summary_consistent(h)) {  // read it again once the layout's writes have all landed
    const hipError_t e = hipEventSynchronize(h->summary_ready);
    if (e != hipSuccess) return fail(EP_ERR_HIP, "layout: %s", hipGetErrorString(e));
    if (!summary_consistent(h)) return fail(EP_ERR_HIP, "layout summary in host memory is inconsistent");
  }
  const int64_t* sm = h->summary_host;
  if (sm[2] != 0) return fail(EP_ERR_ROUTING, "topk_idx holds an expert id outside {-1} U [0, %d)", d.E);
  if (sm[0] >= ((int64_t)1 << 31))
    return fail(EP_ERR_OVERFLOW, "expanded rows %lld reach 2^31 (symmetric windows)", (long long)sm[0]);
  h->total_rows = sm[0];
  h->total_pad = sm[1];
  h->sum_expanded = 0;
  for (int r = 0; r < d.P; ++r) h->sum_expanded += sm[kSummaryHeader + r];
  h->sum_recv = sm[3];
  h->status = 0;
  h->dropped = 0;
  h->counts_known = true;
  h->valid = true;
  if (total_rows) *total_rows = h->total_rows;
  return EP_OK;
}

// Host copies of the layout summary (mutable caches of device results).
// Exact windows read it once, in run_layout.  Fixed windows read it on every
// query: after waiting for the last eager layout, the pinned buffer holds the
// summary of the last layout that ran, which may be a graph replay enqueued
// after it (the caller waits for a replay before asking), so nothing is cached.
ep_status ensure_counts(const ep_handle* hc) {
  ep_handle* h = const_cast<ep_handle*>(hc);
  if (h->counts_known) return EP_OK;
  if (h->done_recorded) {
    const hipError_t e = hipEventSynchronize(h->done_ev);
    if (e != hipSuccess) return fail(EP_ERR_HIP, "layout: %s", hipGetErrorString(e));
  }
  if (!summary_consistent(h)) return fail(EP_ERR_HIP, "layout summary in host memory is inconsistent");
  const int64_t* sm = h->summary_host;
  h->total_pad = sm[1];
  h->sum_recv = sm[3];
  h->sum_expanded = 0;
  for (int r = 0; r < h->dims.P; ++r) h->sum_expanded += sm[kSummaryHeader + r];
  h->dropped = sm[5];
  h->status = (sm[2] != 0 ? EP_STATUS_ROUTING : 0u) | (sm[5] > 0 ? EP_STATUS_TRUNCATED : 0u);
  return EP_OK;
}

// Plain streaming copy for calibration: one wave per KiB, one nontemporal
// 16-byte load and store per lane (the access unit of the row kernels).
__global__ __launch_bounds__(256) void copy_kernel(u32x4* __restrict__ dst, const u32x4* __restrict__ src,
                                                   int64_t waves) {
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= waves) return;
  const int64_t i = w * kWave + (threadIdx.x & 63);
  __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

ep_status check_handle(const ep_handle* h) {
  if (!h) return fail(EP_ERR_NULL, "handle is NULL");
  if (!h->valid) return fail(EP_ERR_HANDLE_MISMATCH, "handle holds no valid layout");
  return EP_OK;
}

// Calls that launch work must run with the handle's device current: its
// arrays live there, and kernels go to the current device.
ep_status check_device(const ep_handle* h) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return fail(EP_ERR_HIP, "hipGetDevice failed");
  if (cur != h->device)
    return fail(EP_ERR_HANDLE_MISMATCH, "handle lives on device %d, the current device is %d", h->device, cur);
  return EP_OK;
}

#include "ep_launch.hpp"

}  // namespace

// Staging memory of ep_dispatch_noalloc: the per-token fp8 scales that the
// column-major scale pass reads, in a fixed array that every GPU the library
// runs on holds until the process ends.  Host code never uses this name as an
// address (on the host it is only a stand-in): the device address comes from
// hipGetSymbolAddress, once per device, in noalloc_scratch().
static __device__ __align__(256) float scratch[EP_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call on that device, then kept).
ep_status noalloc_scratch(int device, float** out) {
  if (device < 0 || device >= kMaxDevices) return fail(EP_ERR_HIP, "device %d beyond the library's table", device);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(EP_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", device, hipGetErrorString(e));
    g_scratch_dev[device] = (float*)p;
  }
  *out = g_scratch_dev[device];
  return EP_OK;
}

// x: bf16 [T][H]; or, with prequant, E4M3 codes [T][H] and x_scales [T][H/128].
// staging: where the column-major fp8 path stages per-token scales (null: the
// handle's tok_scales, ordered across calls by the handle's event).
ep_status dispatch_common(const ep_handle* h, uint32_t flags, const void* x, const float* x_scales, bool prequant,
                          const float* w, void* recv_x, float* recv_scales, float* recv_weights,
                          int32_t* recv_meta, bool meta, hipStream_t s, float* staging = nullptr) {
  ep_status st = check_handle(h);
  if (st == EP_OK) st = check_device(h);
  if (st != EP_OK) return st;
  if (flags & ~(uint32_t)(EP_DISPATCH_FP8 | EP_DISPATCH_ZERO_PADDING | EP_DISPATCH_SCALES_COL_MAJOR |
                          EP_DISPATCH_SCALES_UE8M0))
    return fail(EP_ERR_SHAPE, "unknown dispatch flags 0x%x", flags);
  const bool ue8m0 = flags & EP_DISPATCH_SCALES_UE8M0;
  if (ue8m0 && (prequant || (flags & EP_DISPATCH_SCALES_COL_MAJOR)))
    return fail(EP_ERR_SHAPE, "UE8M0 scales are row-major and come from the fused quantisation: not with "
                              "EP_DISPATCH_SCALES_COL_MAJOR or pre-quantised input");
  const bool fp8 = (flags & EP_DISPATCH_FP8) || prequant || ue8m0;
  const bool zero_pad = flags & EP_DISPATCH_ZERO_PADDING;
  if (fp8 && h->cfg.hidden % 128 != 0)
    return fail(EP_ERR_SHAPE, "fp8 dispatch needs hidden %% 128 == 0 (hidden %d)", h->cfg.hidden);
  const bool rows = h->total_rows > 0;
  if (h->T > 0 && !x) return fail(EP_ERR_NULL, prequant ? "x_codes is NULL" : "x is NULL");
  if (prequant && h->T > 0 && !x_scales) return fail(EP_ERR_NULL, "x_scales is NULL");
  if (misaligned(x_scales, 4)) return fail(EP_ERR_SHAPE, "x_scales must be 4-byte aligned");
  if (rows && !recv_x) return fail(EP_ERR_NULL, "recv_x is NULL");
  if (rows && fp8 && !recv_scales) return fail(EP_ERR_NULL, "recv_scales is NULL (fp8)");
  if (meta && h->T > 0 && !w) return fail(EP_ERR_NULL, "topk_weights is NULL");
  if (meta && rows && (!recv_weights || !recv_meta)) return fail(EP_ERR_NULL, "recv_weights / recv_src_meta is NULL");
  if (misaligned(x, 16) || misaligned(recv_x, 16) || misaligned(recv_scales, 4) || misaligned(w, 4) ||
      misaligned(recv_weights, 4) || misaligned(recv_meta, 8))
    return fail(EP_ERR_SHAPE, "x / recv_x must be 16-byte aligned, fp32 and int32 arrays naturally aligned");
  DispatchArgs a;
  a.x = (const uint16_t*)x;
  a.w = w;
  a.dst_row = h->dst_row;
  a.pad_rows = h->pad_rows;
  a.row_slot = h->row_slot;
  a.packed_base = h->packed_base;
  a.window_row_base = h->window_row_base;
  a.recv_x = recv_x;
  a.recv_scales = recv_scales;
  a.tok_scales = h->tok_scales;
  a.recv_weights = recv_weights;
  a.recv_meta = recv_meta;
  a.T = (int)h->T;
  a.K = h->dims.K;
  a.H = h->cfg.hidden;
  a.P = h->dims.P;
  a.total_pad = (int)h->total_pad;
  a.sum_expanded = (int)h->sum_expanded;
  a.split = 1;
  a.zero_pad = zero_pad ? 1 : 0;
  a.symmetric = h->dims.symmetric;
  a.cap = h->dims.cap;
  a.zero_waves = 0;
  a.counts = h->summary_dev;
  a.tail_base = h->tail_base;
  a.num_expanded = h->num_expanded;
  a.x_codes = prequant ? (const uint8_t*)x : nullptr;
  a.scales_cm = (flags & EP_DISPATCH_SCALES_COL_MAJOR) ? 1 : 0;
  a.scale_rows = h->total_rows;
  if (prequant) {
    a.x = nullptr;
    a.tok_scales = const_cast<float*>(x_scales);  // read only: the rows' scales come from here
    return meta ? launch_dispatch_mode<true, true, true>(a, s) : launch_dispatch_mode<true, false, true>(a, s);
  }
  if (ue8m0)
    return meta ? launch_dispatch_mode<true, true, false, true>(a, s) : launch_dispatch_mode<true, false, false, true>(a, s);
  if (fp8 && a.scales_cm && staging) {
    a.tok_scales = staging;  // the caller's fixed staging: no handle state, no ordering
    return meta ? launch_dispatch_mode<true, true, false>(a, s) : launch_dispatch_mode<true, false, false>(a, s);
  }
  if (fp8 && a.scales_cm) {
    // The per-token scales are staged in the handle's tok_scales: order this
    // call after the previous such call on the handle, whatever its stream
    // (an event wait on the device, no host synchronisation).  A graph capture
    // neither waits nor records; calls inside one graph are ordered by it.
    ep_handle* hm = const_cast<ep_handle*>(h);
    const bool capturing = stream_capturing(s);
    if (!capturing && hm->cm_recorded) EP_HIP(hipStreamWaitEvent(s, hm->cm_done, 0));
    st = meta ? launch_dispatch_mode<true, true, false>(a, s) : launch_dispatch_mode<true, false, false>(a, s);
    if (st == EP_OK && !capturing) {
      EP_HIP(hipEventRecord(hm->cm_done, s));
      hm->cm_recorded = true;
    }
    return st;
  }
  if (fp8) return meta ? launch_dispatch_mode<true, true, false>(a, s) : launch_dispatch_mode<true, false, false>(a, s);
  return meta ? launch_dispatch_mode<false, true, false>(a, s) : launch_dispatch_mode<false, false, false>(a, s);
}

}  // namespace

extern "C" {

ep_status ep_get_layout(const ep_config* cfg, const int64_t* topk_idx, void* stream, ep_handle** out,
                        int64_t* total_rows) {
  if (!out) return fail(EP_ERR_NULL, "out is NULL");
  *out = nullptr;
  ep_status st = validate_config(cfg);
  if (st != EP_OK) return st;
  const int64_t T = (int64_t)cfg->num_ranks * cfg->num_tokens;
  if (T > 0 && !topk_idx) return fail(EP_ERR_NULL, "topk_idx is NULL");
  if (misaligned(topk_idx, 8)) return fail(EP_ERR_SHAPE, "topk_idx must be 8-byte aligned");
  ep_handle* h = new ep_handle();
  h->cfg = *cfg;
  h->dims = make_dims(*cfg);
  h->T = T;
  h->fixed = cfg->num_worst_rows > 0;
  if (hipGetDevice(&h->device) != hipSuccess) {
    delete h;
    return fail(EP_ERR_HIP, "no HIP device");
  }
  st = allocate(h);
  if (st == EP_OK) st = run_layout(h, topk_idx, (hipStream_t)stream, total_rows);
  if (st != EP_OK) {
    const std::string msg = g_last_error;
    release(h);
    g_last_error = msg;
    return st;
  }
  *out = h;
  return EP_OK;
}

ep_status ep_buffer_size_hint(const ep_config* cfg, uint32_t dispatch_flags, ep_size_hint* out) {
  if (!out) return fail(EP_ERR_NULL, "out is NULL");
  ep_status st = validate_config(cfg);
  if (st != EP_OK) return st;
  if (dispatch_flags & ~(uint32_t)(EP_DISPATCH_FP8 | EP_DISPATCH_ZERO_PADDING | EP_DISPATCH_SCALES_COL_MAJOR |
                                   EP_DISPATCH_SCALES_UE8M0))
    return fail(EP_ERR_SHAPE, "unknown dispatch flags 0x%x", dispatch_flags);
  const bool fp8 = dispatch_flags & (EP_DISPATCH_FP8 | EP_DISPATCH_SCALES_UE8M0);
  if (fp8 && cfg->hidden % 128 != 0)
    return fail(EP_ERR_SHAPE, "fp8 dispatch needs hidden %% 128 == 0 (hidden %d)", cfg->hidden);
  ep_handle probe;  // sizes only: nothing is allocated
  probe.cfg = *cfg;
  probe.dims = make_dims(*cfg);
  probe.T = (int64_t)cfg->num_ranks * cfg->num_tokens;
  const LayoutDims& d = probe.dims;
  const int64_t T = probe.T, H = cfg->hidden;
  // every slot valid and every expert one row short of a multiple of A: the
  // largest total_rows a layout can give (symmetric windows: P times the
  // largest window, itself at most all slots plus one rank's padding)
  const int64_t packed = T * d.K + (int64_t)d.E * (d.A - 1);
  int64_t rows = packed;
  if (cfg->num_worst_rows > 0)
    rows = (int64_t)d.P * cfg->num_worst_rows;
  else if (d.symmetric)
    rows = (int64_t)d.P * (T * d.K + (int64_t)d.El * (d.A - 1));
  out->handle_bytes = (int64_t)arena_layout(&probe, nullptr);
  out->max_rows = rows;
  out->recv_x_bytes = rows * H * (fp8 ? 1 : 2);
  out->recv_scales_bytes = fp8 ? rows * (H / 32) : 0;  // fp32 per 128 or UE8M0 per 32: H/32 bytes a row
  out->recv_weights_bytes = rows * 4;
  out->recv_src_meta_bytes = rows * 8;
  out->combine_out_bytes = T * H * 2;
  const int64_t sum = out->handle_bytes + out->recv_x_bytes + out->recv_scales_bytes + out->recv_weights_bytes +
                      out->recv_src_meta_bytes + out->combine_out_bytes;
  const int64_t mib2 = (int64_t)2 << 20;
  out->total_bytes = (sum + mib2 - 1) / mib2 * mib2;
  return EP_OK;
}

ep_status ep_relayout(ep_handle* h, const int64_t* topk_idx, void* stream, int64_t* total_rows) {
  if (!h) return fail(EP_ERR_NULL, "handle is NULL");
  ep_status st = check_device(h);
  if (st != EP_OK) return st;
  if (h->T > 0 && !topk_idx) return fail(EP_ERR_NULL, "topk_idx is NULL");
  if (misaligned(topk_idx, 8)) return fail(EP_ERR_SHAPE, "topk_idx must be 8-byte aligned");
  return run_layout(h, topk_idx, (hipStream_t)stream, total_rows);
}

ep_status ep_dispatch(const ep_handle* h, uint32_t flags, const void* x, const float* topk_weights,
                      void* recv_x, float* recv_scales, float* recv_weights, int32_t* recv_src_meta,
                      void* stream) {
  return dispatch_common(h, flags, x, nullptr, false, topk_weights, recv_x, recv_scales, recv_weights,
                         recv_src_meta, true, (hipStream_t)stream);
}

ep_status ep_dispatch_noalloc(const ep_handle* h, uint32_t flags, const void* x, const float* topk_weights,
                              void* recv_x, float* recv_scales, float* recv_weights, int32_t* recv_src_meta,
                              void* stream) {
  ep_status st = check_handle(h);
  if (st == EP_OK) st = check_device(h);
  if (st != EP_OK) return st;
  float* staging = nullptr;
  if ((flags & EP_DISPATCH_FP8) && (flags & EP_DISPATCH_SCALES_COL_MAJOR) && h->cfg.hidden % 128 == 0) {
    const int64_t need = h->T * (h->cfg.hidden / 128) * (int64_t)sizeof(float);
    if (need > (int64_t)EP_NOALLOC_SCRATCH_BYTES)
      return fail(EP_ERR_OVERFLOW,
                  "ep_dispatch_noalloc stages T * H/128 fp32 scales (%lld bytes), beyond its fixed %lld-byte array",
                  (long long)need, (long long)EP_NOALLOC_SCRATCH_BYTES);
    if (st = noalloc_scratch(h->device, &staging); st != EP_OK) return st;
  }
  return dispatch_common(h, flags, x, nullptr, false, topk_weights, recv_x, recv_scales, recv_weights,
                         recv_src_meta, true, (hipStream_t)stream, staging);
}

ep_status ep_dispatch_cached(const ep_handle* h, uint32_t flags, const void* x, void* recv_x,
                             float* recv_scales, void* stream) {
  return dispatch_common(h, flags, x, nullptr, false, nullptr, recv_x, recv_scales, nullptr, nullptr, false,
                         (hipStream_t)stream);
}

ep_status ep_dispatch_prequant(const ep_handle* h, uint32_t flags, const uint8_t* x_codes, const float* x_scales,
                               const float* topk_weights, void* recv_x, float* recv_scales, float* recv_weights,
                               int32_t* recv_src_meta, void* stream) {
  return dispatch_common(h, flags, x_codes, x_scales, true, topk_weights, recv_x, recv_scales, recv_weights,
                         recv_src_meta, true, (hipStream_t)stream);
}

ep_status ep_dispatch_prequant_cached(const ep_handle* h, uint32_t flags, const uint8_t* x_codes,
                                      const float* x_scales, void* recv_x, float* recv_scales, void* stream) {
  return dispatch_common(h, flags, x_codes, x_scales, true, nullptr, recv_x, recv_scales, nullptr, nullptr,
                         false, (hipStream_t)stream);
}

ep_status ep_combine(const ep_handle* h, const void* y, const float* topk_weights, const void* bias, void* out,
                     void* stream) {
  ep_status st = check_handle(h);
  if (st == EP_OK) st = check_device(h);
  if (st != EP_OK) return st;
  if (h->T == 0) return EP_OK;
  if (!out) return fail(EP_ERR_NULL, "out is NULL");
  if (h->total_rows > 0 && !y) return fail(EP_ERR_NULL, "y is NULL");
  if (misaligned(y, 16) || misaligned(out, 16) || misaligned(bias, 16) || misaligned(topk_weights, 4))
    return fail(EP_ERR_SHAPE, "y / bias / out must be 16-byte aligned, topk_weights 4-byte aligned");
  CombineArgs a{(const uint16_t*)y, topk_weights, h->dst_row, (const uint16_t*)bias, (uint16_t*)out,
                (int)h->T, h->dims.K, h->cfg.hidden, 1};
  return launch_combine(a, (hipStream_t)stream);
}

void ep_handle_free(ep_handle* h) { release(h); }

ep_status ep_handle_config(const ep_handle* h, ep_config* cfg) {
  if (!h || !cfg) return fail(EP_ERR_NULL, "NULL argument");
  *cfg = h->cfg;
  return EP_OK;
}

ep_status ep_handle_check(const ep_handle* h, const ep_config* cfg) {
  if (!h || !cfg) return fail(EP_ERR_NULL, "NULL argument");
  const ep_config& a = h->cfg;
  if (a.num_ranks != cfg->num_ranks || a.num_tokens != cfg->num_tokens || a.hidden != cfg->hidden ||
      a.num_topk != cfg->num_topk || a.num_experts != cfg->num_experts ||
      a.expert_alignment != cfg->expert_alignment || a.flags != cfg->flags ||
      a.num_worst_rows != cfg->num_worst_rows)
    return fail(EP_ERR_HANDLE_MISMATCH,
                "handle built for P=%d S=%d H=%d K=%d E=%d A=%d flags=%u W=%d, got P=%d S=%d H=%d K=%d E=%d A=%d "
                "flags=%u W=%d",
                a.num_ranks, a.num_tokens, a.hidden, a.num_topk, a.num_experts, a.expert_alignment, a.flags,
                a.num_worst_rows, cfg->num_ranks, cfg->num_tokens, cfg->hidden, cfg->num_topk, cfg->num_experts,
                cfg->expert_alignment, cfg->flags, cfg->num_worst_rows);
  return EP_OK;
}

ep_status ep_handle_counts(const ep_handle* h, int64_t* num_expanded, int64_t* num_recv_tokens,
                           int64_t* window_row_base) {
  ep_status st = check_handle(h);
  if (st == EP_OK) st = ensure_counts(h);
  if (st != EP_OK) return st;
  const int P = h->dims.P;
  const int64_t* sm = h->summary_host + kSummaryHeader;
  if (num_expanded) memcpy(num_expanded, sm, P * 8);
  if (num_recv_tokens) memcpy(num_recv_tokens, sm + P, P * 8);
  if (window_row_base) memcpy(window_row_base, sm + 2 * P, (P + 1) * 8);
  return EP_OK;
}

ep_status ep_handle_status(const ep_handle* h, uint32_t* flags, int64_t* dropped_rows) {
  if (!flags) return fail(EP_ERR_NULL, "flags is NULL");
  ep_status st = check_handle(h);
  if (st == EP_OK) st = ensure_counts(h);
  if (st != EP_OK) return st;
  *flags = h->status;
  if (dropped_rows) *dropped_rows = h->dropped;
  return EP_OK;
}

ep_status ep_handle_tensor(const ep_handle* h, int32_t which, const void** dev_ptr, int64_t* numel,
                           int32_t* elem_bytes) {
  ep_status st = check_handle(h);
  if (st != EP_OK) return st;
  if (!dev_ptr || !numel || !elem_bytes) return fail(EP_ERR_NULL, "NULL argument");
  const int64_t T = h->T, P = h->dims.P, E = h->dims.E, K = h->dims.K, El = h->dims.El;
  const void* p = nullptr;
  int64_t n = 0;
  int32_t b = 4;
  switch (which) {
    case EP_T_IS_TOKEN_IN_RANK: p = h->is_token_in_rank; n = T * P; b = 1; break;
    case EP_T_NUM_TOKENS_PER_RANK: p = h->num_tokens_per_rank; n = P * P; break;
    case EP_T_NUM_TOKENS_PER_EXPERT: p = h->num_tokens_per_expert; n = P * E; break;
    case EP_T_RANK_PREFIX_MATRIX: p = h->rank_prefix_matrix; n = P * P; break;
    case EP_T_NUM_RECV_TOKENS: p = h->num_recv; n = P; break;
    case EP_T_NUM_TOKENS_PER_EXPERT_TOTAL: p = h->n_e; n = E; break;
    case EP_T_EXPERT_OFFSET: p = h->expert_offset; n = P * (El + 1); b = 8; break;
    case EP_T_NUM_EXPANDED: p = h->num_expanded; n = P; b = 8; break;
    case EP_T_WINDOW_ROW_BASE: p = h->window_row_base; n = P + 1; b = 8; break;
    case EP_T_DST_SLOT: p = h->dst_slot; n = T * K; break;
    case EP_T_SEND_HEAD: p = h->send_head; n = T * P; break;
    case EP_T_RECV_SRC_IDX:
      st = ensure_counts(h);
      if (st != EP_OK) return st;
      p = h->recv_src_idx;
      n = h->sum_recv;
      break;
    case EP_T_RECV_SRC_BASE: p = h->recv_src_base; n = P + 1; b = 8; break;
    case EP_T_DST_ROW: p = h->dst_row; n = T * K; break;
    default: return fail(EP_ERR_SHAPE, "unknown tensor id %d", which);
  }
  *dev_ptr = p;
  *numel = n;
  *elem_bytes = b;
  return EP_OK;
}

ep_status ep_debug_copy(void* dst, const void* src, int64_t nbytes, void* stream) {
  if (nbytes < 0 || nbytes % 1024 != 0) return fail(EP_ERR_SHAPE, "nbytes must be a non-negative multiple of 1024");
  if (nbytes == 0) return EP_OK;
  if (!dst || !src) return fail(EP_ERR_NULL, "NULL argument");
  if (misaligned(dst, 16) || misaligned(src, 16)) return fail(EP_ERR_SHAPE, "dst / src must be 16-byte aligned");
  const int64_t waves = nbytes / 1024;
  if (waves >= ((int64_t)1 << 31) / kWave) return fail(EP_ERR_OVERFLOW, "nbytes too large");
  const int blocks = (int)((waves + 3) / 4);
  copy_kernel<<<blocks, 256, 0, (hipStream_t)stream>>>((u32x4*)dst, (const u32x4*)src, waves);
  EP_LAUNCHED("copy_kernel");
  return EP_OK;
}

ep_status ep_debug_e4m3_encode(const float* in, uint8_t* out, int64_t n, void* stream) {
  if (n < 0) return fail(EP_ERR_SHAPE, "n < 0");
  if (n == 0) return EP_OK;
  if (!in || !out) return fail(EP_ERR_NULL, "NULL argument");
  const int64_t threads = (n + 3) / 4;
  if ((threads + 255) / 256 >= ((int64_t)1 << 31)) return fail(EP_ERR_OVERFLOW, "n too large");
  e4m3_encode_kernel<<<(int)((threads + 255) / 256), 256, 0, (hipStream_t)stream>>>(in, out, n);
  EP_LAUNCHED("e4m3_encode_kernel");
  return EP_OK;
}

ep_status ep_debug_timing(uint64_t* slots, int64_t n) {
#if EP_DEVICE_TIMING
  if (!slots) return fail(EP_ERR_NULL, "slots is NULL");
  const int64_t all = (int64_t)kEpTimingKernels * kEpTimingPhases * kEpTimingGroups;
  if (n < 0 || n > all) return fail(EP_ERR_SHAPE, "n must be in [0, %lld]", (long long)all);
  EP_HIP(hipMemcpyFromSymbol(slots, HIP_SYMBOL(ep_timing_slots), (size_t)n * sizeof(uint64_t), 0,
                             hipMemcpyDeviceToHost));
  return EP_OK;
#else
  (void)slots;
  (void)n;
  return fail(EP_ERR_SHAPE, "the library was built without EP_DEVICE_TIMING");
#endif
}

const char* ep_last_error(void) { return g_last_error.c_str(); }

int32_t ep_abi_version(void) { return EP_ABI_VERSION; }

}  // extern "C"
