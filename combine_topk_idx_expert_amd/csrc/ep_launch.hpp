// ep_launch.hpp -- launch configuration of the dispatch and combine kernels.
//
// Part of ep_api.hip's translation unit: it is included there, inside the
// anonymous namespace, after the error helpers (fail, EP_LAUNCHED) it uses.
// Grid shapes, workgroup sizes and the column-part choices live here, apart
// from the API's validation code, so that they sit next to the kernels whose
// performance they set.
#pragma once

// Column part per wave, in 16-byte chunks per lane (tunable at build time;
// the defaults are the fastest of sweeps on MI355X at hidden 7168 and 4096:
// dispatch 1 KiB of bf16 input per wave for bf16 and fp8 output, combine
// 1 KiB per wave with all K <= 8 row loads in flight).
#ifndef EP_DISPATCH_NC_BF16
#define EP_DISPATCH_NC_BF16 1
#endif
#ifndef EP_DISPATCH_NC_FP8
#define EP_DISPATCH_NC_FP8 1
#endif
#ifndef EP_ROW_BLOCK_WAVES
#define EP_ROW_BLOCK_WAVES 4  // waves per workgroup of the dispatch kernel
#endif
#ifndef EP_COMBINE_BLOCK_WAVES
#define EP_COMBINE_BLOCK_WAVES 16  // waves per workgroup of the register combine kernel (1 and 16 measured ~1.5% faster than 4 and 8)
#endif
#ifndef EP_DISPATCH_LDS_BYTES
#define EP_DISPATCH_LDS_BYTES 0
#endif
#ifndef EP_COMBINE_NCT
#define EP_COMBINE_NCT 1
#endif
#ifndef EP_COMBINE_G
#define EP_COMBINE_G 8
#endif

// Column part per wave (16-byte chunks per lane) of the dispatch kernels: a
// build-time choice, NC KiB of bf16 input per wave.
constexpr int kNcBf16 = EP_DISPATCH_NC_BF16;
constexpr int kNcFp8 = EP_DISPATCH_NC_FP8;

// Largest instantiated chunk count <= want that the row still needs (combine).
int pick_nc(int H, int want) {
  const int need = ((H >> 3) + kWave - 1) / kWave;  // chunks per lane for the whole row
  const int nc = std::min(want, need);
  return nc >= 14 ? 14 : nc >= 8 ? 8 : nc >= 7 ? 7 : nc >= 4 ? 4 : nc >= 2 ? 2 : 1;
}

int parts_per_row(int H, int nc) { return ((H >> 3) + nc * kWave - 1) / (nc * kWave); }

// Fixed windows: waves that stride over the padding and tail rows (whole rows),
// whose number only the device knows (at most P * cap rows).
constexpr int64_t kZeroWaves = 16384;

template <bool FP8, bool META, bool PREQ, bool FIXED, bool UE8M0 = false>
ep_status launch_dispatch(DispatchArgs a, hipStream_t s) {
  constexpr int nc = FP8 ? kNcFp8 : kNcBf16;
  a.split = parts_per_row(a.H, nc);
  const int64_t out_rows = FIXED ? (int64_t)a.P * a.cap : (int64_t)a.sum_expanded;
  const int64_t meta_items = META ? (out_rows + kWave - 1) / kWave : 0;
  a.zero_waves = FIXED ? (int)std::min<int64_t>((int64_t)a.P * a.cap, kZeroWaves) : 0;
  const int64_t zero_items = FIXED ? a.zero_waves : (a.zero_pad ? (int64_t)a.total_pad * a.split : 0);
  const int64_t waves = (int64_t)a.T * a.split + zero_items + meta_items;
  if (waves >= ((int64_t)1 << 31) / kWave) return fail(EP_ERR_OVERFLOW, "dispatch grid too large (%lld waves)", (long long)waves);
  if (waves > 0) {
    const int threads = EP_ROW_BLOCK_WAVES * kWave;
    const int blocks = (int)((waves + EP_ROW_BLOCK_WAVES - 1) / EP_ROW_BLOCK_WAVES);
    const size_t lds = EP_DISPATCH_LDS_BYTES;  // > 0 caps workgroups per CU (occupancy)
    dispatch_kernel<nc, FP8, META, PREQ, FIXED, UE8M0><<<blocks, threads, lds, s>>>(a);
    EP_LAUNCHED("dispatch_kernel");
  }
  // row-major scales are written by the dispatch waves themselves
  if (FP8 && a.scales_cm && out_rows > 0) {
    if (out_rows >= ((int64_t)1 << 31)) return fail(EP_ERR_OVERFLOW, "scale grid too large");
    dispatch_scales_cm_kernel<<<(int)((out_rows + kCmRows - 1) / kCmRows), 256, 0, s>>>(a);
    EP_LAUNCHED("dispatch_scales_cm_kernel");
  }
  return EP_OK;
}

template <bool FP8, bool META, bool PREQ, bool UE8M0 = false>
ep_status launch_dispatch_mode(const DispatchArgs& a, hipStream_t s) {
  return a.cap > 0 ? launch_dispatch<FP8, META, PREQ, true, UE8M0>(a, s)
                   : launch_dispatch<FP8, META, PREQ, false, UE8M0>(a, s);
}

// Combine: whole rows of up to 8 KiB (K <= 8, so <= 64 KiB of LDS per token
// and two workgroups per CU) go through the LDS kernel, where every wave
// streams one slot's full row; measured faster than the register kernel at
// hidden 4096 and not at 7168, where a token's rows no longer fit twice per
// CU.  Everything else uses the register kernel, and so does a token count
// whose LDS grid (one 8-wave workgroup per token) would pass the 2^31
// work-item limit: the register kernel covers every shape, with its own
// guard.
ep_status launch_combine(CombineArgs a, hipStream_t s) {
  if (a.T <= 0) return EP_OK;
  constexpr int kLdsWaves = 8;
  const bool lds_grid_fits = (int64_t)a.T * kLdsWaves < ((int64_t)1 << 31) / kWave;
  if (a.K <= 8 && a.H <= 4096 && lds_grid_fits) {
    const int need = ((a.H >> 3) + kWave - 1) / kWave;  // chunks per lane for a whole row
    const size_t lds_row = (size_t)a.K * kWave * 16;     // per chunk per lane
    a.split = 1;
    const int grid = a.T;
    if (need <= 1)
      combine_lds_kernel<1><<<grid, kLdsWaves * kWave, lds_row * 1, s>>>(a);
    else if (need <= 2)
      combine_lds_kernel<2><<<grid, kLdsWaves * kWave, lds_row * 2, s>>>(a);
    else if (need <= 4)
      combine_lds_kernel<4><<<grid, kLdsWaves * kWave, lds_row * 4, s>>>(a);
    else
      combine_lds_kernel<8><<<grid, kLdsWaves * kWave, lds_row * 8, s>>>(a);
    EP_LAUNCHED("combine_lds_kernel");
    return EP_OK;
  }
  const int nct = std::min(pick_nc(a.H, EP_COMBINE_NCT), 4);
  a.split = parts_per_row(a.H, nct);
  const int64_t waves = (int64_t)a.T * a.split;
  if (waves >= ((int64_t)1 << 31) / kWave) return fail(EP_ERR_OVERFLOW, "combine grid too large (%lld waves)", (long long)waves);
  const int threads = EP_COMBINE_BLOCK_WAVES * kWave;
  const int blocks = (int)((waves + EP_COMBINE_BLOCK_WAVES - 1) / EP_COMBINE_BLOCK_WAVES);
  switch (nct) {
    case 1: combine_kernel<1, EP_COMBINE_G><<<blocks, threads, 0, s>>>(a); break;
    case 2: combine_kernel<2, EP_COMBINE_G><<<blocks, threads, 0, s>>>(a); break;
    default: combine_kernel<4, EP_COMBINE_G><<<blocks, threads, 0, s>>>(a); break;
  }
  EP_LAUNCHED("combine_kernel");
  return EP_OK;
}
