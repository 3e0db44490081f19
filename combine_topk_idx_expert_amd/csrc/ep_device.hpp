// ep_device.hpp -- wave64 helpers shared by the gfx950 kernels of the
// MoE dispatch / combine library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Device-side timing slots (compile-time switch, off by default): with
// EP_DEVICE_TIMING=1 every kernel stamps the device's constant-rate clock
// (wall_clock64, 100 MHz on MI355X) at its phase boundaries, one slot per
// (kernel, phase, workgroup) for the first kEpTimingGroups workgroups, so a
// profile can split a kernel's time into its steps without a profiler.  Off,
// the marks compile to nothing.
#ifndef EP_DEVICE_TIMING
#define EP_DEVICE_TIMING 0
#endif
constexpr int kEpTimingKernels = 8;   // kernel ids, see EP_TK_*
constexpr int kEpTimingPhases = 8;
constexpr int kEpTimingGroups = 1024;
enum { EP_TK_COUNT = 0, EP_TK_SCAN, EP_TK_FINALIZE, EP_TK_RANK, EP_TK_SMALL, EP_TK_DISPATCH, EP_TK_COMBINE };
#if EP_DEVICE_TIMING
__device__ uint64_t ep_timing_slots[kEpTimingKernels * kEpTimingPhases * kEpTimingGroups];
#define EP_TIMING_MARK(kernel, phase)                                                                    \
  do {                                                                                                   \
    if (threadIdx.x == 0 && blockIdx.x < (unsigned)kEpTimingGroups)                                      \
      ::ep_timing_slots[((kernel) * kEpTimingPhases + (phase)) * kEpTimingGroups + blockIdx.x] =        \
          (uint64_t)wall_clock64();                                                                      \
  } while (0)
#else
#define EP_TIMING_MARK(kernel, phase) \
  do {                                \
  } while (0)
#endif

namespace ep {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() {
  return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// Number of set bits of m in lanes below the calling lane.
__device__ __forceinline__ int count_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Lanes holding the same key as the calling lane.  gfx950 has no match
// instruction, so the key is compared bit by bit with one ballot per bit.
// Every lane of the wave must execute this (uniform control flow).
__device__ __forceinline__ uint64_t match_any(uint32_t key, int bits) {
  uint64_t peers = ballot(true);
  for (int b = 0; b < bits; ++b) {
    const bool bit = (key >> b) & 1u;
    const uint64_t m = ballot(bit);
    peers &= bit ? m : ~m;
  }
  return peers;
}

// Bits needed to represent values 0..n.
__host__ __device__ inline int bits_for(uint32_t n) {
  int b = 1;
  while ((1u << b) <= n) ++b;
  return b;
}

template <typename T>
__device__ __forceinline__ T uniform(T v) {
  return (T)__builtin_amdgcn_readfirstlane((int)v);
}

// Maximum over the 16 lanes of a DPP row (rotations by 8, 4, 2, 1 within the
// row), on the bit patterns of non-negative floats, which order like unsigned
// integers.
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xF, 0xF, false));
  return v;
}

// Maximum over each group of 4 lanes (DPP quad permutes: swap neighbours,
// then swap pairs), on non-negative float bit patterns.
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
  return v;
}

// bf16 pair in a 32-bit word -> two floats (bf16 is the upper half of fp32).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 a = (__bf16)lo;
  const __bf16 b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// float -> OCP FP8 E4M3FN code (bias 7, 3 mantissa bits, no infinity, 0x7F NaN,
// max finite 448), round to nearest, ties to even.  Magnitudes that round past
// 448 (above 464), infinities and NaN give 0x7F (with the sign).
//  - normal range (|q| >= 2^-6): round the fp32 pattern to 3 mantissa bits
//    (the carry runs into the exponent), then rebias the exponent 127 -> 7;
//  - below 2^-6 the code is the subnormal multiple round(|q| * 2^9), 0..8
//    (8 being the smallest normal's code).
__device__ __forceinline__ uint32_t e4m3_rne(float q) {
  const uint32_t b = __float_as_uint(q);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t a = b & 0x7FFFFFFFu;
  uint32_t nrm = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
  nrm = nrm > 0x7Eu ? 0x7Fu : nrm;
  // (clamped so the unused value stays in range when |q| is large)
  const uint32_t sub = (uint32_t)__builtin_rintf(fminf(__uint_as_float(a) * 512.0f, 8.0f));
  return sign | (a >= 0x3C800000u ? nrm : sub);
}

// The same encoding with gfx950's v_cvt_pk_fp8_f32 (OCP E4M3FN, round to
// nearest even), two values per instruction.  An exhaustive comparison with
// e4m3_rne over every fp32 pattern of magnitude <= 464 found no difference;
// larger magnitudes (never produced by x / (amax / 448)) are not used.
__device__ __forceinline__ uint32_t e4m3x4_hw(float q0, float q1, float q2, float q3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, w, true);
  return (uint32_t)w;
}

}  // namespace ep
