// Device helpers for the libfx kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "fx_plan.h"

namespace fx {

typedef uint16_t bf16_t;   // bfloat16 storage: the upper 16 bits of a float32

// ---- element conversions --------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float(uint32_t(x) << 16); }

// float32 -> bfloat16, round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return bf16_t((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return bf16_t(u >> 16);
}

__device__ __forceinline__ void store_elem(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_elem(bf16_t* p, float v) { *p = f32_to_bf16(v); }

// float64 -> bfloat16 with ONE rounding (to nearest, ties to even).  Rounding a
// float64 to float32 first and then to bfloat16 would round twice.  For normal
// bfloat16 results the float64 significand is cut to 7 fraction bits with the
// usual add-half-minus-one-plus-lsb carry; below 2^-126 the quantum is 2^-133 and
// the scaled value is rounded to an integer by v_rndne_f64.
__device__ __forceinline__ bf16_t f64_to_bf16_rne(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint16_t sign = uint16_t((u >> 48) & 0x8000u);
  uint64_t a = u & 0x7FFFFFFFFFFFFFFFull;
  if (a > 0x7FF0000000000000ull) return bf16_t(sign | 0x7FC0u);           // NaN
  if (a < 0x3810000000000000ull) {                                          // |x| < 2^-126
    double y = __builtin_rint(__longlong_as_double((long long)a) * 0x1p133);
    return bf16_t(sign | uint16_t(y));                                      // 0..128
  }
  const uint64_t drop = (1ull << 45) - 1;                                  // 52 - 7 fraction bits
  a += (drop >> 1) + ((a >> 45) & 1ull);
  a &= ~drop;
  if (a >= 0x47F0000000000000ull) return bf16_t(sign | 0x7F80u);           // >= 2^128: inf
  const float f = (float)__longlong_as_double((long long)a);               // exact
  return bf16_t(sign | uint16_t(__float_as_uint(f) >> 16));
}

__device__ __forceinline__ void store_from_f64(float* p, double v) { *p = (float)v; }
__device__ __forceinline__ void store_from_f64(bf16_t* p, double v) { *p = f64_to_bf16_rne(v); }

// Monotone uint32 key of a float32 (larger float -> larger key; -0 and +0 equal;
// NaN maps to 0, below every number; +-inf rank as the largest / smallest numbers).
// Any non-finite value sets *nonfinite.
__device__ __forceinline__ uint32_t f32_key(float f, bool* nonfinite) {
  if (f != f) { *nonfinite = true; return 0u; }
  if (__builtin_isinf(f)) *nonfinite = true;
  if (f == 0.0f) f = 0.0f;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---- raw buffer loads -----------------------------------------------------------------

// 128-bit raw buffer load with the nontemporal hint (for bytes read once per call);
// offsets at or past the resource's byte count read as zero without touching memory.
constexpr int kCachePolicyNT = 2;
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCachePolicyNT));
}
constexpr int kRsrcWord3 = 0x00020000;      // raw (untyped) buffer, gfx9-family descriptor
constexpr uint32_t kOutOfRange = 0x80000000u;

// ---- bounds of one unit ---------------------------------------------------------------

__device__ __forceinline__ int load_seq_len(const int32_t* seq_lens, int b, int t_cap,
                                            uint32_t* err) {
  int T = seq_lens[b];
  if (T < 0 || T > t_cap) {
    if (threadIdx.x == 0) atomicOr(err, (uint32_t)FX_ERR_SEQ_LEN);
    T = T < 0 ? 0 : t_cap;
  }
  return T;
}

// ---- cross-lane reductions ------------------------------------------------------------

// DPP controls (GFX9 encoding).
constexpr int kQuadPerm1032 = 0xB1;     // lanes {1,0,3,2} of each quad
constexpr int kQuadPerm2301 = 0x4E;     // lanes {2,3,0,1}
constexpr int kRowHalfMirror = 0x141;   // lane i <- 7 - i within each 8
constexpr int kRowMirror = 0x140;       // lane i <- 15 - i within each 16

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of LPT consecutive lanes (LPT = 4, 8, 16 or 32); every lane
// of a group ends with the group's sum.
template <int LPT>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LPT == 4 || LPT == 8 || LPT == 16 || LPT == 32, "group size");
  x += dpp_f<kQuadPerm1032>(x);
  x += dpp_f<kQuadPerm2301>(x);
  if constexpr (LPT >= 8) x += dpp_f<kRowHalfMirror>(x);
  if constexpr (LPT >= 16) x += dpp_f<kRowMirror>(x);
  if constexpr (LPT >= 32) x += __shfl_xor(x, 16);
  return x;
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, true);
}

__device__ __forceinline__ uint32_t lane_value(uint32_t x, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)x, lane);
}

// Minimum / maximum / sum over the 64 lanes of a wave (wave-uniform result).  The
// quad permutes and the two mirrors leave every row of 16 lanes holding its row's
// value; the four rows are then combined from lanes 0, 16, 32 and 48.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  x = min(x, dpp_u32<kQuadPerm1032>(x));
  x = min(x, dpp_u32<kQuadPerm2301>(x));
  x = min(x, dpp_u32<kRowHalfMirror>(x));
  x = min(x, dpp_u32<kRowMirror>(x));
  return min(min(lane_value(x, 0), lane_value(x, 16)), min(lane_value(x, 32), lane_value(x, 48)));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, dpp_u32<kQuadPerm1032>(x));
  x = max(x, dpp_u32<kQuadPerm2301>(x));
  x = max(x, dpp_u32<kRowHalfMirror>(x));
  x = max(x, dpp_u32<kRowMirror>(x));
  return max(max(lane_value(x, 0), lane_value(x, 16)), max(lane_value(x, 32), lane_value(x, 48)));
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
  x += dpp_u32<kQuadPerm1032>(x);
  x += dpp_u32<kQuadPerm2301>(x);
  x += dpp_u32<kRowHalfMirror>(x);
  x += dpp_u32<kRowMirror>(x);
  return (lane_value(x, 0) + lane_value(x, 16)) + (lane_value(x, 32) + lane_value(x, 48));
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4 and 8 inside
// each row of 16 lanes (lanes shifted in from outside the row read 0), then the row
// totals of lanes 15, 31 and 47 are added to the rows above them.
__device__ __forceinline__ uint32_t wave_scan_incl_u32(uint32_t x) {
  constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
  x += dpp_u32<kRowShr1>(x);
  x += dpp_u32<kRowShr2>(x);
  x += dpp_u32<kRowShr4>(x);
  x += dpp_u32<kRowShr8>(x);
  const int lane = threadIdx.x & 63;
  const uint32_t r0 = lane_value(x, 15), r1 = lane_value(x, 31), r2 = lane_value(x, 47);
  x += (lane >= 16 ? r0 : 0u) + (lane >= 32 ? r1 : 0u) + (lane >= 48 ? r2 : 0u);
  return x;
}

// Number of set bits of a wave ballot below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t ballot) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(ballot >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)ballot, 0u));
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// Exclusive prefix sum over a workgroup of NT threads (multiple of 64).  `lds` holds
// NT/64 ints.  Returns the exclusive prefix; *total receives the sum over the group.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int x, int* lds, int* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int incl = wave_inclusive_scan(x);
  if (lane == 63) lds[w] = incl;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int v = lds[i];
    off += (i < w) ? v : 0;
    tot += v;
  }
  __syncthreads();
  *total = tot;
  return off + incl - x;
}

template <int NT>
__device__ __forceinline__ int block_sum(int x, int* lds) {
  int total;
  (void)block_exclusive_scan<NT>(x, lds, &total);
  return total;
}

}  // namespace fx
