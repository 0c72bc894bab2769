// Block summaries: two-stage pooling of key rows.
//
// [NOSA-DE] "Technisches Resümee: NOSA: Native und Offloadable Sparse Attention",
// Methodik §1, bullet "Blockweise Implementierung": selection scores come from a
// mean inside each sub-block followed by a max at block level.  Methodik §2, bullet
// "Kernel Fusion": the pooling runs inside one fused kernel.
//
// For full block j of a unit, column c:
//   S[j][c] = round_once( max over sub-blocks u of ( sum of the s rows of u )[c] / s )
// The row sums are accumulated in float64.  bfloat16 and float32 keys of the ranges
// used here sum exactly in float64, so the order of accumulation does not matter; the
// division by the power-of-two s is exact; the max is exact; the one rounding into the
// storage type is to nearest, ties to even (f64_to_bf16_rne / cvt_f32_f64).
//
// Score-side pooling (the block-level max taken later, over scores) keeps the means:
//   S[j*r + u][c] = round_once( ( sum of the s rows of u )[c] / s ),  r = g / s,
// written at the unit's summary rows instead of the max.
//
// Mapping: one 256-thread workgroup per (unit, block).  A key row is WORDS 32-bit
// words (d * sizeof(elem) / 4); thread (w, ph) owns word w and the sub-blocks
// u = ph, ph + PH, ...  Each wave reads whole rows (coalesced 4-byte lanes); the
// sub-block maxima of the PH phases meet in LDS (key side), or every thread stores
// its own means (score side).
#include "fx_device.h"

namespace fx {
namespace {

__device__ __forceinline__ int resolve_slice(int x, int n) {
  if (x < 0) {
    x += n;
    if (x < 0) x = 0;
  }
  return x > n ? n : x;
}

__device__ __forceinline__ void widen(uint32_t w, double* v, float*) { v[0] = (double)__uint_as_float(w); }
__device__ __forceinline__ void widen(uint32_t w, double* v, bf16_t*) {
  v[0] = (double)bf16_lo(w);
  v[1] = (double)bf16_hi(w);
}

template <typename E, int D>
__global__ __launch_bounds__(256) void k_build_summaries(
    const UnitInfo* __restrict__ units, const E* __restrict__ K,
    const int32_t* __restrict__ seq_lens, int32_t bb, int32_t be, E* __restrict__ S,
    uint32_t* __restrict__ err, int Hkv, int t_cap, int blocks_per_unit, bool score_side) {
  constexpr int WORDS = D * (int)sizeof(E) / 4;
  constexpr int EPW = 4 / (int)sizeof(E);
  constexpr int PH = 256 / WORDS;
  static_assert(PH >= 1 && 256 % WORDS == 0, "row words");

  const int u = blockIdx.x / blocks_per_unit;
  const int jr = blockIdx.x % blocks_per_unit;
  const UnitInfo ui = units[u];
  const int b = u / Hkv;
  const int T = load_seq_len(seq_lens, b, t_cap, err);
  const int n_full = T >> ui.log2g;
  const int j0 = resolve_slice(bb, n_full), j1 = resolve_slice(be, n_full);
  const int j = j0 + jr;
  if (j >= j1) return;

  const int w = threadIdx.x % WORDS, ph = threadIdx.x / WORDS;
  const int g = ui.g, s = ui.s, nsub = g / s;
  const double inv_s = 1.0 / (double)s;   // power of two: exact
  const uint32_t* rows =
      reinterpret_cast<const uint32_t*>(K + ((size_t)u * t_cap + (size_t)j * g) * D) + w;

  double mx[EPW];
#pragma unroll
  for (int e = 0; e < EPW; ++e) mx[e] = -__builtin_inf();
  for (int sb = ph; sb < nsub; sb += PH) {
    const uint32_t* p = rows + (size_t)sb * s * WORDS;
    double acc[EPW];
#pragma unroll
    for (int e = 0; e < EPW; ++e) acc[e] = 0.0;
#pragma unroll 16   // a sub-block of 16 rows in one round of loads (nosa_drift: 5.1 -> 4.5 us)
    for (int r = 0; r < s; ++r) {
      double v[EPW];
      widen(p[(size_t)r * WORDS], v, (E*)nullptr);
#pragma unroll
      for (int e = 0; e < EPW; ++e) acc[e] += v[e];
    }
    if (score_side) {
      E* dst = S + ((size_t)ui.sum_off + ((size_t)j << ui.log2r) + sb) * D + (size_t)w * EPW;
#pragma unroll
      for (int e = 0; e < EPW; ++e) store_from_f64(dst + e, acc[e] * inv_s);
      continue;
    }
#pragma unroll
    for (int e = 0; e < EPW; ++e) mx[e] = fmax(mx[e], acc[e] * inv_s);
  }
  if (score_side) return;   // uniform across the workgroup

  __shared__ double red[PH][WORDS * EPW];
#pragma unroll
  for (int e = 0; e < EPW; ++e) red[ph][w * EPW + e] = mx[e];
  __syncthreads();
  if (ph != 0) return;
#pragma unroll
  for (int e = 0; e < EPW; ++e) {
    double m = red[0][w * EPW + e];
    for (int i = 1; i < PH; ++i) m = fmax(m, red[i][w * EPW + e]);
    mx[e] = m;
  }
  E* dst = S + ((size_t)ui.sum_off + (size_t)j) * D + (size_t)w * EPW;
#pragma unroll
  for (int e = 0; e < EPW; ++e) store_from_f64(dst + e, mx[e]);
}

template <typename E, int D>
int launch_t(const fx_plan* p, const void* K, const int32_t* seq_lens, int32_t bb,
                    int32_t be, void* S, int blocks_per_unit, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)blocks_per_unit * p->units));
  k_build_summaries<E, D><<<grid, 256, 0, stream>>>(
      p->d_units, static_cast<const E*>(K), seq_lens, bb, be, static_cast<E*>(S), p->d_error,
      p->desc.num_kv_heads, p->desc.t_cap, blocks_per_unit, p->desc.pooling != FX_POOL_KEY);
  return hipGetLastError();
}

}  // namespace

int launch_build_summaries(const fx_plan* p, const void* K, const int32_t* seq_lens,
                                  int32_t bb, int32_t be, void* S, hipStream_t stream) {
  // Upper bound on the blocks any unit can have in [bb, be) once resolved.
  const int64_t n = p->max_n_full_cap;
  int64_t cnt;
  if (bb >= 0 && be >= 0) cnt = std::min<int64_t>(be, n) - bb;
  else if (bb < 0 && be >= 0) cnt = std::min<int64_t>(-(int64_t)bb, n);
  else if (bb < 0) cnt = (int64_t)be - bb;
  else cnt = n - bb;
  cnt = std::min<int64_t>(cnt, n);
  if (cnt <= 0) return hipSuccess;
  const int bpu = (int)cnt;
  const int d = p->desc.head_dim;
  if (p->desc.dtype == FX_BF16) {
    return d == 128 ? launch_t<bf16_t, 128>(p, K, seq_lens, bb, be, S, bpu, stream)
                    : launch_t<bf16_t, 64>(p, K, seq_lens, bb, be, S, bpu, stream);
  }
  return d == 128 ? launch_t<float, 128>(p, K, seq_lens, bb, be, S, bpu, stream)
                  : launch_t<float, 64>(p, K, seq_lens, bb, be, S, bpu, stream);
}

}  // namespace fx
