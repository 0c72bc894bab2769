// Key-side block scores of 64 consecutive summary rows, one row per lane of a wave.
//
// [NOSA-DE] "Technisches Resümee: NOSA: Native und Offloadable Sparse Attention",
// Methodik §1 "Query-Aware Selection"; [Fluxion-NL] "Technische Samenvatting: Fluxion",
// Systeemcomponenten, "Granularity-Budget Selector" (one score per GQA group).
//
// The score of a summary row S_j is the float32 rounding of the float64 chain
//   acc = ((0 + qs[0]*S_j[0]) + qs[1]*S_j[1]) + ... + qs[d-1]*S_j[d-1]
// with every product and sum rounded to float64 on its own (contraction off), qs being
// the float64 sum of the group's query rows taken in row order.  k_score (the separate
// scoring kernel) evaluates the same chain in the same order, so both give the same bits.
//
// A wave requests its whole tile (64 rows) at once through a buffer resource bounded to
// the unit's rows (rows past the end read zero), then passes it through its own LDS tile
// in column chunks of 32 words with an odd row stride (33 words: lane i reading word c
// of row i never shares a bank with another lane), continuing its row's chain chunk by
// chunk.  The staging tile belongs to one wave, so only wave-level ordering is needed.
#pragma once

#include "fx_device.h"

namespace fx {

__device__ __forceinline__ double elem_f64(const uint32_t* row, int c, float*) {
  return (double)__uint_as_float(row[c]);
}
__device__ __forceinline__ double elem_f64(const uint32_t* row, int c, bf16_t*) {
  const uint32_t w = row[c >> 1];
  return (double)((c & 1) ? bf16_hi(w) : bf16_lo(w));
}

constexpr int kScoreTile = 64;         // summary rows per wave tile (one per lane)
constexpr int kScoreChunkWords = 32;   // row words staged in LDS at a time

typedef uint32_t ScoreStage[kScoreTile][kScoreChunkWords + 1];

// qs[c] = ((q_0[c] + q_1[c]) + ...) + q_{G-1}[c] in float64 for the G query rows at
// qgroup (16-byte aligned, rows D elements apart): the threads load the G * D * sizeof(E)
// / 16 16-byte pieces into `rows` (all in flight together), then sum a column each.
// Every thread of the workgroup calls this; qs is ready after the caller's next barrier.
template <typename E, int D>
__device__ __forceinline__ void group_sum_f64(const E* qgroup, int G, uint4* rows, double* qs) {
  constexpr int QV4 = D * (int)sizeof(E) / 16;
  for (int t = threadIdx.x; t < G * QV4; t += blockDim.x)
    rows[t] = reinterpret_cast<const uint4*>(qgroup)[t];
  __syncthreads();
  const E* qe = reinterpret_cast<const E*>(rows);
  for (int t = threadIdx.x; t < D; t += blockDim.x) {
    double a = (double)to_f32(qe[t]);
    for (int g = 1; g < G; ++g) a = a + (double)to_f32(qe[g * D + t]);
    qs[t] = a;
  }
}

// LDS written by the lanes of a wave is read by other lanes of the same wave: the
// wave's LDS operations complete in order, and the fences keep the compiler from
// moving the reads above the writes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename E, int D>
struct ScoreTile {
  static constexpr int ROW_BYTES = D * (int)sizeof(E);
  static constexpr int WORDS = ROW_BYTES / 4;                    // 32-bit words per row
  static constexpr int NCH = WORDS / kScoreChunkWords;            // column chunks per row
  static constexpr int CPIECES = kScoreChunkWords / 4;            // 16-byte pieces per row chunk
  static constexpr int PER_LANE = kScoreTile * CPIECES / 64;      // pieces per lane per chunk
  static constexpr int CCOLS = kScoreChunkWords * 4 / (int)sizeof(E);   // columns per chunk
  static_assert(WORDS % kScoreChunkWords == 0, "row chunks");
  uint4 buf[NCH][PER_LANE];

  // Requests rows [j0, j0 + 64) (piece m = lane + 64k of chunk ch is row m / CPIECES,
  // 16-byte piece ch * CPIECES + m % CPIECES).
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int j0, int lane) {
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
      for (int k = 0; k < PER_LANE; ++k) {
        const int m = lane + 64 * k;
        const uint32_t row = (uint32_t)(j0 + m / CPIECES);
        buf[ch][k] = buffer_load16(rs, row * (uint32_t)ROW_BYTES +
                                           (uint32_t)((ch * CPIECES + m % CPIECES) * 16));
      }
  }

  // The float64 chain of row j0 + lane against qs (D doubles in LDS).  BLOCK: every
  // wave of the workgroup calls this together and the staging steps use workgroup
  // barriers; else only wave-level ordering.
  template <bool BLOCK = false>
  __device__ __forceinline__ double chain(const double* qs, ScoreStage& stage, int lane) const {
    double acc = 0.0;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
      for (int k = 0; k < PER_LANE; ++k) {
        const int m = lane + 64 * k;
        uint32_t* dst = &stage[m / CPIECES][(m % CPIECES) * 4];
        dst[0] = buf[ch][k].x;
        dst[1] = buf[ch][k].y;
        dst[2] = buf[ch][k].z;
        dst[3] = buf[ch][k].w;
      }
      if constexpr (BLOCK) __syncthreads();
      else wave_lds_sync();
      const uint32_t* row = stage[lane];
      {
#pragma clang fp contract(off)
#pragma unroll 16
        for (int c = 0; c < CCOLS; ++c) {
          const double x = elem_f64(row, c, (E*)nullptr);
          const double prod = qs[ch * CCOLS + c] * x;
          acc = acc + prod;
        }
      }
      if constexpr (BLOCK) __syncthreads();   // the next chunk overwrites the tile
      else wave_lds_sync();
    }
    return acc;
  }
};

}  // namespace fx
