// Block scores against each GQA query group.
//
// [NOSA-DE] "Technisches Resümee: NOSA: Native und Offloadable Sparse Attention",
// Methodik §1: "Query-Aware Selection" (the query decides which blocks to fetch) and
// "ED-DMA" (selection uses pre-exponential values).  [Fluxion-NL] "Technische
// Samenvatting: Fluxion", Systeemcomponenten, "Granularity-Budget Selector": GQA is
// handled per query group, so one score per (kv head, block) serves the whole group.
//
// Score of full block j of unit u, a float32 value defined by this float64 evaluation:
//   qs[c] = ((q_0[c] + q_1[c]) + ...) + q_{G-1}[c]
//   acc   = ((0 + qs[0]*S_j[0]) + qs[1]*S_j[1]) + ... + qs[d-1]*S_j[d-1]
//   score = (float)acc           (round to nearest, ties to even)
// with every product and every sum rounded to float64 on its own (fp contraction is
// off below).  This is the group's sum of raw dot products with the summary; the fixed
// order makes the float32 value, and hence the selection, reproducible bit for bit.
//
// Mapping: one wave per tile of 64 blocks of one unit.  qs goes to LDS once per
// workgroup; the tile's summary rows are staged into LDS with 16-byte loads (row
// stride WORDS+1 words, so lane i reading word c of row i hits bank (i + c) mod 64);
// then lane i runs block j0 + i's d-term chain in order.  Each lane issues all of its
// staging loads before writing any of them, so a tile costs one memory round trip.
#include "fx_device.h"

namespace fx {
namespace {

__device__ __forceinline__ double elem_f64(const uint32_t* row, int c, float*) {
  return (double)__uint_as_float(row[c]);
}
__device__ __forceinline__ double elem_f64(const uint32_t* row, int c, bf16_t*) {
  const uint32_t w = row[c >> 1];
  return (double)((c & 1) ? bf16_hi(w) : bf16_lo(w));
}

constexpr int kTile = 64;

template <typename E, int D>
__global__ __launch_bounds__(64) void k_score(
    const UnitInfo* __restrict__ units, const E* __restrict__ q, const E* __restrict__ S,
    const int32_t* __restrict__ seq_lens, float* __restrict__ scores, uint32_t* __restrict__ err,
    int Hkv, int G, int t_cap, int tiles_per_unit) {
  constexpr int WORDS = D * (int)sizeof(E) / 4;
  const int u = blockIdx.x / tiles_per_unit;
  const int tile = blockIdx.x % tiles_per_unit;
  const UnitInfo ui = units[u];
  if (ui.mode == FX_STREAMING) return;
  const int b = u / Hkv, h = u % Hkv;
  const int T = load_seq_len(seq_lens, b, t_cap, err);
  const int n_full = T >> ui.log2g;
  const int j0 = tile * kTile;
  if (j0 >= n_full) return;
  const int nrows = min(kTile, n_full - j0);
  const int lane = threadIdx.x;

  __shared__ double qs[D];
  __shared__ uint32_t rows[kTile][WORDS + 1];

  const E* qg = q + ((size_t)b * Hkv * G + (size_t)h * G) * D;
  for (int c = lane; c < D; c += 64) {
    double a = (double)to_f32(qg[c]);
    for (int g = 1; g < G; ++g) a = a + (double)to_f32(qg[(size_t)g * D + c]);
    qs[c] = a;
  }
  // Stage the tile: every lane issues all of its 16-byte loads before the first LDS
  // write, so the tile costs one memory round trip.
  const uint4* src = reinterpret_cast<const uint4*>(S + ((size_t)ui.block_off + j0) * D);
  constexpr int V4 = WORDS / 4;                 // 16-byte vectors per row
  constexpr int PER_LANE = kTile * V4 / 64;
  const int nvec = nrows * V4;
  uint4 buf[PER_LANE];
#pragma unroll
  for (int k = 0; k < PER_LANE; ++k) {
    const int i = lane + k * 64;
    buf[k] = i < nvec ? src[i] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int k = 0; k < PER_LANE; ++k) {
    const int i = lane + k * 64;
    if (i < nvec) {
      const int r = i / V4, c = (i % V4) * 4;
      rows[r][c + 0] = buf[k].x;
      rows[r][c + 1] = buf[k].y;
      rows[r][c + 2] = buf[k].z;
      rows[r][c + 3] = buf[k].w;
    }
  }
  __syncthreads();
  if (lane >= nrows) return;

  const uint32_t* row = rows[lane];
  double acc = 0.0;
  {
#pragma clang fp contract(off)
#pragma unroll 16
    for (int c = 0; c < D; ++c) {
      const double prod = qs[c] * elem_f64(row, c, (E*)nullptr);
      acc = acc + prod;
    }
  }
  scores[(size_t)ui.block_off + j0 + lane] = (float)acc;
}

template <typename E, int D>
hipError_t launch_t(const fx_plan* p, const void* q, const void* S, const int32_t* seq_lens,
                    float* scores, hipStream_t stream) {
  const int tiles = (p->max_n_full_cap + kTile - 1) / kTile;
  if (tiles == 0) return hipSuccess;
  const dim3 grid((unsigned)((int64_t)tiles * p->units));
  k_score<E, D><<<grid, 64, 0, stream>>>(p->d_units, static_cast<const E*>(q),
                                         static_cast<const E*>(S), seq_lens, scores, p->d_error,
                                         p->desc.num_kv_heads, p->G, p->desc.t_cap, tiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score(const fx_plan* p, const void* q, const void* S, const int32_t* seq_lens,
                        float* scores, hipStream_t stream) {
  const int d = p->desc.head_dim;
  if (p->desc.dtype == FX_BF16)
    return d == 128 ? launch_t<bf16_t, 128>(p, q, S, seq_lens, scores, stream)
                    : launch_t<bf16_t, 64>(p, q, S, seq_lens, scores, stream);
  return d == 128 ? launch_t<float, 128>(p, q, S, seq_lens, scores, stream)
                  : launch_t<float, 64>(p, q, S, seq_lens, scores, stream);
}

}  // namespace fx
