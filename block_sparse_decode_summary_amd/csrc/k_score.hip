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
// Score-side pooling (the block max taken over scores): the block has r summary rows
// M_u (its sub-block means), and
//   group sum: score = (float) max over u of acc(qs, M_u)
//   group max: score = (float) max over u and g of acc(q_g, M_u)
// acc being the chain above with the given vector.  Rounding is monotone, so each row's
// value is rounded first and the max is taken over floats.  A lane scores one row; the
// r rows of a block are r adjacent lanes (r divides 64), whose max is a butterfly.
//
// Mapping: the grid covers only retrieval and NOSA units (a host-built list); one
// 256-thread workgroup takes four consecutive 64-row tiles of a unit's summary rows,
// one tile per wave and one row per lane, and forms the float64 group sum qs (or the
// G float64 query rows, for the group max) once for all four.
// The unit index varies fastest along the grid: workgroup i runs on XCD i mod 8, so
// this spreads the first tile groups (present for every unit) over all eight XCDs
// instead of stacking them on one.
// Each wave requests its whole tile at once through a buffer resource bounded to the
// rows of the unit's full blocks (rows past the end read as zero without a memory access), in
// column-chunk order: chunk ch holds columns [ch*C, ch*C + C) of all 64 rows, C being
// 32 words, and one load instruction covers eight 128-byte row segments.  The chunks
// then pass one at a time through a per-wave LDS tile with stride 33 words (33 is odd,
// so lane i reading word c of row i never shares a bank with another lane), and the
// lane's chain continues across the chunks in column order.  Small LDS per workgroup
// keeps several workgroups, and their loads, resident on each CU.
#include <atomic>

#include "fx_score_tile.h"

namespace fx {
namespace {

constexpr int kTile = 64;         // summary rows per tile (one per lane)
constexpr int kWaves = 4;         // tiles per workgroup (one per wave)
constexpr int kChunkWords = 32;   // row words staged in LDS at a time

// NaN-propagating max (a NaN score is flagged later by the selection).
__device__ __forceinline__ double max_nan(double a, double b) { return (a != a || a >= b) ? a : b; }
__device__ __forceinline__ float max_nan(float a, float b) { return (a != a || a >= b) ? a : b; }

// The group-max score (score-side pooling with FX_POOL_SCORE_MAX): G = GM query rows,
// each with its own chain, aggregated by a max.
template <typename E, int D, int GM>
__global__ __launch_bounds__(kWaves * 64) void k_score_max(
    const UnitInfo* __restrict__ units, const int32_t* __restrict__ scored,
    const E* __restrict__ q, const E* __restrict__ S, const int32_t* __restrict__ seq_lens,
    float* __restrict__ scores, uint32_t* __restrict__ err, int Hkv, int G, int t_cap,
    int quads_per_unit) {
  constexpr int ROW_BYTES = D * (int)sizeof(E);
  constexpr int WORDS = ROW_BYTES / 4;                    // 32-bit words per summary row
  constexpr int NCH = WORDS / kChunkWords;                 // column chunks per row
  constexpr int CPIECES = kChunkWords / 4;                 // 16-byte pieces per row chunk
  constexpr int PER_LANE = kTile * CPIECES / 64;           // pieces per lane per chunk
  constexpr int CCOLS = kChunkWords * 4 / (int)sizeof(E);  // columns per chunk
  constexpr int QV4 = ROW_BYTES / 16;                      // 16-byte pieces per query row
  static_assert(WORDS % kChunkWords == 0, "row chunks");
  const int n_su = gridDim.x / quads_per_unit;
  const int quad = blockIdx.x / n_su;
  const int su = blockIdx.x % n_su;
  const int u = scored[su];
  const UnitInfo ui = units[u];
  const int b = u / Hkv, h = u % Hkv;
  const int T = load_seq_len(seq_lens, b, t_cap, err);
  const int n_full = T >> ui.log2g;
  const int log2r = ui.log2r;
  const int n_rows = n_full << log2r;
  const int tile0 = quad * kWaves;
  if (tile0 * kTile >= n_rows) return;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j0 = (tile0 + w) * kTile;

  __shared__ uint32_t rows[kWaves][kTile][kChunkWords + 1];
  __shared__ uint4 qrows[kMaxGroup * QV4];
  static_assert(GM >= 1 && GM <= kMaxGroup, "group rows");
  constexpr int NV = GM;                        // query vectors of the chains
  __shared__ double qs[NV * D];

  // The whole tile, chunk by chunk: piece m = lane + 64k of chunk ch is row m / CPIECES,
  // 16-byte piece ch*CPIECES + m % CPIECES.
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(S + (size_t)ui.sum_off * D), 0, n_rows * ROW_BYTES, kRsrcWord3);
  uint4 buf[NCH][PER_LANE];
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
    for (int k = 0; k < PER_LANE; ++k) {
      const int m = lane + 64 * k;
      const uint32_t row = (uint32_t)(j0 + m / CPIECES);
      buf[ch][k] = buffer_load16(rs, row * (uint32_t)ROW_BYTES +
                                         (uint32_t)((ch * CPIECES + m % CPIECES) * 16));
    }
  const uint4* qsrc = reinterpret_cast<const uint4*>(q + ((size_t)b * Hkv * G + (size_t)h * G) * D);
  const int nq = G * QV4;
  uint4 qv = make_uint4(0, 0, 0, 0);
  if ((int)threadIdx.x < nq) qv = qsrc[threadIdx.x];
  if ((int)threadIdx.x < nq) qrows[threadIdx.x] = qv;
  __syncthreads();
  const E* qe = reinterpret_cast<const E*>(qrows);
  if ((int)threadIdx.x < D) {
    const int c = threadIdx.x;
#pragma unroll
    for (int g = 0; g < GM; ++g) qs[g * D + c] = (double)to_f32(qe[g * D + c]);
  }

  double acc[NV];
#pragma unroll
  for (int g = 0; g < NV; ++g) acc[g] = 0.0;
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
    for (int k = 0; k < PER_LANE; ++k) {
      const int m = lane + 64 * k;
      uint32_t* dst = &rows[w][m / CPIECES][(m % CPIECES) * 4];
      dst[0] = buf[ch][k].x;
      dst[1] = buf[ch][k].y;
      dst[2] = buf[ch][k].z;
      dst[3] = buf[ch][k].w;
    }
    __syncthreads();
    const uint32_t* row = rows[w][lane];
    {
#pragma clang fp contract(off)
#pragma unroll 16
      for (int c = 0; c < CCOLS; ++c) {
        const double x = elem_f64(row, c, (E*)nullptr);
#pragma unroll
        for (int g = 0; g < NV; ++g) {
          const double prod = qs[g * D + ch * CCOLS + c] * x;
          acc[g] = acc[g] + prod;
        }
      }
    }
    __syncthreads();
  }
  double v = acc[0];
#pragma unroll
  for (int g = 1; g < NV; ++g) v = max_nan(v, acc[g]);
  float f = (float)v;
  for (int off = 1; off < (1 << log2r); off <<= 1) f = max_nan(f, __shfl_xor(f, off));
  const int row = j0 + lane;
  if ((lane & ((1 << log2r) - 1)) == 0 && row < n_rows)
    scores[(size_t)ui.block_off + (row >> log2r)] = f;
}

// The group-sum score (key-side summaries, or score-side pooling with the group summed):
// the float64 chain of fx_score_tile.h, which the selection kernel that forms its own
// scores shares, so both give the same bits.  A workgroup takes NW consecutive tiles of
// one unit, one per wave; the staging steps use workgroup barriers (measured faster here
// than per-wave ordering, and than two tiles per wave with the next one in flight).
// NW = 4 shares the query group sum among four tiles.  When the four-tile grid is larger
// than what the GPU holds at once, NW = 1: one-tile workgroups need a quarter of the LDS,
// so nearly all tiles are resident from the start instead of the last ones waiting for
// a slot (mixed_serving, 2560 four-tile workgroups: 20.9 against 21.7 us; qwen7b_layer,
// 512 of them, stays at four tiles: 8.3 against 7.1 us with one).
template <typename E, int D, int NW>
__global__ __launch_bounds__(NW * 64) void k_score_sum(
    const UnitInfo* __restrict__ units, const int32_t* __restrict__ scored,
    const E* __restrict__ q, const E* __restrict__ S, const int32_t* __restrict__ seq_lens,
    float* __restrict__ scores, uint32_t* __restrict__ err, int Hkv, int G, int t_cap,
    int quads_per_unit) {
  using Tile = ScoreTile<E, D>;
  // The query rows pass through the tile's own LDS before the tile does (its first staging
  // follows the barrier after qs is formed): 9.3 KB per one-tile workgroup instead of 11.3,
  // so 17 fit a CU instead of 14 (mixed_serving k_score_sum 20.0 against 20.4 us).
  __shared__ union {
    ScoreStage stage[NW];
    uint4 qrows[kMaxGroup * D * sizeof(E) / 16];
  } sh;
  static_assert(sizeof(ScoreStage) * NW >= kMaxGroup * D * sizeof(E), "query rows fit");
  ScoreStage* const stage = sh.stage;
  uint4* const qrows = sh.qrows;
  __shared__ double qs[D];
  const int n_su = gridDim.x / quads_per_unit;
  // One-tile grids run the highest tile indices first: the workgroups past a short unit's
  // end (most of them are at high indices) then come and go while slots are still free,
  // instead of among the last tiles, which wait for slots (mixed_serving k_score_sum 19.8
  // against 20.3 us).
  const int quad = NW == 1 ? quads_per_unit - 1 - (int)(blockIdx.x / n_su) : (int)(blockIdx.x / n_su);
  const int su = blockIdx.x % n_su;
  const int u = scored[su];
  const UnitInfo ui = units[u];
  const int b = u / Hkv, h = u % Hkv;
  const int T = load_seq_len(seq_lens, b, t_cap, err);
  const int log2r = ui.log2r;
  const int n_rows = (T >> ui.log2g) << log2r;
  const int tile0 = quad * NW;
  if (tile0 * kTile >= n_rows) return;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j0 = (tile0 + w) * kTile;
  // Rows past the unit's end read zero without a memory access.
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(S + (size_t)ui.sum_off * D), 0, n_rows * Tile::ROW_BYTES, kRsrcWord3);
  Tile tile;
  tile.load(rs, j0, lane);
  group_sum_f64<E, D>(q + ((size_t)b * Hkv * G + (size_t)h * G) * D, G, qrows, qs);
  __syncthreads();
  float f = (float)tile.template chain<true>(qs, stage[w], lane);
  for (int off = 1; off < (1 << log2r); off <<= 1) f = max_nan(f, __shfl_xor(f, off));
  const int row = j0 + lane;
  if ((lane & ((1 << log2r) - 1)) == 0 && row < n_rows)
    scores[(size_t)ui.block_off + (row >> log2r)] = f;
}

// Four-tile workgroups the current GPU holds at once: four per CU (their LDS).  The CU
// count is looked up once per device.
int64_t resident_quads() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cus[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return 4 * (int64_t)n;
}

template <typename E, int D, int NW>
int launch_sum_nw(const fx_plan* p, const void* q, const void* S, const int32_t* seq_lens,
                  float* scores, hipStream_t stream) {
  const int tiles = (p->max_scored_rows_cap + kTile - 1) / kTile;
  const int groups = (tiles + NW - 1) / NW;
  const dim3 grid((unsigned)((int64_t)groups * p->n_scored));
  k_score_sum<E, D, NW><<<grid, NW * 64, 0, stream>>>(
      p->d_units, p->d_scored, static_cast<const E*>(q), static_cast<const E*>(S), seq_lens,
      scores, p->d_error, p->desc.num_kv_heads, p->G, p->desc.t_cap, groups);
  return hipGetLastError();
}

template <typename E, int D>
int launch_sum(const fx_plan* p, const void* q, const void* S, const int32_t* seq_lens,
                      float* scores, hipStream_t stream) {
  const int tiles = (p->max_scored_rows_cap + kTile - 1) / kTile;
  const int quads = (tiles + kWaves - 1) / kWaves;
  if (quads == 0 || p->n_scored == 0) return hipSuccess;
  if ((int64_t)quads * p->n_scored > resident_quads())
    return launch_sum_nw<E, D, 1>(p, q, S, seq_lens, scores, stream);
  return launch_sum_nw<E, D, kWaves>(p, q, S, seq_lens, scores, stream);
}

template <typename E, int D, int GM>
int launch_gm(const fx_plan* p, const void* q, const void* S, const int32_t* seq_lens,
                     float* scores, hipStream_t stream) {
  const int tiles = (p->max_scored_rows_cap + kTile - 1) / kTile;
  const int quads = (tiles + kWaves - 1) / kWaves;
  if (quads == 0 || p->n_scored == 0) return hipSuccess;
  const dim3 grid((unsigned)((int64_t)quads * p->n_scored));
  k_score_max<E, D, GM><<<grid, kWaves * 64, 0, stream>>>(
      p->d_units, p->d_scored, static_cast<const E*>(q), static_cast<const E*>(S), seq_lens,
      scores, p->d_error, p->desc.num_kv_heads, p->G, p->desc.t_cap, quads);
  return hipGetLastError();
}

template <typename E, int D>
int launch_t(const fx_plan* p, const void* q, const void* S, const int32_t* seq_lens,
                    float* scores, hipStream_t stream) {
  if (p->desc.pooling != FX_POOL_SCORE_MAX)
    return launch_sum<E, D>(p, q, S, seq_lens, scores, stream);
  switch (p->G) {
    case 1: return launch_gm<E, D, 1>(p, q, S, seq_lens, scores, stream);
    case 2: return launch_gm<E, D, 2>(p, q, S, seq_lens, scores, stream);
    case 3: return launch_gm<E, D, 3>(p, q, S, seq_lens, scores, stream);
    case 4: return launch_gm<E, D, 4>(p, q, S, seq_lens, scores, stream);
    case 5: return launch_gm<E, D, 5>(p, q, S, seq_lens, scores, stream);
    case 6: return launch_gm<E, D, 6>(p, q, S, seq_lens, scores, stream);
    case 7: return launch_gm<E, D, 7>(p, q, S, seq_lens, scores, stream);
    default: return launch_gm<E, D, 8>(p, q, S, seq_lens, scores, stream);
  }
}

}  // namespace

int launch_score(const fx_plan* p, const void* q, const void* S, const int32_t* seq_lens,
                        float* scores, hipStream_t stream) {
  const int d = p->desc.head_dim;
  if (p->desc.dtype == FX_BF16)
    return d == 128 ? launch_t<bf16_t, 128>(p, q, S, seq_lens, scores, stream)
                    : launch_t<bf16_t, 64>(p, q, S, seq_lens, scores, stream);
  return d == 128 ? launch_t<float, 128>(p, q, S, seq_lens, scores, stream)
                  : launch_t<float, 64>(p, q, S, seq_lens, scores, stream);
}

}  // namespace fx
