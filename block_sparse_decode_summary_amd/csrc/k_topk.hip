// Per-kv-head block selection.
//
// [Fluxion-NL] "Technische Samenvatting: Fluxion", Kerninzichten item 2 and
// Systeemcomponenten: streaming heads keep the default retained KV (sink and recent
// window) and need no selection; retrieval heads select top-k blocks at their own
// granularity and budget.  [Fluxion-KO] (Korean page on the same paper), section
// 해결책, strategy 2, says the same in lay terms.  [NOSA-DE] "Technisches Resümee:
// NOSA: Native und Offloadable Sparse Attention", Methodik §1: the selection is the
// union of a query-aware part Γq (top-k by score) and a query-agnostic part Γe (top
// k_e by eviction logit) with strict eviction (a block Γe drops can never re-enter
// Γe); "ED-DMA": the logits are ranked as they are, before any exponential.
//
// Definitions (also in include/fx.h): forced set F per mode; retrieval takes the k
// best full blocks outside F by score, k = top_k or ceil(budget * n_tot) in float64;
// NOSA takes Γe among non-evicted full blocks outside F, evicts the rest of them,
// then Γq among full blocks outside F and Γe (evicted ones included).  "Best" is the
// larger value, equal values by the lower block index; -0 equals +0.
//
// Order value.  A block's value becomes a monotone 32-bit key (f32_key) and the pair
// (key, block index) becomes one 64-bit number, key in the upper half and the bitwise
// complement of the index in the lower half.  It is larger exactly when the block is
// better, and no two blocks share it, so "the k best" is "order value >= the k-th
// largest order value" with no tie rule left over.
//
// Selecting the k-th largest order value (select_kth): one reduction gives the
// candidate count and key range, so the bits above the highest one in which
// candidates differ are known; histograms of the next 11-bit digit (LDS atomics, two
// buffers so that clearing one overlaps the pass over the other) narrow the prefix
// until at most 64 candidates share it; those are gathered into one wave, which ranks
// them with lane broadcasts.
//
// Mapping: one 256-thread workgroup per unit.  Thread t owns blocks j = i*256 + t.
// When every unit has at most 32*256 block slots the keys, the candidate flags and the
// old eviction words stay in registers (k_topk_reg), wave ballots of the per-block
// flags give the bitmap words, and a scan over (row, wave) counts compacts the
// selection straight into sel_idx in ascending order.  Larger units keep keys and
// bitmaps in the workspace (k_topk_mem), with the same selection arithmetic.
#include <climits>

#include "fx_device.h"

namespace fx {
namespace {

constexpr int NT = 256;
constexpr int NW = NT / 64;
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;        // 2048 histogram bins, 8 per thread
constexpr int kBinsPerThread = kBins / NT;
constexpr int kRankCap = 64;                  // candidates ranked inside one wave
constexpr int kMaxRows = kTopkRegBlocks / NT; // rows of the register path

__device__ __forceinline__ uint64_t order_value(uint32_t key, int j) {
  return ((uint64_t)key << 32) | (uint64_t)(~(uint32_t)j);
}

struct Kth {
  uint64_t thr;   // chosen iff any && order value >= thr
  bool any;
};

struct SelectLds {
  uint32_t hist[2][kBins];
  uint64_t rank_vals[kRankCap];
  uint64_t thr;
  uint32_t red[3][NW];
  int scan[2][NW];
  int bcast[3];
  int rowcnt[3][kMaxRows * NW];                 // per list: selection, added, removed
  uint32_t prevbits[kTopkRegBlocks / 32];       // the previous selection (fused delta)
};

__device__ __forceinline__ bool bit(const uint32_t* bits, int j) {
  return ((bits[j >> 5] >> (j & 31)) & 1u) != 0;
}

// Bits [a, b) of word w.
__device__ __forceinline__ uint32_t range_bits(int w, int a, int b) {
  const int lo = max(a - w * 32, 0), hi = min(b - w * 32, 32);
  if (hi <= lo) return 0u;
  const uint32_t top = hi == 32 ? 0xFFFFFFFFu : ((1u << hi) - 1u);
  return top & ~((1u << lo) - 1u);
}

// Exclusive prefix sum over the workgroup; slot (NW ints) is written, then read after
// one barrier.  The caller keeps a barrier between this read and the slot's next write.
__device__ __forceinline__ int block_scan_excl(int x, int* slot, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int incl = (int)wave_scan_incl_u32((uint32_t)x);
  if (lane == 63) slot[w] = incl;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int v = slot[i];
    off += i < w ? v : 0;
    tot += v;
  }
  *total = tot;
  return off + incl - x;
}

__device__ __forceinline__ uint64_t lane_value64(uint64_t v, int lane) {
  return ((uint64_t)lane_value((uint32_t)(v >> 32), lane) << 32) | lane_value((uint32_t)v, lane);
}

// The k-th largest order value among the candidates src enumerates (src.each(f) calls
// f(key, j) for each candidate this thread owns).  n_index bounds the candidates'
// block indices.  Entry: hist[0] is zero.  Exit: hist[0] is zero again and a barrier
// has passed, so the LDS may be reused at once.  Every thread must call this.
template <class Src>
__device__ __forceinline__ Kth select_kth(const Src& src, int k, int n_index, SelectLds& L) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t cnt = 0, kmin = 0xFFFFFFFFu, kmax = 0u;
  src.each([&](uint32_t key, int) {
    ++cnt;
    kmin = min(kmin, key);
    kmax = max(kmax, key);
  });
  cnt = wave_sum_u32(cnt);
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  if (lane == 0) {
    L.red[0][w] = cnt;
    L.red[1][w] = kmin;
    L.red[2][w] = kmax;
  }
  __syncthreads();
  cnt = 0;
  kmin = 0xFFFFFFFFu;
  kmax = 0u;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    cnt += L.red[0][i];
    kmin = min(kmin, L.red[1][i]);
    kmax = max(kmax, L.red[2][i]);
  }
  if (k <= 0 || cnt == 0 || k >= (int)cnt) {
    __syncthreads();
    return {0ull, k > 0 && cnt > 0};
  }

  // cnt >= 2 here.  Bits above hb are common to every candidate: with differing keys
  // hb is the top differing key bit; with one key value it is the top bit in which
  // complemented indices below n_index can differ.
  int hb = kmin != kmax ? 63 - __builtin_clz(kmin ^ kmax)
                        : 31 - __builtin_clz((uint32_t)max(n_index - 1, 1));
  uint64_t pmask = hb >= 63 ? 0ull : ~((2ull << hb) - 1ull);
  uint64_t prefix = order_value(kmin, 0) & pmask;
  int need = k, m = (int)cnt, pass = 0;
  while (m > kRankCap && hb >= 0) {
    const int shift = max(hb + 1 - kDigitBits, 0);
    const uint32_t dmask = (2u << (hb - shift)) - 1u;
    uint32_t* H = L.hist[pass & 1];
    src.each([&](uint32_t key, int j) {
      const uint64_t v = order_value(key, j);
      if ((v & pmask) == prefix) atomicAdd(&H[(uint32_t)(v >> shift) & dmask], 1u);
    });
    __syncthreads();
    // Thread t owns digits kBins-1-8t down to kBins-8-8t (descending).
    const uint4 hi4 = *reinterpret_cast<const uint4*>(&H[kBins - 8 * threadIdx.x - 4]);
    const uint4 lo4 = *reinterpret_cast<const uint4*>(&H[kBins - 8 * threadIdx.x - 8]);
    const int c[kBinsPerThread] = {(int)hi4.w, (int)hi4.z, (int)hi4.y, (int)hi4.x,
                                   (int)lo4.w, (int)lo4.z, (int)lo4.y, (int)lo4.x};
    int local = 0;
#pragma unroll
    for (int i = 0; i < kBinsPerThread; ++i) local += c[i];
    int total;
    int above = block_scan_excl(local, L.scan[0], &total);
#pragma unroll
    for (int i = 0; i < kBinsPerThread; ++i) {
      if (above < need && need <= above + c[i]) {
        L.bcast[0] = kBins - 1 - (int)(threadIdx.x * kBinsPerThread + i);
        L.bcast[1] = need - above;
        L.bcast[2] = c[i];
      }
      above += c[i];
    }
    // The other buffer was last read before the previous pass's final barrier.
    uint4* other = reinterpret_cast<uint4*>(&L.hist[(pass + 1) & 1][kBins - 8 * threadIdx.x - 8]);
    other[0] = make_uint4(0, 0, 0, 0);
    other[1] = make_uint4(0, 0, 0, 0);
    __syncthreads();
    const uint32_t d = (uint32_t)L.bcast[0];
    need = L.bcast[1];
    m = L.bcast[2];
    prefix |= (uint64_t)d << shift;
    pmask |= (uint64_t)dmask << shift;
    hb = shift - 1;
    ++pass;
  }

  // The m (<= kRankCap) candidates that match the prefix, gathered in any order; the
  // one with exactly need-1 better ones among them is the threshold.
  int mine = 0;
  src.each([&](uint32_t key, int j) { mine += (order_value(key, j) & pmask) == prefix ? 1 : 0; });
  int total;
  int pos = block_scan_excl(mine, L.scan[1], &total);
  src.each([&](uint32_t key, int j) {
    const uint64_t v = order_value(key, j);
    if ((v & pmask) == prefix) {
      if (pos < kRankCap) L.rank_vals[pos] = v;
      ++pos;
    }
  });
  __syncthreads();
  if (w == 0) {
    const int mm = __builtin_amdgcn_readfirstlane(min(total, kRankCap));
    const uint64_t v = lane < mm ? L.rank_vals[lane] : 0ull;
    int better = 0;
    for (int i = 0; i < mm; ++i) better += lane_value64(v, i) > v ? 1 : 0;
    if (lane < mm && better == need - 1) L.thr = v;
  }
  __syncthreads();
  const uint64_t thr = L.thr;
  if (pass & 1) {   // the last pass used hist[0]
    uint4* mine4 = reinterpret_cast<uint4*>(&L.hist[0][kBins - 8 * threadIdx.x - 8]);
    mine4[0] = make_uint4(0, 0, 0, 0);
    mine4[1] = make_uint4(0, 0, 0, 0);
  }
  __syncthreads();
  return {thr, true};
}

// Forced set F of a unit: [0, fa1) U [fb0, fb1) U {n_tot-1 if the last block is
// partial} (every mode; see include/fx.h).
struct Forced {
  int fa1, fb0, fb1, extra;
  __device__ __forceinline__ bool has(int j) const {
    return j < fa1 || (j >= fb0 && j < fb1) || j == extra;
  }
};

__device__ __forceinline__ Forced forced_set(const UnitInfo& ui, int T, int n_full, int n_tot) {
  Forced f{0, 0, 0, -1};
  const int g = ui.g;
  const bool partial = n_full < n_tot;
  if (ui.mode == FX_STREAMING) {
    f.fa1 = (min(ui.sink, T) + g - 1) >> ui.log2g;
    if (ui.local > 0) {
      f.fb0 = max(0, T - ui.local) >> ui.log2g;
      f.fb1 = n_tot;
    }
  } else {
    if (ui.force_sink) f.fa1 = min(1, n_tot);
    if (ui.force_last) {
      f.fb0 = max(n_tot - 1, 0);
      f.fb1 = n_tot;
    }
  }
  if (partial) f.extra = n_tot - 1;
  return f;
}

// ---- register path --------------------------------------------------------------------

template <int KPT>
struct RegSrc {
  const uint32_t (&key)[KPT];
  uint32_t cand;   // bit i: block i*NT + t is a candidate
  template <class F>
  __device__ __forceinline__ void each(F f) const {
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      if ((cand >> i) & 1u) f(key[i], i * NT + (int)threadIdx.x);
  }
};

template <int KPT>
__device__ __forceinline__ uint32_t chosen_bits(const Kth& s, const uint32_t (&key)[KPT], uint32_t cand) {
  uint32_t out = 0;
  if (!s.any) return 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const bool c = ((cand >> i) & 1u) && order_value(key[i], i * NT + (int)threadIdx.x) >= s.thr;
    out |= c ? (1u << i) : 0u;
  }
  return out;
}

// The set differences against the previous selection, computed by the same workgroup
// (prev == nullptr: none).  Block j of the unit is bit j / NT of thread j % NT, as for
// the selection itself.
struct DeltaArgs {
  const int32_t* prev_idx;
  const int32_t* prev_cnt;
  int32_t* added;
  int32_t* added_cnt;
  int32_t* removed;
  int32_t* removed_cnt;
};

// Writes the blocks of the per-thread masks m (bit i: block i*NT + t) in ascending order
// to out[0 .. count), pads out to max_sel with -1 and stores the count.  rowcnt holds,
// after a barrier, the number of set bits of row i in wave w at rowcnt[i*NW + w].
template <int KPT>
__device__ __forceinline__ int write_list(uint32_t m, const int* rowcnt, int32_t* out,
                                          int max_sel) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  constexpr int NE = KPT * NW;
  constexpr int R = (NE + 63) / 64;
  uint32_t excl[R];
  uint32_t running = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int idx = r * 64 + lane;
    const uint32_t v = idx < NE ? (uint32_t)rowcnt[idx] : 0u;
    const uint32_t incl = wave_scan_incl_u32(v);
    excl[r] = running + incl - v;
    running += lane_value(incl, 63);
  }
  const int total = (int)running;
  const int wu = __builtin_amdgcn_readfirstlane(w);
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    // Entries i*NW .. i*NW+NW-1 lie in one 64-entry chunk.
    const uint64_t b = __ballot((m >> i) & 1u);
    const int base = (int)lane_value(excl[(i * NW) >> 6], ((i * NW) & 63) + wu);
    if ((m >> i) & 1u) {
      const int pos = base + (int)lanes_below(b);
      if (pos < max_sel) out[pos] = i * NT + t;
    }
  }
  for (int i = min(total, max_sel) + t; i < max_sel; i += NT) out[i] = -1;
  return total;
}

template <int KPT>
__device__ __forceinline__ int row_count(uint32_t m, int i_lane) {
  int c = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int v = __popcll(__ballot((m >> i) & 1u));
    c = i_lane == i ? v : c;
  }
  return c;
}

template <int KPT>
__global__ __launch_bounds__(NT) void k_topk_reg(
    const UnitInfo* __restrict__ units, const float* __restrict__ scores,
    const float* __restrict__ logits, uint32_t* __restrict__ mask,
    const int32_t* __restrict__ seq_lens, int32_t* __restrict__ sel_idx,
    int32_t* __restrict__ sel_cnt, DeltaArgs D, uint32_t* __restrict__ err, int Hkv, int t_cap,
    int max_sel) {
  static_assert(KPT <= 32 && KPT * NT <= kTopkRegBlocks, "rows per thread");
  __shared__ SelectLds L;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  {
    uint4* h = reinterpret_cast<uint4*>(&L.hist[0][8 * t]);
    h[0] = make_uint4(0, 0, 0, 0);
    h[1] = make_uint4(0, 0, 0, 0);
    if (D.prev_idx)
      for (int i = t; i < KPT * NT / 32; i += NT) L.prevbits[i] = 0u;
  }
  const int u = blockIdx.x;
  const UnitInfo ui = units[u];
  const int T = load_seq_len(seq_lens, u / Hkv, t_cap, err);
  const int n_full = T >> ui.log2g;
  const int n_tot = (T + ui.g - 1) >> ui.log2g;
  const Forced F = forced_set(ui, T, n_full, n_tot);
  const bool scored = ui.mode != FX_STREAMING;
  const bool evict_keys = ui.mode == FX_NOSA && ui.k_evict > 0;
  const bool old_mask = ui.mode == FX_NOSA && mask != nullptr;

  // Issue every load before using any.
  float sv[KPT], lv[KPT];
  uint32_t oldw[KPT];
  const float* sc = scores + ui.block_off;
  const float* lg = logits + ui.block_off;
  const uint32_t* mk = mask + ui.mask_off;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int j = i * NT + t;
    sv[i] = (scored && j < n_full) ? sc[j] : 0.0f;
    lv[i] = (evict_keys && j < n_full) ? lg[j] : 0.0f;
    oldw[i] = (old_mask && j < n_tot) ? mk[j >> 5] : 0u;
  }
  uint32_t full = 0, forced = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int j = i * NT + t;
    full |= j < n_full ? (1u << i) : 0u;
    forced |= (j < n_tot && F.has(j)) ? (1u << i) : 0u;
  }
  bool nonfinite = false;
  uint32_t skey[KPT], lkey[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const bool in = (full >> i) & 1u;
    skey[i] = (scored && in) ? f32_key(sv[i], &nonfinite) : 0u;
    lkey[i] = (evict_keys && in) ? f32_key(lv[i], &nonfinite) : 0u;
  }
  __syncthreads();   // hist[0] cleared

  uint32_t sel = forced;
  if (ui.mode == FX_RETRIEVAL) {
    const int k = ui.top_k > 0 ? ui.top_k : (int)ceil((double)ui.budget * (double)n_tot);
    const uint32_t cand = full & ~forced;
    const Kth A = select_kth(RegSrc<KPT>{skey, cand}, k, n_full, L);
    sel |= chosen_bits(A, skey, cand);
  } else if (ui.mode == FX_NOSA) {
    uint32_t oldev = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) oldev |= ((oldw[i] >> (t & 31)) & 1u) << i;
    const uint32_t E = full & ~forced & ~oldev;
    uint32_t ge = 0;
    if (ui.k_evict > 0) {
      const Kth A = select_kth(RegSrc<KPT>{lkey, E}, ui.k_evict, n_full, L);
      ge = chosen_bits(A, lkey, E);
    }
    if (mask) {
      // Every block of E outside Γe becomes evicted: OR the new bits into the words.
      const uint32_t ev = E & ~ge;
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const uint64_t b = __ballot((ev >> i) & 1u);
        const int word = (i * NT + w * 64) >> 5;
        if (lane == 0 && (uint32_t)b) mask[ui.mask_off + word] = oldw[i] | (uint32_t)b;
        if (lane == 32 && (uint32_t)(b >> 32)) mask[ui.mask_off + word + 1] = oldw[i] | (uint32_t)(b >> 32);
      }
    }
    const uint32_t candq = full & ~forced & ~ge;
    const Kth Q = select_kth(RegSrc<KPT>{skey, candq}, ui.top_k, n_full, L);
    sel |= ge | chosen_bits(Q, skey, candq);
  }

  // The previous selection as a bitmap (the zeroing above is behind a barrier).  Its
  // entries must be ascending blocks of the unit (as this kernel writes them); others are
  // skipped and flagged.
  uint32_t prevm = 0;
  if (D.prev_idx) {
    int pc = D.prev_cnt[u];
    if (pc < 0 || pc > max_sel) {
      if (t == 0) atomicOr(err, (uint32_t)FX_ERR_SEL_COUNT);
      pc = min(max(pc, 0), max_sel);
    }
    const int32_t* prev = D.prev_idx + (size_t)u * max_sel;
    for (int i = t; i < pc; i += NT) {
      const int pj = prev[i];
      if (pj >= 0 && pj < ui.n_cap && (i == 0 || prev[i - 1] < pj))
        atomicOr(&L.prevbits[pj >> 5], 1u << (pj & 31));
      else
        atomicOr(err, (uint32_t)FX_ERR_SEL_INDEX);
    }
  }

  // Compact in ascending block order: rows i, then waves w, then lanes.
  const int c0 = row_count<KPT>(sel, lane);
  if (lane < KPT) L.rowcnt[0][lane * NW + w] = c0;
  __syncthreads();   // row counts and the previous-selection bitmap
  if (D.prev_idx) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int j = i * NT + t;
      prevm |= ((L.prevbits[j >> 5] >> (j & 31)) & 1u) << i;
    }
    const int c1 = row_count<KPT>(sel & ~prevm, lane);
    const int c2 = row_count<KPT>(prevm & ~sel, lane);
    if (lane < KPT) {
      L.rowcnt[1][lane * NW + w] = c1;
      L.rowcnt[2][lane * NW + w] = c2;
    }
  }
  const int total = write_list<KPT>(sel, L.rowcnt[0], sel_idx + (size_t)u * max_sel, max_sel);
  if (t == 0) {
    sel_cnt[u] = min(total, max_sel);
    if (total > max_sel) atomicOr(err, (uint32_t)FX_ERR_SEL_COUNT);
  }
  if (D.prev_idx) {
    __syncthreads();   // the added / removed row counts
    const int na = write_list<KPT>(sel & ~prevm, L.rowcnt[1], D.added + (size_t)u * max_sel,
                                   max_sel);
    const int nr = write_list<KPT>(prevm & ~sel, L.rowcnt[2], D.removed + (size_t)u * max_sel,
                                   max_sel);
    if (t == 0) {
      D.added_cnt[u] = min(na, max_sel);
      D.removed_cnt[u] = min(nr, max_sel);
    }
  }
  if (nonfinite) atomicOr(err, (uint32_t)FX_ERR_NONFINITE);
}

// ---- workspace path (units with more than kTopkRegBlocks block slots) -----------------

struct MemSrc {
  const uint32_t* keys;
  const uint32_t* excl_a;   // candidates: j < n with neither bit set
  const uint32_t* excl_b;   // may be null
  int n;
  template <class F>
  __device__ __forceinline__ void each(F f) const {
    for (int j = threadIdx.x; j < n; j += NT)
      if (!bit(excl_a, j) && !(excl_b && bit(excl_b, j))) f(keys[j], j);
  }
};

__device__ __forceinline__ bool chosen(const Kth& s, uint32_t key, int j) {
  return s.any && order_value(key, j) >= s.thr;
}

// Per 64 consecutive blocks one wave ballot gives two bitmap words; lanes 0 and 32
// write them.  pred(j) is evaluated for j < n only; every thread must call this.
template <class PredF>
__device__ __forceinline__ void ballot_words(int n, int nwords, PredF pred, uint32_t* words_out) {
  const int lane = threadIdx.x & 63;
  for (int base = (int)(threadIdx.x & ~63); base < nwords * 32; base += NT) {
    const int j = base + lane;
    const bool p = j < n && pred(j);
    const uint64_t m = __ballot(p);
    const int wd = base >> 5;
    if (lane == 0 && wd < nwords) words_out[wd] = (uint32_t)m;
    if (lane == 32 && wd + 1 < nwords) words_out[wd + 1] = (uint32_t)(m >> 32);
  }
}

__device__ __forceinline__ void load_keys(uint32_t* keys, const float* vals, int n, bool* nonfinite) {
  for (int j = threadIdx.x; j < n; j += NT) keys[j] = f32_key(vals[j], nonfinite);
  __syncthreads();
}

__global__ __launch_bounds__(NT) void k_topk_mem(
    const UnitInfo* __restrict__ units, const float* __restrict__ scores,
    const float* __restrict__ logits, uint32_t* __restrict__ mask,
    const int32_t* __restrict__ seq_lens, int32_t* __restrict__ sel_idx,
    int32_t* __restrict__ sel_cnt, uint32_t* __restrict__ err, uint32_t* __restrict__ ws_keys,
    uint32_t* __restrict__ ws_bits, int Hkv, int t_cap, int max_sel) {
  __shared__ SelectLds L;
  const int t = threadIdx.x;
  {
    uint4* h = reinterpret_cast<uint4*>(&L.hist[0][8 * t]);
    h[0] = make_uint4(0, 0, 0, 0);
    h[1] = make_uint4(0, 0, 0, 0);
  }
  const int u = blockIdx.x;
  const UnitInfo ui = units[u];
  const int T = load_seq_len(seq_lens, u / Hkv, t_cap, err);
  const int n_full = T >> ui.log2g;
  const int n_tot = (T + ui.g - 1) >> ui.log2g;
  const int nwords = (n_tot + 31) >> 5;
  const Forced F = forced_set(ui, T, n_full, n_tot);

  // Keys, then the forced / Γe / old-eviction bitmaps of this unit.
  const int wcap = (ui.n_cap + 31) >> 5;
  uint32_t* keys = ws_keys + ui.block_off;
  uint32_t* selb = ws_bits + 3 * (size_t)ui.mask_off;
  uint32_t* geb = selb + wcap;
  uint32_t* evb = geb + wcap;
  const uint32_t* mk_old = (ui.mode == FX_NOSA && mask) ? mask + ui.mask_off : nullptr;
  for (int wd = t; wd < nwords; wd += NT) {
    uint32_t f = range_bits(wd, 0, F.fa1) | range_bits(wd, F.fb0, F.fb1);
    if (F.extra >= 0) f |= range_bits(wd, F.extra, F.extra + 1);
    selb[wd] = f;
    geb[wd] = 0u;
    evb[wd] = mk_old ? mk_old[wd] : 0u;
  }
  __syncthreads();

  bool nonfinite = false;
  const float* sc = scores + ui.block_off;
  if (ui.mode == FX_RETRIEVAL) {
    const int k = ui.top_k > 0 ? ui.top_k : (int)ceil((double)ui.budget * (double)n_tot);
    load_keys(keys, sc, n_full, &nonfinite);
    const Kth A = select_kth(MemSrc{keys, selb, nullptr, n_full}, k, n_full, L);
    ballot_words(n_full, nwords, [&](int j) { return !bit(selb, j) && chosen(A, keys[j], j); }, geb);
    __syncthreads();
    for (int wd = t; wd < nwords; wd += NT) selb[wd] |= geb[wd];
    __syncthreads();
  } else if (ui.mode == FX_NOSA) {
    if (ui.k_evict > 0) {
      load_keys(keys, logits + ui.block_off, n_full, &nonfinite);
      const Kth A = select_kth(MemSrc{keys, selb, evb, n_full}, ui.k_evict, n_full, L);
      ballot_words(n_full, nwords,
                   [&](int j) { return !bit(selb, j) && !bit(evb, j) && chosen(A, keys[j], j); }, geb);
      __syncthreads();
    }
    if (mask) {
      // Every block of E outside Γe becomes evicted.
      uint32_t* mk = mask + ui.mask_off;
      for (int wd = t; wd < nwords; wd += NT) {
        const uint32_t ev = range_bits(wd, 0, n_full) & ~selb[wd] & ~evb[wd] & ~geb[wd];
        if (ev) mk[wd] = evb[wd] | ev;
      }
    }
    __syncthreads();   // the Γe select used keys[]
    load_keys(keys, sc, n_full, &nonfinite);
    const Kth Q = select_kth(MemSrc{keys, selb, geb, n_full}, ui.top_k, n_full, L);
    // Γq bits into evb (no longer needed), then selection = F | Γe | Γq.
    ballot_words(n_full, nwords,
                 [&](int j) { return !bit(selb, j) && !bit(geb, j) && chosen(Q, keys[j], j); }, evb);
    __syncthreads();
    for (int wd = t; wd < nwords; wd += NT) selb[wd] |= geb[wd] | evb[wd];
    __syncthreads();
  }

  // Compact the selection bits in ascending order.
  int running = 0;
  int32_t* out = sel_idx + (size_t)u * max_sel;
  bool overflow = false;
  for (int wbase = 0, it = 0; wbase < nwords; wbase += NT, ++it) {
    const int wd = wbase + t;
    uint32_t bits = wd < nwords ? selb[wd] : 0u;
    int total;
    int pos = running + block_scan_excl(__popc(bits), L.scan[it & 1], &total);
    while (bits) {
      const int e = __ffs(bits) - 1;
      bits &= bits - 1;
      if (pos < max_sel) out[pos] = wd * 32 + e;
      else overflow = true;
      ++pos;
    }
    running += total;
  }
  const int cnt = min(running, max_sel);
  for (int i = cnt + t; i < max_sel; i += NT) out[i] = -1;
  if (t == 0) sel_cnt[u] = cnt;
  if (overflow) atomicOr(err, (uint32_t)FX_ERR_SEL_COUNT);
  if (nonfinite) atomicOr(err, (uint32_t)FX_ERR_NONFINITE);
}

template <int KPT>
void launch_reg(const fx_plan* p, const float* scores, const float* logits, uint32_t* mask,
                const int32_t* seq_lens, int32_t* sel_idx, int32_t* sel_cnt, const DeltaArgs& D,
                hipStream_t stream) {
  k_topk_reg<KPT><<<dim3((unsigned)p->units), NT, 0, stream>>>(
      p->d_units, scores, logits, mask, seq_lens, sel_idx, sel_cnt, D, p->d_error,
      p->desc.num_kv_heads, p->desc.t_cap, p->max_sel);
}

}  // namespace

bool topk_in_registers(const fx_plan* p) { return p->max_n_cap <= kTopkRegBlocks; }

hipError_t launch_topk(const fx_plan* p, const float* scores, const float* logits, uint32_t* mask,
                       const int32_t* seq_lens, int32_t* sel_idx, int32_t* sel_cnt,
                       uint32_t* ws_keys, uint32_t* ws_bits, const int32_t* prev_idx,
                       const int32_t* prev_cnt, int32_t* added, int32_t* added_cnt,
                       int32_t* removed, int32_t* removed_cnt, hipStream_t stream) {
  const DeltaArgs D{prev_idx, prev_cnt, added, added_cnt, removed, removed_cnt};
  const int n = p->max_n_cap;
  if (n <= 1 * NT) launch_reg<1>(p, scores, logits, mask, seq_lens, sel_idx, sel_cnt, D, stream);
  else if (n <= 2 * NT) launch_reg<2>(p, scores, logits, mask, seq_lens, sel_idx, sel_cnt, D, stream);
  else if (n <= 4 * NT) launch_reg<4>(p, scores, logits, mask, seq_lens, sel_idx, sel_cnt, D, stream);
  else if (n <= 8 * NT) launch_reg<8>(p, scores, logits, mask, seq_lens, sel_idx, sel_cnt, D, stream);
  else if (n <= 16 * NT) launch_reg<16>(p, scores, logits, mask, seq_lens, sel_idx, sel_cnt, D, stream);
  else if (n <= 32 * NT) launch_reg<32>(p, scores, logits, mask, seq_lens, sel_idx, sel_cnt, D, stream);
  else {
    k_topk_mem<<<dim3((unsigned)p->units), NT, 0, stream>>>(
        p->d_units, scores, logits, mask, seq_lens, sel_idx, sel_cnt, p->d_error, ws_keys, ws_bits,
        p->desc.num_kv_heads, p->desc.t_cap, p->max_sel);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !prev_idx) return e;
    // The workspace path leaves the differences to the delta kernel.
    return launch_delta(p, prev_idx, prev_cnt, sel_idx, sel_cnt, added, added_cnt, removed,
                        removed_cnt, stream);
  }
  return hipGetLastError();
}

}  // namespace fx
