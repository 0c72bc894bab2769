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
// Mapping: one 256-thread workgroup per unit.  The unit's values become monotone
// 32-bit keys in LDS (or, for units with more blocks than fit, in workspace memory;
// a template parameter picks which), and the forced set, the old eviction state and
// Γe are bitmaps next to them.  A radix select (4 passes of 8-bit digits, histogram
// in LDS) finds the threshold key tau and how many blocks with key == tau to take;
// the last taken tie's index jt comes from a prefix count in index order.
// Membership is then the O(1) test  key > tau  or  (key == tau and j <= jt).  Word-
// parallel passes turn that into selection bits (and eviction-mask updates), and a
// workgroup prefix sum compacts the selected indices in ascending order.
#include <climits>

#include "fx_device.h"

namespace fx {
namespace {

constexpr int NT = 256;

struct Threshold {
  uint32_t tau;
  int jt;
};

__device__ __forceinline__ bool chosen(const Threshold& t, uint32_t key, int j) {
  return key > t.tau || (key == t.tau && j <= t.jt);
}

struct SelectLds {
  uint32_t hist[256];
  int scan[NT / 64];
  int bcast[2];
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

// Threshold of the k best candidates among blocks [0, n) (see file comment).
template <class CandF>
__device__ Threshold block_select(int n, int k, const uint32_t* keys, CandF cand, SelectLds& L) {
  int c = 0;
  for (int j = threadIdx.x; j < n; j += NT) c += cand(j) ? 1 : 0;
  const int ncand = block_sum<NT>(c, L.scan);
  if (k <= 0 || ncand == 0) return {0xFFFFFFFFu, -1};   // nothing
  if (k >= ncand) return {0u, INT_MAX};                  // every candidate

  uint32_t prefix = 0, pmask = 0;
  int need = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    L.hist[threadIdx.x] = 0;
    __syncthreads();
    for (int j = threadIdx.x; j < n; j += NT) {
      const uint32_t kk = keys[j];
      if ((kk & pmask) == prefix && cand(j)) atomicAdd(&L.hist[(kk >> shift) & 255u], 1u);
    }
    __syncthreads();
    const int digit = 255 - (int)threadIdx.x;          // thread t looks at digit 255 - t
    const int hc = (int)L.hist[digit];
    int total;
    const int above = block_exclusive_scan<NT>(hc, L.scan, &total);   // count of larger digits
    if (above < need && need <= above + hc) {
      L.bcast[0] = digit;
      L.bcast[1] = need - above;
    }
    __syncthreads();
    const int d = L.bcast[0];
    need = L.bcast[1];
    __syncthreads();
    prefix |= (uint32_t)d << shift;
    pmask |= 255u << shift;
  }
  // `need` candidates with key == prefix are taken, lowest indices first.
  int seen = 0;
  for (int base = 0; base < n; base += NT) {
    const int j = base + (int)threadIdx.x;
    const int t = (j < n && keys[j] == prefix && cand(j)) ? 1 : 0;
    int total;
    const int before = block_exclusive_scan<NT>(t, L.scan, &total);
    if (t && seen + before + 1 == need) L.bcast[0] = j;
    seen += total;
    if (seen >= need) break;
  }
  __syncthreads();
  const int jt = L.bcast[0];
  __syncthreads();
  return {prefix, jt};
}

// keys[j] = monotone key of vals[j] for j < n.
__device__ __forceinline__ void load_keys(uint32_t* keys, const float* vals, int n, bool* nonfinite) {
  for (int j = threadIdx.x; j < n; j += NT) keys[j] = f32_key(vals[j], nonfinite);
  __syncthreads();
}

template <bool IN_LDS>
__global__ __launch_bounds__(NT) void k_topk(
    const UnitInfo* __restrict__ units, const float* __restrict__ scores,
    const float* __restrict__ logits, uint32_t* __restrict__ mask,
    const int32_t* __restrict__ seq_lens, int32_t* __restrict__ sel_idx,
    int32_t* __restrict__ sel_cnt, uint32_t* __restrict__ err, uint32_t* __restrict__ ws_keys,
    uint32_t* __restrict__ ws_bits, int Hkv, int t_cap, int max_sel, int key_cap, int word_cap) {
  extern __shared__ uint32_t dyn[];
  __shared__ SelectLds L;
  const int u = blockIdx.x;
  const UnitInfo ui = units[u];
  const int b = u / Hkv;
  const int T = load_seq_len(seq_lens, b, t_cap, err);
  const int g = ui.g;
  const int n_full = T >> ui.log2g;
  const int n_tot = (T + g - 1) >> ui.log2g;
  const int nwords = (n_tot + 31) >> 5;

  // Per-unit storage: keys, then the selection / Γe / old-eviction bitmaps.
  uint32_t* keys;
  uint32_t* selb;
  uint32_t* geb;
  uint32_t* evb;
  if constexpr (IN_LDS) {
    keys = dyn;
    selb = dyn + key_cap;
    geb = selb + word_cap;
    evb = geb + word_cap;
  } else {
    const int wcap = (ui.n_cap + 31) >> 5;
    keys = ws_keys + ui.block_off;
    selb = ws_bits + 3 * (size_t)ui.mask_off;
    geb = selb + wcap;
    evb = geb + wcap;
  }

  // Forced set F into selb (closed forms); clear geb; old eviction bits into evb.
  int fa0 = 0, fa1 = 0, fb0 = 0, fb1 = 0;   // F = [fa0, fa1) U [fb0, fb1) U extras
  const bool partial = n_full < n_tot;
  if (ui.mode == FX_STREAMING) {
    fa1 = (min(ui.sink, T) + g - 1) >> ui.log2g;
    if (ui.local > 0) {
      fb0 = max(0, T - ui.local) >> ui.log2g;
      fb1 = n_tot;
    }
  } else {
    if (ui.force_sink) fa1 = min(1, n_tot);
    if (ui.force_last || partial) {
      fb0 = max(n_tot - 1, 0);
      fb1 = n_tot;
    }
  }
  const uint32_t* mk_old = (ui.mode == FX_NOSA && mask) ? mask + ui.mask_off : nullptr;
  for (int w = threadIdx.x; w < nwords; w += NT) {
    uint32_t f = range_bits(w, fa0, fa1) | range_bits(w, fb0, fb1);
    if (partial) f |= range_bits(w, n_tot - 1, n_tot);
    selb[w] = f;
    geb[w] = 0u;
    evb[w] = mk_old ? mk_old[w] : 0u;
  }
  __syncthreads();

  bool nonfinite = false;
  const float* sc = scores + ui.block_off;
  if (ui.mode == FX_RETRIEVAL) {
    const int k = ui.top_k > 0 ? ui.top_k : (int)ceil((double)ui.budget * (double)n_tot);
    load_keys(keys, sc, n_full, &nonfinite);
    const Threshold A = block_select(n_full, k, keys, [&](int j) { return !bit(selb, j); }, L);
    for (int w = threadIdx.x; w < nwords; w += NT) {
      uint32_t s = selb[w];
      const uint32_t f = s;
      for (int e = 0; e < 32; ++e) {
        const int j = w * 32 + e;
        if (j >= n_full) break;
        if (!((f >> e) & 1u) && chosen(A, keys[j], j)) s |= 1u << e;
      }
      selb[w] = s;
    }
    __syncthreads();
  } else if (ui.mode == FX_NOSA) {
    if (ui.k_evict > 0) {
      load_keys(keys, logits + ui.block_off, n_full, &nonfinite);
      auto in_E = [&](int j) { return !bit(selb, j) && !bit(evb, j); };
      const Threshold A = block_select(n_full, ui.k_evict, keys, in_E, L);
      uint32_t* mk = mask + ui.mask_off;
      for (int w = threadIdx.x; w < nwords; w += NT) {
        uint32_t ge = 0, ev = 0;
        for (int e = 0; e < 32; ++e) {
          const int j = w * 32 + e;
          if (j >= n_full) break;
          if (in_E(j)) {
            if (chosen(A, keys[j], j)) ge |= 1u << e;
            else ev |= 1u << e;
          }
        }
        geb[w] = ge;
        if (ev) mk[w] = evb[w] | ev;
      }
      __syncthreads();
    } else if (mask) {
      // Γe is empty: every non-forced, not yet evicted full block becomes evicted.
      uint32_t* mk = mask + ui.mask_off;
      for (int w = threadIdx.x; w < nwords; w += NT) {
        const uint32_t full = range_bits(w, 0, n_full);
        const uint32_t ev = full & ~selb[w] & ~evb[w];
        if (ev) mk[w] = evb[w] | ev;
      }
    }
    load_keys(keys, sc, n_full, &nonfinite);
    auto in_Q = [&](int j) { return !bit(selb, j) && !bit(geb, j); };
    const Threshold Q = block_select(n_full, ui.top_k, keys, in_Q, L);
    for (int w = threadIdx.x; w < nwords; w += NT) {
      uint32_t s = selb[w] | geb[w];
      for (int e = 0; e < 32; ++e) {
        const int j = w * 32 + e;
        if (j >= n_full) break;
        if (in_Q(j) && chosen(Q, keys[j], j)) s |= 1u << e;
      }
      selb[w] = s;
    }
    __syncthreads();
  }

  // Compact the selection bits in ascending order.
  int running = 0;
  int32_t* out = sel_idx + (size_t)u * max_sel;
  bool overflow = false;
  for (int wbase = 0; wbase < nwords; wbase += NT) {
    const int w = wbase + (int)threadIdx.x;
    uint32_t bits = w < nwords ? selb[w] : 0u;
    int total;
    int pos = running + block_exclusive_scan<NT>(__popc(bits), L.scan, &total);
    while (bits) {
      const int e = __ffs(bits) - 1;
      bits &= bits - 1;
      if (pos < max_sel) out[pos] = w * 32 + e;
      else overflow = true;
      ++pos;
    }
    running += total;
  }
  const int cnt = min(running, max_sel);
  for (int i = cnt + (int)threadIdx.x; i < max_sel; i += NT) out[i] = -1;
  if (threadIdx.x == 0) sel_cnt[u] = cnt;
  if (overflow) atomicOr(err, (uint32_t)FX_ERR_SEL_COUNT);
  if (nonfinite) atomicOr(err, (uint32_t)FX_ERR_NONFINITE);
}

}  // namespace

size_t topk_lds_bytes(const fx_plan* p) {
  const size_t key_cap = (size_t)p->max_n_full_cap;
  const size_t word_cap = ((size_t)p->max_n_cap + 31) / 32;
  return (key_cap + 3 * word_cap) * 4;
}

hipError_t launch_topk(const fx_plan* p, const float* scores, const float* logits, uint32_t* mask,
                       const int32_t* seq_lens, int32_t* sel_idx, int32_t* sel_cnt,
                       uint32_t* ws_keys, uint32_t* ws_bits, hipStream_t stream) {
  const size_t lds = topk_lds_bytes(p);
  const int key_cap = p->max_n_full_cap;
  const int word_cap = (p->max_n_cap + 31) / 32;
  if (lds <= kTopkLdsLimit) {
    k_topk<true><<<dim3((unsigned)p->units), NT, lds, stream>>>(
        p->d_units, scores, logits, mask, seq_lens, sel_idx, sel_cnt, p->d_error, ws_keys, ws_bits,
        p->desc.num_kv_heads, p->desc.t_cap, p->max_sel, key_cap, word_cap);
  } else {
    k_topk<false><<<dim3((unsigned)p->units), NT, 0, stream>>>(
        p->d_units, scores, logits, mask, seq_lens, sel_idx, sel_cnt, p->d_error, ws_keys, ws_bits,
        p->desc.num_kv_heads, p->desc.t_cap, p->max_sel, key_cap, word_cap);
  }
  return hipGetLastError();
}

}  // namespace fx
