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
// Mapping: one 256-thread workgroup per unit.  A radix select over 32-bit monotone
// keys (4 passes of 8-bit digits, histograms in LDS) finds the threshold key tau and
// how many blocks with key == tau to take; the last taken tie's index jt comes from
// a prefix count in index order.  Membership is then the O(1) test
//     key > tau  or  (key == tau and j <= jt),
// so no per-block state is stored.  A final pass builds 32-block selection words,
// writes eviction-mask updates word by word, and compacts the selected indices in
// ascending order with a workgroup prefix sum.
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

// Threshold of the k best candidates among blocks [0, n) (see file comment).
template <class KeyF, class CandF>
__device__ Threshold block_select(int n, int k, KeyF key, CandF cand, SelectLds& L) {
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
      if (!cand(j)) continue;
      const uint32_t kk = key(j);
      if ((kk & pmask) == prefix) atomicAdd(&L.hist[(kk >> shift) & 255u], 1u);
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
    const int t = (j < n && cand(j) && key(j) == prefix) ? 1 : 0;
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

__global__ __launch_bounds__(NT) void k_topk(
    const UnitInfo* __restrict__ units, const float* __restrict__ scores,
    const float* __restrict__ logits, uint32_t* __restrict__ mask,
    const int32_t* __restrict__ seq_lens, int32_t* __restrict__ sel_idx,
    int32_t* __restrict__ sel_cnt, uint32_t* __restrict__ err, int Hkv, int t_cap, int max_sel) {
  __shared__ SelectLds L;
  const int u = blockIdx.x;
  const UnitInfo ui = units[u];
  const int b = u / Hkv;
  const int T = load_seq_len(seq_lens, b, t_cap, err);
  const int g = ui.g;
  const int n_full = T >> ui.log2g;
  const int n_tot = (T + g - 1) >> ui.log2g;
  const bool partial = n_full < n_tot;

  int sink_blocks = 0, local_start = INT_MAX;
  if (ui.mode == FX_STREAMING) {
    sink_blocks = (min(ui.sink, T) + g - 1) >> ui.log2g;
    if (ui.local > 0) local_start = max(0, T - ui.local) >> ui.log2g;
  }
  const bool mode_stream = ui.mode == FX_STREAMING;
  auto forced = [&](int j) -> bool {
    if (j == n_tot - 1 && partial) return true;
    if (mode_stream) return j < sink_blocks || j >= local_start;
    return (ui.force_sink && j == 0) || (ui.force_last && j == n_tot - 1);
  };

  bool nonfinite = false;
  const float* sc = scores + ui.block_off;
  const float* lg = logits ? logits + ui.block_off : nullptr;
  uint32_t* mk = mask ? mask + ui.mask_off : nullptr;
  auto key_sc = [&](int j) -> uint32_t { return f32_key(sc[j], &nonfinite); };
  auto key_lg = [&](int j) -> uint32_t { return f32_key(lg[j], &nonfinite); };
  auto evicted = [&](int j) -> bool { return mk ? ((mk[j >> 5] >> (j & 31)) & 1u) != 0 : false; };

  Threshold A{0xFFFFFFFFu, -1}, Q{0xFFFFFFFFu, -1};
  if (ui.mode == FX_RETRIEVAL) {
    const int k = ui.top_k > 0 ? ui.top_k
                               : (int)ceil((double)ui.budget * (double)n_tot);
    A = block_select(n_full, k, key_sc, [&](int j) { return !forced(j); }, L);
  } else if (ui.mode == FX_NOSA) {
    if (ui.k_evict > 0)
      A = block_select(n_full, ui.k_evict, key_lg,
                       [&](int j) { return !forced(j) && !evicted(j); }, L);
    auto in_e = [&](int j) -> bool {
      return ui.k_evict > 0 && !forced(j) && !evicted(j) && chosen(A, key_lg(j), j);
    };
    Q = block_select(n_full, ui.top_k, key_sc, [&](int j) { return !forced(j) && !in_e(j); }, L);
  }

  const int nwords = (n_tot + 31) >> 5;
  int running = 0;
  int32_t* out = sel_idx + (size_t)u * max_sel;
  bool overflow = false;
  for (int wbase = 0; wbase < nwords; wbase += NT) {
    const int wi = wbase + (int)threadIdx.x;
    uint32_t bits = 0, ev = 0;
    if (wi < nwords) {
      for (int e = 0; e < 32; ++e) {
        const int j = wi * 32 + e;
        if (j >= n_tot) break;
        const bool f = forced(j);
        bool s = f;
        if (!f && j < n_full) {
          if (ui.mode == FX_RETRIEVAL) {
            s = chosen(A, key_sc(j), j);
          } else if (ui.mode == FX_NOSA) {
            const bool ce = !evicted(j);
            const bool ie = ui.k_evict > 0 && ce && chosen(A, key_lg(j), j);
            s = ie || chosen(Q, key_sc(j), j);
            if (ce && !ie) ev |= 1u << e;
          }
        }
        if (s) bits |= 1u << e;
      }
      if (mk && ev) mk[wi] |= ev;
    }
    int total;
    int pos = running + block_exclusive_scan<NT>(__popc(bits), L.scan, &total);
    while (bits) {
      const int e = __ffs(bits) - 1;
      bits &= bits - 1;
      if (pos < max_sel) out[pos] = wi * 32 + e;
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

hipError_t launch_topk(const fx_plan* p, const float* scores, const float* logits, uint32_t* mask,
                       const int32_t* seq_lens, int32_t* sel_idx, int32_t* sel_cnt,
                       hipStream_t stream) {
  k_topk<<<dim3((unsigned)p->units), NT, 0, stream>>>(p->d_units, scores, logits, mask, seq_lens,
                                                      sel_idx, sel_cnt, p->d_error,
                                                      p->desc.num_kv_heads, p->desc.t_cap,
                                                      p->max_sel);
  return hipGetLastError();
}

}  // namespace fx
