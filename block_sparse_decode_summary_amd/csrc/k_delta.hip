// Selection set differences between consecutive decode steps.
//
// [NOSA-DE] "Technisches Resümee: NOSA: Native und Offloadable Sparse Attention",
// Methodik §2, bullet "Optimierte Speicherlayout": the KV cache is kept in minimal
// block units and set differences between selections decide which blocks to swap;
// Methodik §1, "Lokalitätsgarantie": consecutive selections overlap by at least
// k_e / k.
//
// Per unit: added = cur \ prev, removed = prev \ cur, both ascending, padded with -1.
// A list enters as its longest prefix that is strictly ascending within the unit's block
// slots [0, n_cap); entries past that prefix are ignored and flagged (FX_ERR_SEL_INDEX),
// so both lists the differences are formed from are ascending.  One 256-thread
// workgroup per unit; each element of one list binary-searches the other, and a
// workgroup prefix sum compacts the survivors in order.
#include "fx_device.h"

namespace fx {
namespace {

constexpr int NT = 256;

__device__ __forceinline__ bool contains(const int32_t* a, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    const int v = a[mid];
    if (v < x) lo = mid + 1;
    else if (v > x) hi = mid;
    else return true;
  }
  return false;
}

// Lowers *first_bad to the index of every entry of a[0 .. n) that is outside [0, lim) or
// not above its predecessor; after the caller's next barrier *first_bad is the length of
// the longest valid prefix (or stays n).
__device__ __forceinline__ void mark_invalid(const int32_t* a, int n, int lim, int* first_bad) {
  for (int i = threadIdx.x; i < n; i += NT) {
    const int x = a[i];
    const bool ok = x >= 0 && x < lim && (i == 0 || a[i - 1] < x);
    if (!ok) atomicMin(first_bad, i);
  }
}

__device__ void difference(const int32_t* a, int na, const int32_t* b, int nb, int32_t* out,
                           int32_t* out_cnt, int max_sel, int* lds) {
  int running = 0;
  for (int base = 0; base < na; base += NT) {
    const int i = base + (int)threadIdx.x;
    int x = 0;
    const int keep = (i < na && !contains(b, nb, x = a[i])) ? 1 : 0;
    int total;
    const int pos = running + block_exclusive_scan<NT>(keep, lds, &total);
    if (keep) out[pos] = x;
    running += total;
  }
  for (int i = running + (int)threadIdx.x; i < max_sel; i += NT) out[i] = -1;
  if (threadIdx.x == 0) *out_cnt = running;
}

__global__ __launch_bounds__(NT) void k_delta(const UnitInfo* __restrict__ units,
                                              const int32_t* __restrict__ prev_idx,
                                              const int32_t* __restrict__ prev_cnt,
                                              const int32_t* __restrict__ cur_idx,
                                              const int32_t* __restrict__ cur_cnt,
                                              int32_t* __restrict__ added, int32_t* __restrict__ added_cnt,
                                              int32_t* __restrict__ removed,
                                              int32_t* __restrict__ removed_cnt,
                                              uint32_t* __restrict__ err, int max_sel) {
  __shared__ int lds[NT / 64];
  __shared__ int first_bad[2];
  const int u = blockIdx.x;
  const int n_cap = units[u].n_cap;
  int np = prev_cnt[u], nc = cur_cnt[u];
  if (np < 0 || np > max_sel || nc < 0 || nc > max_sel) {
    if (threadIdx.x == 0) atomicOr(err, (uint32_t)FX_ERR_SEL_COUNT);
    np = min(max(np, 0), max_sel);
    nc = min(max(nc, 0), max_sel);
  }
  if (threadIdx.x == 0) {
    first_bad[0] = np;
    first_bad[1] = nc;
  }
  __syncthreads();
  const size_t off = (size_t)u * max_sel;
  mark_invalid(prev_idx + off, np, n_cap, &first_bad[0]);
  mark_invalid(cur_idx + off, nc, n_cap, &first_bad[1]);
  __syncthreads();
  const int vp = first_bad[0], vc = first_bad[1];
  if (threadIdx.x == 0 && (vp < np || vc < nc)) atomicOr(err, (uint32_t)FX_ERR_SEL_INDEX);
  difference(cur_idx + off, vc, prev_idx + off, vp, added + off, added_cnt + u, max_sel, lds);
  difference(prev_idx + off, vp, cur_idx + off, vc, removed + off, removed_cnt + u, max_sel, lds);
}

}  // namespace

int launch_delta(const fx_plan* p, const int32_t* prev_idx, const int32_t* prev_cnt,
                        const int32_t* cur_idx, const int32_t* cur_cnt, int32_t* added,
                        int32_t* added_cnt, int32_t* removed, int32_t* removed_cnt,
                        hipStream_t stream) {
  k_delta<<<dim3((unsigned)p->units), NT, 0, stream>>>(p->d_units, prev_idx, prev_cnt, cur_idx,
                                                       cur_cnt, added, added_cnt, removed,
                                                       removed_cnt, p->d_error, p->max_sel);
  return hipGetLastError();
}

}  // namespace fx
