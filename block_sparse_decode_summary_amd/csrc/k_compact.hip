// Delta-driven compaction: the selected full blocks of each unit kept in an array of
// block slots, moved by set difference.
//
// [NOSA-DE] "Technisches Resümee: NOSA: Native und Offloadable Sparse Attention",
// Methodik §2 (NOSI), bullet "Optimierte Speicherlayout": the KV cache is held in
// minimal block units, and the set difference between what is selected and what is
// held decides which blocks are swapped, so no contiguous allocation is needed.
//
// Per unit, with `target` the selected full blocks (ascending) and `slots` the block
// held by each slot (-1 = free):
//   1. a slot whose block is not in target is freed;
//   2. the target blocks no slot holds ("added", ascending) take the free slots in
//      ascending slot order, the i-th added block the i-th free slot;
//   3. each added block's g key rows and g value rows are copied into its slot.
// Held blocks never move.  The growing partial last block is never held.
//
// k_compact_plan: one wave per unit.  The target list, the slot row, a held flag per
// target and the added / free lists live in LDS (at most kMaxCompactSlots entries
// each); membership is a binary search in the ascending target list, and ballots keep
// every list in order.  It rewrites the slot row and leaves the (slot, block) moves and
// their count in the workspace.
// k_compact_copy: kCopyGroups workgroups per unit share its moves (move k goes to
// group k mod kCopyGroups); a move is two contiguous spans of g*d elements (K, then V),
// copied with 16-byte loads, kCopyUnroll of each per thread in flight before the stores.
#include "fx_device.h"

namespace fx {
namespace {

constexpr int NT = 256;
constexpr int kCopyGroups = 8;
constexpr int kCopyUnroll = 4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int find_sorted(const int* a, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    const int v = a[mid];
    if (v < x) lo = mid + 1;
    else if (v > x) hi = mid;
    else return mid;
  }
  return -1;
}

struct CompactLds {
  int tgt[kMaxCompactSlots];
  int slot[kMaxCompactSlots];
  int held[kMaxCompactSlots];
  int added[kMaxCompactSlots];
  int freed[kMaxCompactSlots];
};

// One wave per unit: lists are compacted 64 entries at a time with a ballot and the
// lanes' popcount below them, so no workgroup scan (and no barrier) is needed for them.
__global__ __launch_bounds__(64) void k_compact_plan(
    const UnitInfo* __restrict__ units, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ sel_cnt,
    int32_t* __restrict__ slot_map, int2* __restrict__ moves, int32_t* __restrict__ move_cnt,
    int32_t* __restrict__ moved_out, uint32_t* __restrict__ err, int Hkv, int t_cap,
    int max_sel) {
  __shared__ CompactLds L;
  const int u = blockIdx.x;
  const int lane = threadIdx.x;
  const UnitInfo ui = units[u];
  const int T = load_seq_len(seq_lens, u / Hkv, t_cap, err);
  const int n_full = T >> ui.log2g;
  const int n_tot = (T + ui.g - 1) >> ui.log2g;
  const int nslot = ui.max_sel;   // slots of this unit (<= max_sel, the row stride)
  int cnt = sel_cnt[u];
  if (cnt < 0 || cnt > max_sel) {
    if (lane == 0) atomicOr(err, (uint32_t)FX_ERR_SEL_COUNT);
    cnt = min(max(cnt, 0), max_sel);
  }
  const int32_t* sel = sel_idx + (size_t)u * max_sel;
  int32_t* row = slot_map + (size_t)u * max_sel;

  // 0. Stage the selection (in `added`) and the slot row with independent loads.
#pragma unroll 4
  for (int i = lane; i < cnt; i += 64) L.added[i] = sel[i];
#pragma unroll 4
  for (int s = lane; s < nslot; s += 64) L.slot[s] = row[s];
  __syncthreads();

  // 1. The target list: valid, ascending entries that are full blocks.
  int nt = 0;
  for (int base = 0; base < cnt; base += 64) {
    const int i = base + lane;
    int b = -1;
    bool keep = false;
    if (i < cnt) {
      b = L.added[i];
      const bool ok = b >= 0 && b < n_tot && (i == 0 || L.added[i - 1] < b);
      if (!ok) atomicOr(err, (uint32_t)FX_ERR_SEL_INDEX);
      keep = ok && b < n_full;
    }
    const uint64_t m = __ballot(keep);
    const int pos = nt + (int)lanes_below(m);
    if (keep && pos < nslot) L.tgt[pos] = b;
    nt += __popcll(m);
  }
  if (nt > nslot) {              // more selected full blocks than slots: hold the first ones
    if (lane == 0) atomicOr(err, (uint32_t)FX_ERR_SEL_COUNT);
    nt = nslot;
  }
  for (int i = lane; i < nt; i += 64) L.held[i] = 0;
  __syncthreads();

  // 2. Free the slots whose block left the target; flag the targets still held.
  for (int s = lane; s < nslot; s += 64) {
    const int b = L.slot[s];
    const int i = b >= 0 ? find_sorted(L.tgt, nt, b) : -1;
    if (i >= 0) L.held[i] = 1;
    else L.slot[s] = -1;
  }
  __syncthreads();

  // 3. Added targets and free slots, both in ascending order.
  int na = 0, nf = 0;
  for (int base = 0; base < nt; base += 64) {
    const int i = base + lane;
    const bool a = i < nt && !L.held[i];
    const uint64_t m = __ballot(a);
    if (a) L.added[na + (int)lanes_below(m)] = L.tgt[i];
    na += __popcll(m);
  }
  for (int base = 0; base < nslot; base += 64) {
    const int s = base + lane;
    const bool f = s < nslot && L.slot[s] < 0;
    const uint64_t m = __ballot(f);
    if (f) L.freed[nf + (int)lanes_below(m)] = s;
    nf += __popcll(m);
  }
  __syncthreads();

  // 4. Place the added blocks; record the moves in slot order of the free list.  With a
  // valid slot row na <= nf (the targets fit in the slots); a row holding one block
  // twice can break that, and the blocks without a slot are then not held.
  if (na > nf) {
    if (lane == 0) atomicOr(err, (uint32_t)FX_ERR_SLOT_MAP);
    na = nf;
  }
  int2* mv = moves + (size_t)u * max_sel;
  for (int k = lane; k < na; k += 64) {
    const int s = L.freed[k];
    L.slot[s] = L.added[k];
    mv[k] = make_int2(s, L.added[k]);
  }
  __syncthreads();
  for (int s = lane; s < nslot; s += 64) row[s] = L.slot[s];
  if (lane == 0) {
    move_cnt[u] = na;
    if (moved_out) moved_out[u] = na;
  }
}

template <typename E>
__global__ __launch_bounds__(NT) void k_compact_copy(
    const UnitInfo* __restrict__ units, const E* __restrict__ K, const E* __restrict__ V,
    const int2* __restrict__ moves, const int32_t* __restrict__ move_cnt,
    E* __restrict__ work_K, E* __restrict__ work_V, int t_cap, int d, int max_sel) {
  const int u = blockIdx.x / kCopyGroups, grp = blockIdx.x % kCopyGroups;
  const int n = move_cnt[u];
  if (grp >= n) return;
  const UnitInfo ui = units[u];
  const int g = ui.g;
  const size_t span = (size_t)g * d * sizeof(E) / 16;   // 16-byte pieces per block of K (or V)
  const int2* mv = moves + (size_t)u * max_sel;
  for (int k = grp; k < n; k += kCopyGroups) {
    const int2 m = mv[k];
    const size_t src = ((size_t)u * t_cap + (size_t)m.y * g) * d;
    const size_t dst = ((size_t)ui.work_off + (size_t)m.x * g) * d;
    const u32x4* sk = reinterpret_cast<const u32x4*>(K + src);
    const u32x4* sv = reinterpret_cast<const u32x4*>(V + src);
    u32x4* dk = reinterpret_cast<u32x4*>(work_K + dst);
    u32x4* dv = reinterpret_cast<u32x4*>(work_V + dst);
    // All of a thread's loads first (read once: nontemporal), then its stores.
    for (size_t i0 = threadIdx.x; i0 < span; i0 += (size_t)NT * kCopyUnroll) {
      u32x4 a[kCopyUnroll], b[kCopyUnroll];
#pragma unroll
      for (int j = 0; j < kCopyUnroll; ++j) {
        const size_t i = i0 + (size_t)j * NT;
        if (i < span) {
          a[j] = __builtin_nontemporal_load(sk + i);
          b[j] = __builtin_nontemporal_load(sv + i);
        }
      }
#pragma unroll
      for (int j = 0; j < kCopyUnroll; ++j) {
        const size_t i = i0 + (size_t)j * NT;
        if (i < span) {
          dk[i] = a[j];
          dv[i] = b[j];
        }
      }
    }
  }
}

}  // namespace

int launch_compact(const fx_plan* p, const void* K, const void* V, const int32_t* seq_lens,
                   const int32_t* sel_idx, const int32_t* sel_cnt, int32_t* slot_map,
                   void* work_K, void* work_V, int32_t* moved_cnt, void* moves_raw,
                   int32_t* move_cnt, hipStream_t stream) {
  int2* moves = static_cast<int2*>(moves_raw);
  k_compact_plan<<<dim3((unsigned)p->units), 64, 0, stream>>>(
      p->d_units, seq_lens, sel_idx, sel_cnt, slot_map, moves, move_cnt, moved_cnt, p->d_error,
      p->desc.num_kv_heads, p->desc.t_cap, p->max_sel);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((int64_t)p->units * kCopyGroups));
  if (p->desc.dtype == FX_BF16)
    k_compact_copy<bf16_t><<<grid, NT, 0, stream>>>(
        p->d_units, static_cast<const bf16_t*>(K), static_cast<const bf16_t*>(V), moves, move_cnt,
        static_cast<bf16_t*>(work_K), static_cast<bf16_t*>(work_V), p->desc.t_cap,
        p->desc.head_dim, p->max_sel);
  else
    k_compact_copy<float><<<grid, NT, 0, stream>>>(
        p->d_units, static_cast<const float*>(K), static_cast<const float*>(V), moves, move_cnt,
        static_cast<float*>(work_K), static_cast<float*>(work_V), p->desc.t_cap,
        p->desc.head_dim, p->max_sel);
  return hipGetLastError();
}

}  // namespace fx
