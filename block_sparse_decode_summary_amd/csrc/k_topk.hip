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
// Mapping: one NT-thread workgroup per unit (NT = 256; 512 for the selection that forms
// its own scores when units have 257-512 block slots, and for plans of many units with
// 1025-4096 block slots; 1024 for plans with few units and more than 1024 block slots).  Thread t owns blocks j = i*NT + t.  When every
// unit has at most 8192 block slots the keys, the candidate flags and the old eviction
// words stay in registers (k_topk_reg), wave ballots of the per-block flags give the
// bitmap words, and a scan over (row, wave) counts compacts the selection straight into
// sel_idx in ascending order; with a previous selection (fx_select_delta) the added and
// removed lists are compacted the same way.  Larger units keep keys and bitmaps in the
// workspace (k_topk_mem, 256 threads), with the same selection arithmetic.
//
// Plans whose units have at most 512 block slots and key-side summaries of at most 256
// bytes per row skip the separate scoring kernel: k_select_fused forms each unit's scores
// in its own selection workgroup (wave w scores blocks 64w .. 64w+63, each lane one
// block, into the register the selection reads), with the float64 chain of k_score_sum,
// so the scores are the same bits.  Larger units keep k_score_sum: one CU streams a unit's
// summaries far more slowly than the whole GPU scoring its tiles in parallel.
#include <climits>
#include <type_traits>

#include "fx_score_tile.h"

namespace fx {

// 256 threads per unit, with the workspace path for units of more than 8192 block slots.
namespace topk256 {
constexpr int NT = 256;
#define FX_TOPK_WORKSPACE_PATH 1
#include "k_topk_body.inc"
#undef FX_TOPK_WORKSPACE_PATH
}  // namespace topk256

// 512 threads per unit: the selection that forms its own scores for units of 257-512 block
// slots (one 64-block tile per wave).
namespace topk512 {
constexpr int NT = 512;
#define FX_TOPK_WORKSPACE_PATH 0
#include "k_topk_body.inc"
#undef FX_TOPK_WORKSPACE_PATH
}  // namespace topk512

// 1024 threads per unit: plans with few units, whose selections would otherwise run on a
// few CUs with many blocks per thread.
namespace topk1024 {
constexpr int NT = 1024;
#define FX_TOPK_WORKSPACE_PATH 0
#include "k_topk_body.inc"
#undef FX_TOPK_WORKSPACE_PATH
}  // namespace topk1024

namespace {

// Units below which a plan cannot fill the GPU with one 256-thread workgroup each; such
// plans with large units take 1024 threads per unit.
constexpr int kFewUnits = 128;

template <int NTW, class DA, class LaunchReg>
int dispatch_reg(int n, const DA& D, LaunchReg&& launch) {
  // n <= kTopkRegBlocks here, so KPT * NTW never exceeds it.
  if (n <= 1 * NTW) launch(std::integral_constant<int, 1>{}, D);
  else if (n <= 2 * NTW) launch(std::integral_constant<int, 2>{}, D);
  else if (n <= 4 * NTW) launch(std::integral_constant<int, 4>{}, D);
  else if constexpr (8 * NTW >= kTopkRegBlocks) launch(std::integral_constant<int, 8>{}, D);
  else if (n <= 8 * NTW) launch(std::integral_constant<int, 8>{}, D);
  else if (n <= 16 * NTW) launch(std::integral_constant<int, 16>{}, D);
  else launch(std::integral_constant<int, 32>{}, D);
  return hipGetLastError();
}

// Summary element type and head dim of the fused kernel (rows of at most 256 bytes).
template <class F>
int by_element(const fx_plan* p, F&& f) {
  if (p->desc.dtype == FX_BF16) {
    if (p->desc.head_dim == 128) f(bf16_t{}, std::integral_constant<int, 128>{});
    else f(bf16_t{}, std::integral_constant<int, 64>{});
  } else {
    f(float{}, std::integral_constant<int, 64>{});
  }
  return hipGetLastError();
}

}  // namespace

int launch_select_fused(const fx_plan* p, const void* q, const void* summaries,
                               float* scores, const float* logits, uint32_t* mask,
                               const int32_t* seq_lens, int32_t* sel_idx, int32_t* sel_cnt,
                               const int32_t* prev_idx, const int32_t* prev_cnt, int32_t* added,
                               int32_t* added_cnt, int32_t* removed, int32_t* removed_cnt,
                               hipStream_t stream) {
  const int n = p->max_n_cap;
  if (n <= topk256::NT) {
    const topk256::DeltaArgs D{prev_idx, prev_cnt, added, added_cnt, removed, removed_cnt};
    return by_element(p, [&](auto e, auto dim) {
      topk256::launch_fused<1, decltype(e), decltype(dim)::value>(
          p, q, summaries, scores, logits, mask, seq_lens, sel_idx, sel_cnt, D, stream);
    });
  }
  if (n <= topk512::NT) {
    const topk512::DeltaArgs D{prev_idx, prev_cnt, added, added_cnt, removed, removed_cnt};
    return by_element(p, [&](auto e, auto dim) {
      topk512::launch_fused<1, decltype(e), decltype(dim)::value>(
          p, q, summaries, scores, logits, mask, seq_lens, sel_idx, sel_cnt, D, stream);
    });
  }
  return hipErrorInvalidValue;   // select_fused() admits no larger units
}

int launch_topk(const fx_plan* p, const float* scores, const float* logits, uint32_t* mask,
                       const int32_t* seq_lens, int32_t* sel_idx, int32_t* sel_cnt,
                       uint32_t* ws_keys, uint32_t* ws_bits, const int32_t* prev_idx,
                       const int32_t* prev_cnt, int32_t* added, int32_t* added_cnt,
                       int32_t* removed, int32_t* removed_cnt, hipStream_t stream) {
  const int n = p->max_n_cap;
  if (n > kTopkRegBlocks) {
    topk256::k_topk_mem<<<dim3((unsigned)p->units), topk256::NT, 0, stream>>>(
        p->d_units, scores, logits, mask, seq_lens, sel_idx, sel_cnt, p->d_error, ws_keys, ws_bits,
        p->desc.num_kv_heads, p->desc.t_cap, p->max_sel);
    const int e = hipGetLastError();
    if (e != 0 || !prev_idx) return e;
    // The workspace path leaves the differences to the delta kernel.
    return launch_delta(p, prev_idx, prev_cnt, sel_idx, sel_cnt, added, added_cnt, removed,
                        removed_cnt, stream);
  }
  if (p->units >= kFewUnits && n > 2 * topk512::NT && n <= 8 * topk512::NT) {
    // 1025-4096 block slots: 512 threads per unit (4 or 8 blocks per thread) halve the
    // per-thread serial parts of the k-th search against 256 (mixed_serving, 2048 slots:
    // k_topk_reg 8.1 against 9.0 us).
    const topk512::DeltaArgs D{prev_idx, prev_cnt, added, added_cnt, removed, removed_cnt};
    if (n <= 4 * topk512::NT)
      topk512::launch_reg<4>(p, scores, logits, mask, seq_lens, sel_idx, sel_cnt, D, stream);
    else
      topk512::launch_reg<8>(p, scores, logits, mask, seq_lens, sel_idx, sel_cnt, D, stream);
    return hipGetLastError();
  }
  if (p->units < kFewUnits && n > topk1024::NT) {
    const topk1024::DeltaArgs D{prev_idx, prev_cnt, added, added_cnt, removed, removed_cnt};
    return dispatch_reg<topk1024::NT>(n, D, [&](auto kpt, const topk1024::DeltaArgs& d) {
      topk1024::launch_reg<decltype(kpt)::value>(p, scores, logits, mask, seq_lens, sel_idx,
                                                 sel_cnt, d, stream);
    });
  }
  const topk256::DeltaArgs D{prev_idx, prev_cnt, added, added_cnt, removed, removed_cnt};
  return dispatch_reg<topk256::NT>(n, D, [&](auto kpt, const topk256::DeltaArgs& d) {
    topk256::launch_reg<decltype(kpt)::value>(p, scores, logits, mask, seq_lens, sel_idx, sel_cnt,
                                              d, stream);
  });
}

}  // namespace fx
