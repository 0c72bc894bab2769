// libfx host side: plan creation, argument validation, workspace layout, entry points.
//
// Everything here runs on the host and is plain C++ (no HIP header): the device calls
// go through the fx::dev_* functions and the kernel launchers of the .hip files.
// Validation happens before any device call, so the error paths work (and are tested,
// with stand-ins for those functions and under the address and undefined-behaviour
// sanitizers) on machines without a GPU.  No C++ exception leaves this file: every
// entry point catches and maps to a status.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>
#include <new>

#include "fx_plan.h"

namespace {

using fx::UnitInfo;

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int log2i(int64_t x) {
  int r = 0;
  while ((int64_t(1) << r) < x) ++r;
  return r;
}
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool req(const void* p, size_t a) { return p != nullptr && aligned(p, a); }
bool opt(const void* p, size_t a) { return p == nullptr || aligned(p, a); }

fx_status check_desc(const fx_plan_desc* d) {
  if (!d) return FX_E_INVALID;
  if (d->batch < 1 || d->num_kv_heads < 1 || d->num_q_heads < 1) return FX_E_INVALID;
  if (d->num_q_heads % d->num_kv_heads != 0) return FX_E_INVALID;
  const int G = d->num_q_heads / d->num_kv_heads;
  if (G < 1 || G > fx::kMaxGroup) return FX_E_INVALID;
  if (d->head_dim != 64 && d->head_dim != 128) return FX_E_INVALID;
  if (d->t_cap < 1 || d->t_cap > fx::kMaxTcap) return FX_E_INVALID;
  if (d->dtype != FX_F32 && d->dtype != FX_BF16) return FX_E_INVALID;
  if (d->split_tokens != 0 &&
      (!is_pow2(d->split_tokens) || d->split_tokens < fx::kMinSplit ||
       d->split_tokens > fx::kMaxSplit))
    return FX_E_INVALID;
  if ((int64_t)d->batch * d->num_kv_heads > (1 << 20)) return FX_E_INVALID;
  if (d->pooling != FX_POOL_KEY && d->pooling != FX_POOL_SCORE_SUM &&
      d->pooling != FX_POOL_SCORE_MAX)
    return FX_E_INVALID;
  // One unit's K (or V) rows are addressed with 32-bit byte offsets below 2^31.
  const int64_t unit_bytes = (int64_t)d->t_cap * d->head_dim * (d->dtype == FX_BF16 ? 2 : 4);
  if (unit_bytes > 0x7FFFFFFF) return FX_E_UNSUPPORTED;
  return FX_OK;
}

fx_status check_policy(const fx_head_policy& p) {
  if (p.mode != FX_RETRIEVAL && p.mode != FX_STREAMING && p.mode != FX_NOSA) return FX_E_INVALID;
  if (!is_pow2(p.block) || p.block > fx::kMaxBlock) return FX_E_INVALID;
  if (!is_pow2(p.sub_block) || p.sub_block > p.block) return FX_E_INVALID;
  if ((p.force_sink != 0 && p.force_sink != 1) || (p.force_last != 0 && p.force_last != 1))
    return FX_E_INVALID;
  switch (p.mode) {
    case FX_RETRIEVAL:
      if (p.top_k < 0) return FX_E_INVALID;
      if (p.top_k == 0 && !(p.budget > 0.0f && p.budget <= 1.0f)) return FX_E_INVALID;
      break;
    case FX_STREAMING:
      if (p.sink_tokens < 0 || p.local_tokens < 0) return FX_E_INVALID;
      break;
    case FX_NOSA:
      if (p.top_k < 0 || p.k_evict < 0 || (int64_t)p.top_k + p.k_evict < 1) return FX_E_INVALID;
      break;
  }
  return FX_OK;
}

// Largest selection a unit can produce for any seq_len <= t_cap.
int64_t max_selected(const fx_head_policy& p, int64_t n_cap) {
  int64_t m;
  switch (p.mode) {
    case FX_STREAMING:
      m = ceil_div(p.sink_tokens, p.block) + ceil_div(p.local_tokens, p.block) + 2;
      break;
    case FX_RETRIEVAL: {
      const int64_t k = p.top_k > 0 ? p.top_k
                                    : (int64_t)std::ceil((double)p.budget * (double)n_cap);
      m = k + 2;
      break;
    }
    default:
      m = (int64_t)p.top_k + p.k_evict + 2;
  }
  return std::min(m, n_cap);
}

}  // namespace

namespace fx {

// The selection keeps keys, candidate flags and old eviction words in registers when
// every unit has at most kTopkRegBlocks block slots; larger units use the workspace.
bool topk_in_registers(const fx_plan* p) { return p->max_n_cap <= kTopkRegBlocks; }

// Scores and selection in one kernel: key-side summaries, summary rows of at most 256
// bytes (a wave's 64-row tile then fits in 64 registers per lane) and at most
// kFusedSelectBlocks block slots per unit (one 64-block tile per wave, 256 threads per
// unit up to 256 block slots, else 512).  Larger units keep the separate scoring kernel:
// one CU cannot stream a large unit's summaries as fast as the whole GPU scoring it tile
// by tile.
bool select_fused(const fx_plan* p) {
  const int row_bytes = p->desc.head_dim * (p->desc.dtype == FX_BF16 ? 2 : 4);
  return p->any_scored && p->desc.pooling == FX_POOL_KEY && row_bytes <= 256 &&
         p->max_n_cap <= kFusedSelectBlocks;
}

}  // namespace fx

namespace {

// Decode partials for `grid` segments: a head and a tail piece per segment.
fx::DecodeScratch decode_scratch_layout(int64_t grid, int G, int d) {
  fx::DecodeScratch s;
  const size_t slots = (size_t)grid * 2;
  s.part_o = 0;
  s.part_ml = align_up(slots * G * d * 4, 256);
  s.seg = s.part_ml + align_up(slots * G * 8, 256);
  s.end = s.seg + align_up((size_t)grid * 8, 256);
  return s;
}

fx_status plan_create(const fx_plan_desc* desc, const fx_head_policy* pol, fx_plan_t* out) {
  if (!out) return FX_E_INVALID;
  fx_status st = check_desc(desc);
  if (st != FX_OK) return st;
  if (!pol) return FX_E_INVALID;
  const int units = desc->batch * desc->num_kv_heads;
  for (int u = 0; u < units; ++u) {
    st = check_policy(pol[u]);
    if (st != FX_OK) return st;
  }
  if (desc->pooling != FX_POOL_KEY)
    for (int u = 0; u < units; ++u)
      if (pol[u].block / pol[u].sub_block > fx::kMaxScoreRows) return FX_E_UNSUPPORTED;

  fx_plan* p = new (std::nothrow) fx_plan();
  if (!p) return FX_E_HIP;
  p->desc = *desc;
  p->G = desc->num_q_heads / desc->num_kv_heads;
  p->units = units;
  p->host_units.resize(units);
  int64_t boff = 0, soff = 0, woff = 0, moff = 0, max_sel = 1, max_ncap = 0, max_nfull = 0;
  for (int u = 0; u < units; ++u) {
    const fx_head_policy& q = pol[u];
    UnitInfo& ui = p->host_units[u];
    const int64_t n_cap = ceil_div(desc->t_cap, q.block);
    ui.mode = q.mode;
    ui.g = q.block;
    ui.log2g = log2i(q.block);
    ui.s = q.sub_block;
    ui.top_k = q.top_k;
    ui.budget = q.budget;
    ui.k_evict = q.k_evict;
    ui.sink = q.sink_tokens;
    ui.local = q.local_tokens;
    ui.force_sink = q.force_sink;
    ui.force_last = q.force_last;
    const int64_t ms = max_selected(q, n_cap);
    ui.max_sel = (int32_t)ms;
    ui.n_cap = (int32_t)n_cap;
    ui.mask_off = (int32_t)moff;
    ui.block_off = boff;
    ui.log2r = desc->pooling == FX_POOL_KEY ? 0 : log2i(q.block / q.sub_block);
    ui.reserved = 0;
    ui.sum_off = soff;
    ui.work_off = woff;
    boff += n_cap;
    soff += n_cap << ui.log2r;
    woff += ms * q.block;
    moff += ceil_div(n_cap, 32);
    max_sel = std::max(max_sel, ms);
    max_ncap = std::max(max_ncap, n_cap);
    max_nfull = std::max<int64_t>(max_nfull, desc->t_cap / q.block);
    if (q.mode != FX_STREAMING) {
      p->any_scored = true;
      p->host_scored.push_back(u);
      p->max_scored_n_full_cap =
          std::max<int32_t>(p->max_scored_n_full_cap, (int32_t)(desc->t_cap / q.block));
      p->max_scored_rows_cap = std::max<int32_t>(
          p->max_scored_rows_cap, (int32_t)((desc->t_cap / q.block) << ui.log2r));
    }
    if (q.mode == FX_NOSA && q.k_evict > 0) p->needs_logits = true;
    if (q.mode == FX_NOSA) p->any_nosa = true;
  }
  if (moff > INT32_MAX || max_sel > INT32_MAX / 2) {
    delete p;
    return FX_E_UNSUPPORTED;
  }
  p->total_blocks = boff;
  p->summary_rows = soff;
  p->work_rows = woff;
  p->mask_words = moff;
  p->max_sel = (int32_t)max_sel;
  p->max_n_cap = (int32_t)max_ncap;
  p->max_n_full_cap = (int32_t)max_nfull;

  // The decode lays the token slots of every unit's selected blocks end to end and indexes
  // them with 32-bit integers.  A valid list of unit u has at most min(n_cap(u), max_sel)
  // blocks (max_sel being the lists' row stride), and the decode clamps counts to that.
  int64_t slots = 0;
  for (const UnitInfo& ui : p->host_units) slots += std::min<int64_t>(ui.n_cap, max_sel) * ui.g;
  if (slots > INT32_MAX) {
    delete p;
    return FX_E_UNSUPPORTED;
  }
  p->split = desc->split_tokens != 0 ? desc->split_tokens : fx::kAutoSplit;
  p->decode_grid = fx::decode_grid(p, false);
  p->decode_grid_ed = std::min(fx::decode_grid(p, true), p->decode_grid);
  if (p->decode_grid <= 0 || p->decode_grid_ed <= 0) {
    delete p;
    return FX_E_HIP;
  }
  // With the automatic split, plans whose units all fit a short piece keep every unit
  // whole: the decode cuts each unit into its own pieces (few units on a large grid, the
  // kernel's unit-aligned rule), each at least decode_split slots long, so a minimum as
  // large as the longest possible unit leaves one piece per unit and nothing to merge.
  // A second kernel's launch and round trips cost more than streaming such a unit in
  // one workgroup (the tiny workload's 320-slot units).
  p->decode_split = p->split;
  {
    int64_t max_unit_slots = 0;
    for (const UnitInfo& ui : p->host_units)
      max_unit_slots = std::max<int64_t>(max_unit_slots, std::min<int64_t>(ui.n_cap, max_sel) * ui.g);
    auto aligned_on = [&](int grid) {
      return grid >= 2 * fx::kCUsMin && (int64_t)units * fx::kAlignedUnitsDiv <= grid / 2;
    };
    if (desc->split_tokens == 0 && max_unit_slots <= fx::kUncutSlots &&
        aligned_on(p->decode_grid) && aligned_on(p->decode_grid_ed)) {
      p->decode_uncut = true;
      p->decode_split = std::max<int32_t>(p->split, (int32_t)max_unit_slots);
    }
  }

  const int d = desc->head_dim;
  size_t off = 0;
  p->ws_scores_off = off;
  off += align_up((size_t)(p->any_scored ? p->total_blocks : 0) * 4, 256);
  const bool topk_regs = fx::topk_in_registers(p);
  p->ws_keys_off = off;
  off += align_up(topk_regs ? 0 : (size_t)p->total_blocks * 4, 256);
  p->ws_bits_off = off;
  off += align_up(topk_regs ? 0 : (size_t)p->mask_words * 3 * 4, 256);
  p->ws_decode = decode_scratch_layout(p->decode_grid, p->G, d);
  p->ws_decode_off = off;
  off += p->ws_decode.end;
  p->ws_moves_off = off;
  off += align_up((size_t)units * p->max_sel * 8, 256);
  p->ws_move_cnt_off = off;
  off += align_up((size_t)units * 4, 256);
  p->ws_total = std::max<size_t>(off, 256);

  // Device table: units | error word | scored unit ids | every unit id, scored first.
  const size_t tab_units = align_up(sizeof(UnitInfo) * units, 256);
  p->n_scored = (int32_t)p->host_scored.size();
  const size_t tab_scored = align_up(sizeof(int32_t) * p->host_scored.size(), 256);
  const size_t tab_bytes = tab_units + 256 + tab_scored + align_up(sizeof(int32_t) * units, 256);
  std::vector<int32_t> host_order(p->host_scored);
  for (int32_t u = 0; u < units; ++u)
    if (p->host_units[u].mode == FX_STREAMING) host_order.push_back(u);
  if (fx::dev_current(&p->device) != 0 || fx::dev_alloc(&p->d_table, tab_bytes) != 0) {
    delete p;
    return FX_E_HIP;
  }
  char* base = static_cast<char*>(p->d_table);
  p->d_units = reinterpret_cast<UnitInfo*>(base);
  p->d_error = reinterpret_cast<uint32_t*>(base + tab_units);
  p->d_scored = reinterpret_cast<int32_t*>(base + tab_units + 256);
  p->d_order = reinterpret_cast<int32_t*>(base + tab_units + 256 + tab_scored);
  if (fx::dev_upload(p->d_units, p->host_units.data(), sizeof(UnitInfo) * units) != 0 ||
      fx::dev_upload(p->d_order, host_order.data(), sizeof(int32_t) * units) != 0 ||
      (p->n_scored > 0 &&
       fx::dev_upload(p->d_scored, p->host_scored.data(), sizeof(int32_t) * p->n_scored) != 0) ||
      fx::dev_zero(base + tab_units, 256) != 0) {
    (void)fx::dev_free(p->d_table);
    delete p;
    return FX_E_HIP;
  }
  // The no-allocation decode's scratch: the plan device's static array (looked up once
  // per device, here at set-up, never in the entry point).
  size_t scratch_bytes = 0;
  p->static_scratch = fx::dev_static_scratch(&scratch_bytes);
  p->static_scratch_fits = p->static_scratch != nullptr && p->ws_decode.end <= scratch_bytes;
  *out = p;
  return FX_OK;
}

fx_status hip_status(int e) { return e == 0 ? FX_OK : FX_E_HIP; }

}  // namespace

extern "C" {

fx_status fx_plan_create(const fx_plan_desc* desc, const fx_head_policy* host_policies,
                         fx_plan_t* out) {
  try {
    return plan_create(desc, host_policies, out);
  } catch (...) {
    return FX_E_HIP;
  }
}

fx_status fx_plan_destroy(fx_plan_t plan) {
  if (!plan) return FX_OK;
  fx_status st = FX_OK;
  if (plan->d_table && fx::dev_free(plan->d_table) != 0) st = FX_E_HIP;
  delete plan;
  return st;
}

size_t fx_summary_bytes(fx_plan_t p) {
  if (!p) return 0;
  return (size_t)p->summary_rows * p->desc.head_dim * (p->desc.dtype == FX_BF16 ? 2 : 4);
}
size_t fx_logits_bytes(fx_plan_t p) { return p ? (size_t)p->total_blocks * 4 : 0; }
size_t fx_evict_mask_bytes(fx_plan_t p) { return p ? (size_t)p->mask_words * 4 : 0; }
size_t fx_workspace_bytes(fx_plan_t p) { return p ? p->ws_total : 0; }
int32_t fx_max_selected(fx_plan_t p) { return p ? p->max_sel : -1; }
int32_t fx_split_tokens(fx_plan_t p) { return p ? p->split : -1; }
int64_t fx_unit_block_offset(fx_plan_t p, int32_t unit) {
  if (!p || unit < 0 || unit >= p->units) return -1;
  return p->host_units[unit].block_off;
}
int64_t fx_unit_summary_offset(fx_plan_t p, int32_t unit) {
  if (!p || unit < 0 || unit >= p->units) return -1;
  return p->host_units[unit].sum_off;
}
size_t fx_work_bytes(fx_plan_t p) {
  if (!p) return 0;
  return (size_t)p->work_rows * p->desc.head_dim * (p->desc.dtype == FX_BF16 ? 2 : 4);
}
int32_t fx_unit_max_selected(fx_plan_t p, int32_t unit) {
  if (!p || unit < 0 || unit >= p->units) return -1;
  return p->host_units[unit].max_sel;
}
int64_t fx_unit_work_offset(fx_plan_t p, int32_t unit) {
  if (!p || unit < 0 || unit >= p->units) return -1;
  return p->host_units[unit].work_off;
}

const char* fx_status_string(fx_status s) {
  switch (s) {
    case FX_OK: return "FX_OK";
    case FX_E_INVALID: return "FX_E_INVALID: an argument or policy is out of range, null or misaligned";
    case FX_E_UNSUPPORTED: return "FX_E_UNSUPPORTED: no kernel for this request";
    case FX_E_WORKSPACE: return "FX_E_WORKSPACE: workspace smaller than fx_workspace_bytes()";
    case FX_E_HIP: return "FX_E_HIP: a HIP runtime call or kernel launch failed";
  }
  return "unknown fx_status";
}

fx_status fx_read_error(fx_plan_t p, uint32_t* host_word) {
  if (!p || !host_word) return FX_E_INVALID;
  return fx::dev_take_error(p->d_error, host_word) == 0 ? FX_OK : FX_E_HIP;
}

size_t fx_stream_read_sink_words(size_t bytes) {
  return (size_t)((bytes + fx::kStreamReadSpan - 1) / fx::kStreamReadSpan);
}

fx_status fx_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!req(src, 16) || !req(sink, 4) || bytes == 0 || bytes % 16 != 0 ||
      fx_stream_read_sink_words(bytes) > (size_t)INT32_MAX)
    return FX_E_INVALID;
  try {
    return hip_status(fx::launch_stream_read(src, bytes, sink, stream));
  } catch (...) {
    return FX_E_HIP;
  }
}

fx_status fx_build_summaries(fx_plan_t p, const void* K, const int32_t* seq_lens,
                             int32_t block_begin, int32_t block_end, void* summaries,
                             hipStream_t stream) {
  if (!p || !req(K, 16) || !req(seq_lens, 4) || !req(summaries, 16)) return FX_E_INVALID;
  try {
    return hip_status(
        fx::launch_build_summaries(p, K, seq_lens, block_begin, block_end, summaries, stream));
  } catch (...) {
    return FX_E_HIP;
  }
}

namespace {

fx_status select_blocks(fx_plan_t p, const void* q, const void* summaries,
                        const float* evict_logits, uint32_t* evicted_mask,
                        const int32_t* seq_lens, const int32_t* prev_idx,
                        const int32_t* prev_cnt, int32_t* sel_idx, int32_t* sel_cnt,
                        int32_t* added, int32_t* added_cnt, int32_t* removed,
                        int32_t* removed_cnt, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  if (!p || !req(q, 16) || !req(seq_lens, 4) || !req(sel_idx, 4) || !req(sel_cnt, 4) ||
      !req(workspace, 16))
    return FX_E_INVALID;
  if (p->any_scored && !req(summaries, 16)) return FX_E_INVALID;
  if (!opt(evict_logits, 4) || !opt(evicted_mask, 4)) return FX_E_INVALID;
  if (p->needs_logits && (!evict_logits || !evicted_mask)) return FX_E_INVALID;
  if (workspace_bytes < p->ws_total) return FX_E_WORKSPACE;
  try {
    float* scores = reinterpret_cast<float*>(static_cast<char*>(workspace) + p->ws_scores_off);
    if (fx::select_fused(p))
      return hip_status(fx::launch_select_fused(p, q, summaries, scores, evict_logits,
                                                evicted_mask, seq_lens, sel_idx, sel_cnt,
                                                prev_idx, prev_cnt, added, added_cnt, removed,
                                                removed_cnt, stream));
    if (p->any_scored) {
      if (fx::launch_score(p, q, summaries, seq_lens, scores, stream) != 0) return FX_E_HIP;
    }
    char* ws = static_cast<char*>(workspace);
    return hip_status(fx::launch_topk(p, scores, evict_logits, evicted_mask, seq_lens, sel_idx,
                                      sel_cnt, reinterpret_cast<uint32_t*>(ws + p->ws_keys_off),
                                      reinterpret_cast<uint32_t*>(ws + p->ws_bits_off), prev_idx,
                                      prev_cnt, added, added_cnt, removed, removed_cnt, stream));
  } catch (...) {
    return FX_E_HIP;
  }
}

}  // namespace

fx_status fx_select(fx_plan_t p, const void* q, const void* summaries, const float* evict_logits,
                    uint32_t* evicted_mask, const int32_t* seq_lens, int32_t* sel_idx,
                    int32_t* sel_cnt, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  return select_blocks(p, q, summaries, evict_logits, evicted_mask, seq_lens, nullptr, nullptr,
                       sel_idx, sel_cnt, nullptr, nullptr, nullptr, nullptr, workspace,
                       workspace_bytes, stream);
}

fx_status fx_select_delta(fx_plan_t p, const void* q, const void* summaries,
                          const float* evict_logits, uint32_t* evicted_mask,
                          const int32_t* seq_lens, const int32_t* prev_idx,
                          const int32_t* prev_cnt, int32_t* sel_idx, int32_t* sel_cnt,
                          int32_t* added, int32_t* added_cnt, int32_t* removed,
                          int32_t* removed_cnt, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  if (!req(prev_idx, 4) || !req(prev_cnt, 4) || !req(added, 4) || !req(added_cnt, 4) ||
      !req(removed, 4) || !req(removed_cnt, 4) || prev_idx == sel_idx || prev_cnt == sel_cnt)
    return FX_E_INVALID;
  return select_blocks(p, q, summaries, evict_logits, evicted_mask, seq_lens, prev_idx,
                       prev_cnt, sel_idx, sel_cnt, added, added_cnt, removed, removed_cnt,
                       workspace, workspace_bytes, stream);
}

namespace {

fx_status check_decode_args(fx_plan_t p, const void* q, const void* K, const void* V,
                            const int32_t* seq_lens, const int32_t* sel_idx,
                            const int32_t* sel_cnt, float softmax_scale, const void* out,
                            const float* lse) {
  if (!p || !req(q, 16) || !req(K, 16) || !req(V, 16) || !req(seq_lens, 4) ||
      !req(sel_idx, 4) || !req(sel_cnt, 4) || !req(out, 16) || !opt(lse, 4))
    return FX_E_INVALID;
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale)) return FX_E_INVALID;
  return FX_OK;
}

fx_status sparse_decode(fx_plan_t p, const void* q, const void* K, const void* V,
                        const int32_t* seq_lens, const int32_t* sel_idx, const int32_t* sel_cnt,
                        const float* logits, float softmax_scale, void* out, float* lse,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  fx_status st = check_decode_args(p, q, K, V, seq_lens, sel_idx, sel_cnt, softmax_scale, out, lse);
  if (st != FX_OK) return st;
  if (!req(workspace, 16)) return FX_E_INVALID;
  if (workspace_bytes < p->ws_total) return FX_E_WORKSPACE;
  try {
    char* ws = static_cast<char*>(workspace);
    return hip_status(fx::launch_decode(p, q, K, V, seq_lens, sel_idx, sel_cnt, logits,
                                        softmax_scale, out, lse, ws + p->ws_decode_off, stream));
  } catch (...) {
    return FX_E_HIP;
  }
}

}  // namespace

fx_status fx_sparse_decode(fx_plan_t p, const void* q, const void* K, const void* V,
                           const int32_t* seq_lens, const int32_t* sel_idx,
                           const int32_t* sel_cnt, float softmax_scale, void* out, float* lse,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return sparse_decode(p, q, K, V, seq_lens, sel_idx, sel_cnt, nullptr, softmax_scale, out, lse,
                       workspace, workspace_bytes, stream);
}

fx_status fx_sparse_decode_ed(fx_plan_t p, const void* q, const void* K, const void* V,
                              const int32_t* seq_lens, const int32_t* sel_idx,
                              const int32_t* sel_cnt, const float* evict_logits,
                              float softmax_scale, void* out, float* lse, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  if (!p || !opt(evict_logits, 4) || (p->any_nosa && !evict_logits)) return FX_E_INVALID;
  // Without NOSA units there is no eviction term: plain attention.
  return sparse_decode(p, q, K, V, seq_lens, sel_idx, sel_cnt,
                       p->any_nosa ? evict_logits : nullptr, softmax_scale, out, lse, workspace,
                       workspace_bytes, stream);
}

fx_status fx_sparse_decode_noalloc(fx_plan_t p, const void* q, const void* K, const void* V,
                                   const int32_t* seq_lens, const int32_t* sel_idx,
                                   const int32_t* sel_cnt, float softmax_scale, void* out,
                                   float* lse, hipStream_t stream) {
  fx_status st = check_decode_args(p, q, K, V, seq_lens, sel_idx, sel_cnt, softmax_scale, out, lse);
  if (st != FX_OK) return st;
  if (!p->static_scratch) return FX_E_HIP;
  if (!p->static_scratch_fits) return FX_E_WORKSPACE;
  try {
    return hip_status(fx::launch_decode(p, q, K, V, seq_lens, sel_idx, sel_cnt, nullptr,
                                        softmax_scale, out, lse, p->static_scratch, stream));
  } catch (...) {
    return FX_E_HIP;
  }
}

size_t fx_noalloc_scratch_bytes(fx_plan_t p) { return p ? p->ws_decode.end : 0; }

fx_status fx_compact_update(fx_plan_t p, const void* K, const void* V, const int32_t* seq_lens,
                            const int32_t* sel_idx, const int32_t* sel_cnt, int32_t* slot_map,
                            void* work_K, void* work_V, int32_t* moved_cnt, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  if (!p || !req(K, 16) || !req(V, 16) || !req(seq_lens, 4) || !req(sel_idx, 4) ||
      !req(sel_cnt, 4) || !req(slot_map, 4) || !req(work_K, 16) || !req(work_V, 16) ||
      !opt(moved_cnt, 4) || !req(workspace, 16))
    return FX_E_INVALID;
  if (workspace_bytes < p->ws_total) return FX_E_WORKSPACE;
  if (p->max_sel > fx::kMaxCompactSlots) return FX_E_UNSUPPORTED;
  try {
    char* ws = static_cast<char*>(workspace);
    return hip_status(fx::launch_compact(p, K, V, seq_lens, sel_idx, sel_cnt, slot_map, work_K,
                                         work_V, moved_cnt,
                                         ws + p->ws_moves_off,
                                         reinterpret_cast<int32_t*>(ws + p->ws_move_cnt_off),
                                         stream));
  } catch (...) {
    return FX_E_HIP;
  }
}

fx_status fx_selection_delta(fx_plan_t p, const int32_t* prev_idx, const int32_t* prev_cnt,
                             const int32_t* cur_idx, const int32_t* cur_cnt, int32_t* added,
                             int32_t* added_cnt, int32_t* removed, int32_t* removed_cnt,
                             hipStream_t stream) {
  if (!p || !req(prev_idx, 4) || !req(prev_cnt, 4) || !req(cur_idx, 4) || !req(cur_cnt, 4) ||
      !req(added, 4) || !req(added_cnt, 4) || !req(removed, 4) || !req(removed_cnt, 4))
    return FX_E_INVALID;
  try {
    return hip_status(fx::launch_delta(p, prev_idx, prev_cnt, cur_idx, cur_cnt, added, added_cnt,
                                       removed, removed_cnt, stream));
  } catch (...) {
    return FX_E_HIP;
  }
}

}  // extern "C"
