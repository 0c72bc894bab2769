// Internal declarations shared by the host code (fx_api.cpp) and the kernel files of
// libfx.  Host-only: no HIP header is needed to compile this file, so the plan logic,
// argument validation and workspace layout build with a plain C++ compiler as well
// (the CPU checks of the host path do that, with stand-ins for the device calls).
// Not part of the ABI (include/fx.h is).
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

#include "fx.h"

namespace fx {

constexpr int kMaxGroup = 8;          // G = Hq / Hkv
constexpr int kMaxBlock = 256;        // largest block size g
constexpr int kMaxSplit = 2048;       // largest minimum decode segment; also the token run
                                      // whose block indices one LDS list holds
constexpr int kMinSplit = 64;
constexpr int kAutoSplit = 256;       // minimum decode segment when the caller passes 0
constexpr int kShortSegment = 1024;   // below this many tokens per segment, use half the grid
constexpr int kCUsMin = 64;           // (only on grids of at least 2 * kCUsMin workgroups)
constexpr int kAlignedUnitsDiv = 8;   // unit-aligned decode pieces when units <= half grid / this
constexpr int kUncutSlots = 512;      // auto split: units of at most this many token slots stay whole
constexpr uint64_t kStreamReadSpan = 1ull << 20;   // bytes per workgroup of fx_stream_read
constexpr int kMaxTcap = 1 << 24;
constexpr int kTopkRegBlocks = 8192;   // selection keeps keys in registers up to this n_cap
constexpr int kFusedSelectBlocks = 512;   // scores formed inside the selection up to this n_cap
constexpr int kMaxScoreRows = 64;     // summary rows per block under score-side pooling
constexpr int kMaxCompactSlots = 2048;   // compaction slots per unit (LDS lists)
// Decode scratch of fx_sparse_decode_noalloc: one static device array per GPU.
constexpr size_t kStaticScratchBytes = size_t(8) << 20;

// Per-unit policy as the kernels read it (device table owned by the plan).
struct UnitInfo {
  int32_t mode;
  int32_t g;           // block size
  int32_t log2g;
  int32_t s;           // sub-block size
  int32_t top_k;
  float budget;
  int32_t k_evict;
  int32_t sink;
  int32_t local;
  int32_t force_sink;
  int32_t force_last;
  int32_t max_sel;     // upper bound on this unit's selection size
  int32_t n_cap;       // ceil(t_cap / g)
  int32_t mask_off;    // first eviction-mask word of the unit
  int64_t block_off;   // first block slot of the unit in the packed per-block arrays
  int32_t log2r;       // log2 of the summary rows per block (0 under key-side pooling)
  int32_t reserved;
  int64_t sum_off;     // first summary row of the unit
  int64_t work_off;    // first row of the unit's compaction slots (max_sel * g rows)
};
static_assert(sizeof(UnitInfo) == 88, "UnitInfo layout");

// Byte offsets of the decode partials inside a scratch buffer (the caller's workspace,
// or the static array of fx_sparse_decode_noalloc).
struct DecodeScratch {
  size_t part_o = 0;     // float [decode_grid][2][G][d]   (head, tail pieces)
  size_t part_ml = 0;    // float2 [decode_grid][2][G]     (m, l)
  size_t seg = 0;        // int2 [decode_grid]             (unit, pieces)
  size_t end = 0;        // first byte past the three arrays
};

}  // namespace fx

struct fx_plan {
  fx_plan_desc desc;
  int32_t G = 0;
  int32_t units = 0;
  std::vector<fx::UnitInfo> host_units;
  std::vector<int32_t> host_scored;
  int device = 0;
  // device table: [units] UnitInfo | uint32 error word | [n_scored] int32 unit ids |
  // [units] int32 unit ids
  void* d_table = nullptr;
  fx::UnitInfo* d_units = nullptr;
  uint32_t* d_error = nullptr;
  int32_t* d_scored = nullptr;   // retrieval and NOSA units, ascending
  int32_t* d_order = nullptr;    // every unit: the scored ones, then the others (ascending)
  int32_t n_scored = 0;
  int32_t max_scored_n_full_cap = 0;   // max over scored units of t_cap / g
  int32_t max_scored_rows_cap = 0;     // max over scored units of (t_cap / g) * r

  int64_t total_blocks = 0;
  int64_t summary_rows = 0;      // sum over units of n_cap * r
  int64_t work_rows = 0;         // sum over units of max_sel * g (compaction slots)
  int64_t mask_words = 0;
  int32_t max_sel = 0;
  int32_t max_n_cap = 0;
  int32_t max_n_full_cap = 0;    // max over units of t_cap / g
  int32_t split = 0;             // minimum decode segment in tokens (power of two)
  int32_t decode_split = 0;      // the minimum segment the decode kernel uses (>= split)
  bool decode_uncut = false;     // no unit can be cut into pieces: no merge kernel
  int32_t decode_grid = 0;       // decode workgroups = decode segments
  int32_t decode_grid_ed = 0;    // the same for fx_sparse_decode_ed (<= decode_grid)
  bool any_scored = false;       // some unit is retrieval or NOSA
  bool needs_logits = false;     // some NOSA unit has k_evict > 0
  bool any_nosa = false;         // some unit is NOSA

  // workspace layout (byte offsets)
  size_t ws_scores_off = 0;      // float [total_blocks]
  size_t ws_keys_off = 0;        // uint32 [total_blocks]     (top-k keys, workspace path only)
  size_t ws_bits_off = 0;        // uint32 [3 * mask_words]   (top-k bitmaps, workspace path only)
  fx::DecodeScratch ws_decode;   // decode partials, from ws_decode_off
  size_t ws_decode_off = 0;
  size_t ws_moves_off = 0;       // int2 [units][max_sel]          (compaction moves)
  size_t ws_move_cnt_off = 0;    // int32 [units]
  size_t ws_total = 0;

  // fx_sparse_decode_noalloc: the plan device's static scratch array (null if that
  // device's address could not be found) and whether the decode partials fit in it.
  void* static_scratch = nullptr;
  bool static_scratch_fits = false;
};

namespace fx {

// Kernel launchers (one per .hip file).  They assume validated arguments and return 0 or
// the HIP error code of the failed launch.
int launch_build_summaries(const fx_plan* p, const void* K, const int32_t* seq_lens,
                           int32_t block_begin, int32_t block_end, void* summaries,
                           hipStream_t stream);
int launch_score(const fx_plan* p, const void* q, const void* summaries, const int32_t* seq_lens,
                 float* scores, hipStream_t stream);
// prev_idx == nullptr: no delta; else also the differences against prev (fused into
// the register path, a second kernel on the workspace path).
int launch_topk(const fx_plan* p, const float* scores, const float* logits, uint32_t* mask,
                const int32_t* seq_lens, int32_t* sel_idx, int32_t* sel_cnt, uint32_t* ws_keys,
                uint32_t* ws_bits, const int32_t* prev_idx, const int32_t* prev_cnt,
                int32_t* added, int32_t* added_cnt, int32_t* removed, int32_t* removed_cnt,
                hipStream_t stream);
int launch_select_fused(const fx_plan* p, const void* q, const void* summaries, float* scores,
                        const float* logits, uint32_t* mask, const int32_t* seq_lens,
                        int32_t* sel_idx, int32_t* sel_cnt, const int32_t* prev_idx,
                        const int32_t* prev_cnt, int32_t* added, int32_t* added_cnt,
                        int32_t* removed, int32_t* removed_cnt, hipStream_t stream);
// logits == nullptr: plain attention; else each NOSA unit's token of block j also adds
// logits[block_off + j] to its attention logit.  scratch: the decode partials, laid out
// as p->ws_decode says.
int launch_decode(const fx_plan* p, const void* q, const void* K, const void* V,
                  const int32_t* seq_lens, const int32_t* sel_idx, const int32_t* sel_cnt,
                  const float* logits, float softmax_scale, void* out, float* lse,
                  void* scratch, hipStream_t stream);
int launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);
// moves: int2 [units][max_sel] in the workspace.
int launch_compact(const fx_plan* p, const void* K, const void* V, const int32_t* seq_lens,
                   const int32_t* sel_idx, const int32_t* sel_cnt, int32_t* slot_map,
                   void* work_K, void* work_V, int32_t* moved_cnt, void* moves,
                   int32_t* move_cnt, hipStream_t stream);
int launch_delta(const fx_plan* p, const int32_t* prev_idx, const int32_t* prev_cnt,
                 const int32_t* cur_idx, const int32_t* cur_cnt, int32_t* added,
                 int32_t* added_cnt, int32_t* removed, int32_t* removed_cnt, hipStream_t stream);

bool topk_in_registers(const fx_plan* p);   // else keys and bitmaps use the workspace
// Scores formed by the selection kernel itself (no k_score launch, no score reload).
bool select_fused(const fx_plan* p);

// Resident decode workgroups on the current device (0: error); ed: the instantiation
// with the eviction-logit term.
int decode_grid(const fx_plan* p, bool ed);

// Device runtime calls the host code makes (HIP in the library).  Each returns 0 or an
// error code.
int dev_current(int* device);
int dev_alloc(void** ptr, size_t bytes);
int dev_free(void* ptr);
int dev_upload(void* dst, const void* src, size_t bytes);   // synchronous host -> device
int dev_zero(void* dst, size_t bytes);                      // synchronous
// Waits for the current device, copies the error word at dev_word to *host_word and
// clears it.
int dev_take_error(uint32_t* dev_word, uint32_t* host_word);
// The static scratch array of the current device (looked up once per device); nullptr
// when the lookup fails.  *bytes receives its size.
void* dev_static_scratch(size_t* bytes);

}  // namespace fx
