/*
 * fx.h -- block-sparse decode attention over a KV cache resident in one GPU's HBM.
 *
 * A small C ABI over hand-written HIP kernels for gfx950 (AMD Instinct MI355X).
 * One decode step of one layer runs:
 *
 *   fx_build_summaries  pooled per-block key summaries (when blocks fill)
 *   fx_select           block scores against each GQA query group and per-kv-head
 *                       block selection (streaming / retrieval top-k / NOSA)
 *   fx_sparse_decode    flash-decoding over the selected blocks only, split evenly
 *                       across the GPU
 *   fx_sparse_decode_ed the same with each NOSA block's eviction logit added to its
 *                       tokens' attention logits (exp-delayed eviction scores)
 *   fx_selection_delta  blocks added to / removed from the previous selection
 *   fx_select_delta     fx_select and fx_selection_delta in one call (the differences
 *                       are formed where the selection is made)
 *   fx_compact_update   keep the selected full blocks in a block-slot working set,
 *                       moving only the newly selected ones
 *
 * Sources, cited by page title and section:
 *   [Fluxion-NL] "Technische Samenvatting: Fluxion" (gist.science/nl/paper/2605.07719)
 *   [NOSA-DE]    "Technisches Resümee: NOSA: Native und Offloadable Sparse Attention"
 *                (gist.science/de/paper/2510.13602)
 *   [Fluxion-KO] "An Efficient Hybrid Sparse Attention with CPU-GPU Parallelism for
 *                Long-Context Inference" (gist.science/ko/paper/2605.07719)
 * The pages describe offloaded KV caches; here the whole cache stays in HBM, so
 * none of their transfer machinery appears.  The pages give no formulas; each
 * entry point below states the definition it computes.
 *
 * ---------------------------------------------------------------------------------
 * Terms and layouts (all arrays are contiguous, row-major, device memory unless noted)
 *
 *   B  batch (sequences), Hq query heads, Hkv kv heads, G = Hq / Hkv (1..8),
 *   d  head_dim (64 or 128), t_cap tokens of capacity per (sequence, kv head).
 *   unit u = b * Hkv + h is one (sequence b, kv head h).  Query head hq belongs to
 *   kv head hq / G: the G query rows of unit u are q[b][h*G .. h*G+G-1].
 *   elem = float32 (FX_F32) or bfloat16 (FX_BF16), chosen per plan.
 *
 *   q        elem [B][Hq][d]
 *   K, V     elem [B][Hkv][t_cap][d]; row t of a unit is token t.
 *   seq_lens int32 [B] (device): tokens T_b valid in sequence b (0 <= T_b <= t_cap).
 *   out      elem [B][Hq][d];  lse float32 [B][Hq] (natural log, scale included).
 *
 *   Blocks: unit u uses block size g_u (its policy's `block`).  Block j covers
 *   tokens [j*g_u, min((j+1)*g_u, T_b)).  n_full = T_b / g_u full blocks,
 *   n_tot = ceil(T_b / g_u) blocks; only the last block can be partial.
 *   n_cap(u) = ceil(t_cap / g_u) block slots.
 *
 *   Per-block arrays are packed per unit: unit u owns n_cap(u) consecutive slots
 *   starting at block_off(u) = sum over u' < u of n_cap(u').  In this layout:
 *     evict_logits  float32 [total_blocks]
 *   Summaries have r(u) rows per block slot: r = 1 under FX_POOL_KEY, block /
 *   sub_block under score-side pooling.  Unit u owns n_cap(u) * r(u) rows starting at
 *   row sum_off(u) = sum over u' < u of n_cap(u') * r(u'); block j's rows are
 *   sum_off(u) + j*r .. + r - 1 (sum_off = block_off under FX_POOL_KEY):
 *     summaries     elem [summary_rows][d]
 *   The eviction mask packs ceil(n_cap(u)/32) uint32 words per unit starting at
 *   word mask_off(u) = sum over u' < u of ceil(n_cap(u')/32); block j of unit u is
 *   bit (j % 32) of word mask_off(u) + j / 32.  Bits set = evicted.
 *
 *   Selections: sel_idx int32 [units][max_sel], ascending block indices of the
 *   unit, padded with -1; sel_cnt int32 [units].  max_sel = fx_max_selected().
 *
 * Ownership and ordering
 *   The caller owns every buffer, stream and the eviction mask.  A plan owns only
 *   a small device table (per-unit policies, the list of scored units and an error
 *   word), allocated by
 *   fx_plan_create and freed by fx_plan_destroy; the hot calls only read it (and
 *   set error bits).  The four hot calls never allocate, never synchronise and
 *   never copy between host and device: they enqueue kernels on `stream` and
 *   return.  Calls that overlap in time must not share a workspace or output
 *   buffers.
 *
 * Errors
 *   Every call validates its host-side arguments first; on failure it returns a
 *   nonzero status and enqueues nothing.  Null pointers for required buffers, and
 *   pointers to q, K, V, summaries, out or workspace that are not 16-byte aligned
 *   (any other pointer: not aligned to its element size) are FX_E_INVALID.  A
 *   failed kernel launch is FX_E_HIP.  No C++ exception crosses this ABI.  Bad
 *   device-side data (a seq_len outside [0, t_cap], a selection index outside the
 *   unit's blocks, a non-finite score) is clamped or skipped so that no access
 *   leaves its buffer, and sets a bit in the plan's error word (fx_read_error).
 * ---------------------------------------------------------------------------------
 */
#ifndef FX_H_
#define FX_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;   /* HIP's stream handle; NULL = default stream */

typedef int32_t fx_status;
enum {
  FX_OK = 0,
  FX_E_INVALID = 1,       /* an argument or policy is out of range, null or misaligned */
  FX_E_UNSUPPORTED = 2,   /* a valid request the library has no kernel for */
  FX_E_WORKSPACE = 3,     /* workspace smaller than fx_workspace_bytes() */
  FX_E_HIP = 4            /* a HIP runtime call or kernel launch failed */
};

enum { FX_F32 = 0, FX_BF16 = 1 };

/* Head modes.
 *   FX_RETRIEVAL: top-k blocks by score under a per-head granularity and budget
 *                 ([Fluxion-NL] Kerninzichten item 2, Systeemcomponenten).
 *   FX_STREAMING: only the sink and the local window, no selection
 *                 ([Fluxion-NL] Kerninzichten item 2; [Fluxion-KO] 해결책, strategy 2).
 *   FX_NOSA:      query-aware top-k (Γq) plus query-agnostic top-k_e by eviction
 *                 logit (Γe) with strict eviction ([NOSA-DE] Methodik §1).          */
enum { FX_RETRIEVAL = 0, FX_STREAMING = 1, FX_NOSA = 2 };

/* Where the block-level max of the two-stage pooling acts ([NOSA-DE] Methodik §1,
 * "Blockweise Implementierung": mean inside sub-blocks, then max at block level).
 *   FX_POOL_KEY:       on the key side.  One summary row per block, the elementwise max
 *                      of its sub-block means; the score sums the group's dot products
 *                      with it.
 *   FX_POOL_SCORE_SUM: on the score side.  r = block / sub_block summary rows per block,
 *                      one per sub-block mean; the score is the max over them of the
 *                      group's summed dot product.
 *   FX_POOL_SCORE_MAX: as FX_POOL_SCORE_SUM with the group aggregated by a max over its
 *                      G query rows instead of a sum.                                   */
enum { FX_POOL_KEY = 0, FX_POOL_SCORE_SUM = 1, FX_POOL_SCORE_MAX = 2 };

/* Error-word bits (fx_read_error). */
enum {
  FX_ERR_SEQ_LEN = 1u << 0,        /* a seq_len was outside [0, t_cap]; clamped */
  FX_ERR_SEL_INDEX = 1u << 1,      /* a selection entry was outside [0, n_tot) or not ascending; skipped */
  FX_ERR_SEL_COUNT = 1u << 2,      /* a sel_cnt was outside [0, max_sel]; clamped */
  FX_ERR_NONFINITE = 1u << 3,      /* a non-finite score or eviction logit: NaN ranked
                                      lowest, +-inf ranked as the largest / smallest value
                                      (fx_sparse_decode_ed: counted as 0) */
  FX_ERR_SLOT_MAP = 1u << 4        /* fx_compact_update: a slot row held one block twice and
                                      some selected blocks found no free slot */
};

typedef struct {
  int32_t batch;           /* B >= 1 */
  int32_t num_q_heads;     /* Hq, a multiple of num_kv_heads with G = Hq/Hkv in [1, 8] */
  int32_t num_kv_heads;    /* Hkv >= 1 */
  int32_t head_dim;        /* d: 64 or 128 */
  int32_t t_cap;           /* tokens of capacity per unit, 1 .. 2^24, with t_cap * head_dim *
                              sizeof(elem) < 2^31 (else FX_E_UNSUPPORTED) */
  int32_t dtype;           /* FX_F32 or FX_BF16: element type of q, K, V, summaries, out */
  int32_t split_tokens;    /* fewest selected tokens per decode workgroup (a power of two,
                              64..2048), 0 = automatic (256) */
  int32_t pooling;         /* FX_POOL_KEY (0), FX_POOL_SCORE_SUM or FX_POOL_SCORE_MAX; the
                              score-side kinds need block / sub_block <= 64 in every unit
                              (else FX_E_UNSUPPORTED) */
} fx_plan_desc;

/* Per-unit selection policy.  Blocks of one unit are `block` tokens (a power of
 * two, 1..256); `sub_block` (a power of two dividing `block`) is the mean-pooling
 * span of the block summaries.
 *
 * Forced blocks F (always selected, never candidates):
 *   streaming       : every block overlapping tokens [0, min(sink_tokens, T)) or
 *                     [max(0, T - local_tokens), T);
 *   retrieval, NOSA : block 0 if force_sink, block n_tot-1 if force_last;
 *   every mode      : the partial last block, if T is not a multiple of `block`
 *                     (it has no summary and holds the newest tokens).
 * Retrieval: k = top_k if top_k > 0, else ceil(budget * n_tot) evaluated in
 *   float64 (exact); the k best full blocks outside F by score are chosen, k
 *   clamped to the number of candidates.  Forced blocks come on top of k.
 * NOSA: top_k is the size of Γq, k_evict the size of Γe (top_k + k_evict >= 1).
 * "Best" means larger value first and, for equal values, the lower block index.  */
typedef struct {
  int32_t mode;            /* FX_RETRIEVAL | FX_STREAMING | FX_NOSA */
  int32_t block;           /* g: power of two in [1, 256] */
  int32_t sub_block;       /* s: power of two, divides g */
  int32_t top_k;           /* retrieval: > 0 overrides budget; NOSA: |Γq| */
  float budget;            /* retrieval with top_k == 0: fraction of blocks in (0, 1] */
  int32_t k_evict;         /* NOSA: |Γe| >= 0 */
  int32_t sink_tokens;     /* streaming: >= 0 */
  int32_t local_tokens;    /* streaming: >= 0 */
  int32_t force_sink;      /* retrieval / NOSA: 0 or 1 */
  int32_t force_last;      /* retrieval / NOSA: 0 or 1 */
} fx_head_policy;

typedef struct fx_plan* fx_plan_t;

/* Validate the shapes and the per-unit policies (host array of B*Hkv entries,
 * copied), compute the packed layouts, and allocate the plan's device table on
 * the current HIP device; the decode split is sized for that device.  The token slots
 * of the longest valid selection lists, sum over u of min(n_cap(u), max_sel) * block(u)
 * (n_cap(u) = ceil(t_cap / block(u)), max_sel the lists' row stride), must stay below
 * 2^31 (else FX_E_UNSUPPORTED).  *out is set only on FX_OK. */
fx_status fx_plan_create(const fx_plan_desc* desc, const fx_head_policy* host_policies,
                         fx_plan_t* out);
/* Free the plan's device table.  NULL is a no-op.  Waits for nothing: the caller
 * must not destroy a plan while its kernels may still run. */
fx_status fx_plan_destroy(fx_plan_t plan);

/* Sizes derived from the plan (0 / -1 for a NULL plan). */
size_t fx_summary_bytes(fx_plan_t plan);       /* summary_rows * d * sizeof(elem) */
size_t fx_logits_bytes(fx_plan_t plan);        /* total_blocks * 4 */
size_t fx_evict_mask_bytes(fx_plan_t plan);    /* total mask words * 4 */
size_t fx_workspace_bytes(fx_plan_t plan);     /* workspace for fx_select and fx_sparse_decode */
int32_t fx_max_selected(fx_plan_t plan);       /* max_sel: row stride of sel_idx and delta lists */
int64_t fx_unit_block_offset(fx_plan_t plan, int32_t unit);   /* block_off(u), -1 if out of range */
int64_t fx_unit_summary_offset(fx_plan_t plan, int32_t unit); /* sum_off(u), -1 if out of range */
size_t fx_work_bytes(fx_plan_t plan);          /* work_rows * d * sizeof(elem): each of work_K, work_V */
int64_t fx_unit_work_offset(fx_plan_t plan, int32_t unit);    /* work_off(u), -1 if out of range */
int32_t fx_unit_max_selected(fx_plan_t plan, int32_t unit);   /* max_sel(u): selection bound and
                                                                 compaction slots, -1 if out of range */
int32_t fx_split_tokens(fx_plan_t plan);       /* the split_tokens value the plan uses */

const char* fx_status_string(fx_status status);

/* Copy the plan's device error word to *host_word and clear it.  Synchronises
 * the current device (a debugging / harness call, not for the hot loop). */
fx_status fx_read_error(fx_plan_t plan, uint32_t* host_word);

/* Measurement utility, not part of the decode path: the attainable streaming-read
 * bandwidth reference.  Reads the `bytes` bytes at `src` (device memory, 16-byte
 * aligned) once with 16-byte nontemporal loads, one workgroup per 1 MiB span, and
 * writes the XOR of each span to sink[span] (fx_stream_read_sink_words(bytes) uint32
 * words of device memory), so the reads cannot be removed.  Enqueued on `stream`;
 * allocates nothing. */
size_t fx_stream_read_sink_words(size_t bytes);
fx_status fx_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

/* [NOSA-DE] Methodik §1, bullet "Blockweise Implementierung" (two-stage pooling:
 * mean inside sub-blocks, then max at block level); Methodik §2, bullet "Kernel
 * Fusion" (pooling runs inside a fused kernel).
 * For every unit and every FULL block j in the range, writes
 *     S[j][c] = round_once( max over sub-blocks u of (sum of the s rows of u)[c] / s )
 * where the sums are exact (float64) and the single rounding is to nearest, ties
 * to even, into elem.  The range is [block_begin, block_end) in block indices,
 * resolved per unit like a Python slice against n_full (negative values count
 * from n_full; both ends are clamped to [0, n_full]); (0, INT32_MAX) is every full
 * block, (-1, INT32_MAX) the newest one.  Slots outside the range are untouched.
 * Under score-side pooling (FX_POOL_SCORE_*) the max is not taken here: block j's r
 * summary rows are the r sub-block means, each rounded once:
 *     S[j*r + u][c] = round_once( (sum of the s rows of sub-block u)[c] / s ).
 * K: elem [B][Hkv][t_cap][d]; summaries: elem [summary_rows][d] (fx_summary_bytes). */
fx_status fx_build_summaries(fx_plan_t plan, const void* K, const int32_t* seq_lens,
                             int32_t block_begin, int32_t block_end, void* summaries,
                             hipStream_t stream);

/* [NOSA-DE] Methodik §1 ("Query-Aware Selection", "Query-Agnostic Selection" with
 * strict eviction, "Lokalitätsgarantie", "ED-DMA": ranking on pre-exponential
 * values); [Fluxion-NL] Kerninzichten item 2 and Systeemcomponenten ("Granularity-
 * Budget Selector": one selection per GQA group).
 * Score of full block j of unit u (retrieval and NOSA units), a float32 value:
 *     qs = ((q_0 + q_1) + ...) + q_{G-1}      float64, the unit's G query rows in order
 *     acc = ((0 + qs[0]*S_j[0]) + qs[1]*S_j[1]) + ...   float64, columns in order,
 *                                               every product and sum rounded (no FMA)
 *     score = (float)acc                        round to nearest, ties to even
 * i.e. the sum over the group of the raw dot products with the summary (no
 * 1/sqrt(d), no softmax).  Under score-side pooling the same chain runs over each of
 * the block's r summary rows M_u and
 *     FX_POOL_SCORE_SUM: score = (float) max over u of acc(qs, M_u)
 *     FX_POOL_SCORE_MAX: score = (float) max over u and g of acc(q_g, M_u)
 * (acc(v, M) being the chain above with v in place of qs).
 * Then per unit, with F the forced set (see fx_head_policy):
 *   streaming : selection = F;
 *   retrieval : selection = F + the k best full blocks outside F by score;
 *   NOSA      : E = full blocks outside F not evicted; Γe = the k_evict best of E by
 *               evict_logits (raw); every block of E outside Γe becomes evicted
 *               (bit set in evicted_mask, in place); Γq = the top_k best full blocks
 *               outside F and Γe by score (evicted blocks stay eligible);
 *               selection = F + Γe + Γq.
 * Writes sel_idx (ascending, padded with -1) and sel_cnt.  evict_logits and
 * evicted_mask are required when any unit is NOSA with k_evict > 0, else may be
 * NULL.  workspace: >= fx_workspace_bytes(plan) bytes, 256-byte aligned; its
 * contents need no initialisation and are scratch after the call. */
fx_status fx_select(fx_plan_t plan, const void* q, const void* summaries,
                    const float* evict_logits, uint32_t* evicted_mask,
                    const int32_t* seq_lens, int32_t* sel_idx, int32_t* sel_cnt,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* fx_select followed by fx_selection_delta(prev, the new selection), in one call: for
 * plans whose units have at most 8192 block slots the differences are formed by the
 * selection kernel itself (no separate kernel).  Arguments as for the two calls; prev_idx /
 * prev_cnt must not be sel_idx / sel_cnt.  prev is read as fx_selection_delta reads it
 * (its longest valid prefix; entries past it are ignored and set FX_ERR_SEL_INDEX). */
fx_status fx_select_delta(fx_plan_t plan, const void* q, const void* summaries,
                          const float* evict_logits, uint32_t* evicted_mask,
                          const int32_t* seq_lens, const int32_t* prev_idx,
                          const int32_t* prev_cnt, int32_t* sel_idx, int32_t* sel_cnt,
                          int32_t* added, int32_t* added_cnt, int32_t* removed,
                          int32_t* removed_cnt, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* [Fluxion-NL] Probleemstelling item 1 (after top-k selection, attention runs over
 * the selected KV blocks only); [NOSA-DE] Methodik §1, "ED-DMA" (the exponential
 * belongs to the attention phase).
 * For each unit and each of its G query rows q: over the valid tokens t of the
 * selected blocks, s_t = softmax_scale * (q . K_t); out = sum_t e^{s_t - m} V_t / l
 * with m = max s_t and l = sum_t e^{s_t - m}; lse = m + ln l.  Computed as
 * flash-decoding with a float32 online softmax: the token slots of the units' selected
 * blocks (block(u) per selected block; slots past the sequence end or in an invalid
 * entry are masked and read no memory), laid end to end, are cut into as many equal
 * segments (at least split_tokens long) as the GPU holds decode workgroups at once, one
 * per workgroup; a unit cut by a segment
 * boundary is finished by a log-sum-exp merge of its pieces in a second kernel, in
 * piece order.  Results depend only on the inputs and the plan (on one device), not
 * on scheduling.  A unit with no valid token gets out = 0, lse = -inf.
 * sel_idx / sel_cnt as written by fx_select (any ascending list of valid block
 * indices of the unit is accepted).  lse may be NULL.  workspace as for fx_select
 * (the two calls may share one workspace; they use disjoint parts of it). */
fx_status fx_sparse_decode(fx_plan_t plan, const void* q, const void* K, const void* V,
                           const int32_t* seq_lens, const int32_t* sel_idx,
                           const int32_t* sel_cnt, float softmax_scale, void* out,
                           float* lse, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* [NOSA-DE] Methodik §1, "ED-DMA": the eviction head's exponential is taken only in the
 * attention phase; selection ranks the values before it.  The page gives no formula;
 * this call reads it as an additive pre-softmax term.
 * As fx_sparse_decode, except that for every NOSA unit u each valid token t of a
 * selected block j has
 *     s_t = softmax_scale * (q . K_t) + b_j,   b_j = evict_logits[block_off(u) + j],
 * so e^{b_j} multiplies the block's weights inside the softmax and is never formed on
 * its own (lse includes the term).  Retrieval and streaming units have no eviction head
 * and get exactly fx_sparse_decode's result.  evict_logits: float32 [total_blocks] in
 * fx_select's layout (slots of blocks that are not selected are not read); required when
 * the plan has a NOSA unit, else may be NULL.  A non-finite b_j counts as 0 and sets
 * FX_ERR_NONFINITE.  Workspace and the other arguments as for fx_sparse_decode. */
fx_status fx_sparse_decode_ed(fx_plan_t plan, const void* q, const void* K, const void* V,
                              const int32_t* seq_lens, const int32_t* sel_idx,
                              const int32_t* sel_cnt, const float* evict_logits,
                              float softmax_scale, void* out, float* lse, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory while decoding: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * fx_sparse_decode with no workspace argument: its decode partials go to a static device
 * array of the library, 8 MiB per GPU (one per GPU the library runs on, held until the
 * process ends; its address is looked up at fx_plan_create, on the plan's device).  The
 * call allocates nothing.  Arguments, results and errors as for fx_sparse_decode; a plan
 * whose partials need more than 8 MiB (fx_noalloc_scratch_bytes) is refused with
 * FX_E_WORKSPACE, and FX_E_HIP means the array's address could not be found.  Every call
 * on one GPU shares that GPU's array, which keeps the last call's partials (nothing in it
 * needs clearing): calls whose kernels overlap in time on one GPU race, so they must be
 * ordered (one stream, or events). */
fx_status fx_sparse_decode_noalloc(fx_plan_t plan, const void* q, const void* K, const void* V,
                                   const int32_t* seq_lens, const int32_t* sel_idx,
                                   const int32_t* sel_cnt, float softmax_scale, void* out,
                                   float* lse, hipStream_t stream);
/* Bytes of the static array a plan's fx_sparse_decode_noalloc uses (0 for a NULL plan). */
size_t fx_noalloc_scratch_bytes(fx_plan_t plan);

/* [NOSA-DE] Methodik §2 (NOSI), bullet "Optimierte Speicherlayout": the cache is held in
 * minimal block units and blocks are swapped by set difference, with no contiguous
 * allocation.  Keeps, per unit, a copy of its selected FULL blocks in a working set of
 * block slots.  Unit u has max_sel(u) slots (its policy's selection bound); slot s holds
 * rows work_off(u) + s*g .. + g - 1 of work_K and work_V, elem [work_rows][d]
 * (fx_work_bytes, fx_unit_work_offset; work_off = sum over u' < u of max_sel(u') * g_u').
 * slot_map int32 [units][max_sel] names the block in each slot (-1 = free); it is
 * state owned by the caller, set to -1 before the first call, updated in place (entries
 * past max_sel(u) are not read).  With target = the valid selected blocks j < n_full
 * (sel_idx / sel_cnt as written by fx_select; the partial last block still grows and is
 * never held), each call:
 *   1. frees every slot whose block is not in target;
 *   2. gives the target blocks no slot holds, in ascending block order, the free slots
 *      in ascending slot order (held blocks never move);
 *   3. copies each newly placed block's g key rows and g value rows from K, V into its
 *      slot (rows of slots that did not change are not touched).
 * moved_cnt int32 [units] (may be NULL) receives the number of blocks copied per unit.
 * Needs max_sel <= 2048 (else FX_E_UNSUPPORTED).  workspace as for fx_select (a part of
 * it that select and decode do not use).  Bad device data: a selection entry that is not
 * valid is skipped (FX_ERR_SEL_INDEX); more target blocks than slots keeps the lowest
 * ones (FX_ERR_SEL_COUNT); a slot row naming a block twice can leave blocks without a
 * slot (FX_ERR_SLOT_MAP).  No access leaves its buffer in any of these cases. */
fx_status fx_compact_update(fx_plan_t plan, const void* K, const void* V,
                            const int32_t* seq_lens, const int32_t* sel_idx,
                            const int32_t* sel_cnt, int32_t* slot_map, void* work_K,
                            void* work_V, int32_t* moved_cnt, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* [NOSA-DE] Methodik §2, bullet "Optimierte Speicherlayout" (set differences of
 * block selections drive block swapping); Methodik §1, "Lokalitätsgarantie".
 * Per unit: added = cur \ prev and removed = prev \ cur, each ascending, padded
 * with -1 to max_sel, with their counts.  prev / cur are sel_idx / sel_cnt arrays in
 * fx_select's layout; a prev_cnt of 0 (the first step) makes every current block "added".
 * Each list enters as its longest prefix that is strictly ascending within the unit's
 * block slots [0, n_cap(u)) (fx_select writes such lists); an entry past that prefix is
 * ignored and sets FX_ERR_SEL_INDEX, and a count outside [0, max_sel] is clamped and sets
 * FX_ERR_SEL_COUNT.  |cur| = |prev| - |removed| + |added| holds per unit for the lists
 * as entered. */
fx_status fx_selection_delta(fx_plan_t plan, const int32_t* prev_idx, const int32_t* prev_cnt,
                             const int32_t* cur_idx, const int32_t* cur_cnt,
                             int32_t* added, int32_t* added_cnt, int32_t* removed,
                             int32_t* removed_cnt, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FX_H_ */
