// Split-K flash-decoding over the selected blocks, then a chunk merge.
//
// [Fluxion-NL] "Technische Samenvatting: Fluxion", Probleemstelling item 1: after
// top-k block selection, attention runs over the selected KV blocks only; Kerninzichten
// item 3: this work is bound by data movement, not arithmetic.  [NOSA-DE]
// "Technisches Resümee: NOSA: Native und Offloadable Sparse Attention", Methodik §1,
// "ED-DMA": the exponential belongs to the attention phase.
//
// Per unit (sequence b, kv head h) and query row q of its group:
//   s_t = scale * (q . K_t) over the valid tokens t of the selected blocks,
//   out = sum_t e^{s_t - m} V_t / l,  l = sum_t e^{s_t - m},  lse = m + ln l.
// With exp-delayed eviction scores (the ED instantiation), a NOSA unit's token t of
// block j has s_t = scale * (q . K_t) + b_j, b_j the block's raw eviction logit: its
// exponential is formed only inside the softmax.  Other units have no eviction head.
// A unit with cnt selected blocks has N = cnt * g token slots, numbered i = 0 .. N-1 in
// list order: slot i is offset i % g of selected block i / g.  Slots past the sequence
// end (the tail of a partial last block) and slots of invalid entries are masked: they
// read zeros without a memory access and take no weight.
//
// Work split (stream-K): the units' slot ranges, laid end to end in unit order, form
// one sequence of `total` slots, cut into equal segments of S = max(ceil(total / P),
// split) slots, P being the number of workgroups that fit on the device at once, or half
// of them when total / P is below kShortSegment slots or when the half grid's segments
// cut no unit and the full grid's would.  The grid holds the resident
// workgroups; workgroup s streams segment s, which may
// cover the end of one unit, whole units, and the start of another.  Every workgroup
// first scans all units (N_u from sel_cnt and the block size: one round of independent
// loads, no dependent read of the list) for the prefix sums; that costs a load round
// once per workgroup instead of once per chunk, and equal segments leave no tail of late
// chunks and no imbalance between XCDs.  A unit that lies inside one segment is finished by
// that workgroup.  A unit that crosses segment boundaries leaves one partial (o, m, l)
// per segment it touches: in its first segment in slot 1 ("tail") of that segment, in
// later ones in slot 0 ("head"); its first segment also records (unit, piece count).
// Units with no selected block (N_u = 0) get out = 0 and lse = -inf from workgroup
// u mod (grid size); a unit whose slots are all masked gets the same from its merge (l = 0).
//
// k_decode (4 waves per workgroup): within a piece of a unit, tokens go through LDS
// lists of at most kMaxSplit tokens' block indices; each list is shared out to the four
// waves in equal runs.  A token's d-vector is spread over LPT lanes, each lane holding
// 16 bytes (8 bfloat16 / 4 float32) of the K and V rows, so every load is a 128-bit
// load and each wave instruction reads 64/LPT whole rows.  K and V are read through raw
// buffer resources bounded to the unit's T valid rows: masked token slots get an
// out-of-range offset and read zeros without a branch or a memory access.  Loads for
// the next step of U tokens per lane group are issued before the current step is
// computed (register double buffering), so two steps are in flight per wave.  Each lane
// keeps the G query rows' matching 16 bytes in registers and forms G x U partial dot
// products (v_dot2_f32_bf16 for bfloat16).  Instead of reducing every one of them across
// the LPT lanes (and repeating the softmax in all of them), the partials pass through
// LDS transposed, so that each lane sums the LPT partials of its own (row, token) slots
// (see Slots): the cross-lane work per step drops from G x U reductions to one LDS round
// trip, and each score's exponential is taken once.  The online softmax runs in base 2
// (scores pre-multiplied by scale*log2(e)) per lane group, rescaling o and l only in
// steps where some running max grew.  For bfloat16 the P.V update takes tokens in pairs:
// p is rounded to bfloat16, paired within the quad, broadcast along the row (DPP
// row_newbcast), and one v_dot2_f32_bf16 per (row, column) accumulates both tokens.
// The lane groups of a wave merge down to as many as fit in its LDS area, those publish
// their partial (o, m, l), and the workgroup merges them with the log-sum-exp rule in a
// fixed order.
//
// k_combine (one workgroup per segment, exits unless the segment recorded a unit that
// continues past it) merges that unit's partials in segment order with the
// log-sum-exp rule, each output on its own thread in a fixed order, so results do not
// depend on scheduling.  The kernel boundary makes every partial visible to
// it; no fence is needed inside k_decode (an agent-scope fence per workgroup would
// write back the L2 each time).
#include <mutex>
#include <type_traits>

#include "fx_device.h"

namespace fx {
namespace {

constexpr int NT = 256;
constexpr int NWAVES = NT / 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;   // running max before any token (finite: no inf - inf)

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <typename E>
struct Lanes;
template <>
struct Lanes<bf16_t> {
  static constexpr int EPL = 8;   // elements per lane per row (16 bytes)
};
template <>
struct Lanes<float> {
  static constexpr int EPL = 4;
};

constexpr int kU = 4;   // tokens per lane group per step (the four lanes of a quad, below)

// Score slots of one step.  A lane group (LPT lanes, one token at a time) forms, for its
// kU tokens u and G query rows g, LPT partial dot products per (g, u).  They go to LDS
// and come back transposed: slot k = g * kU + u is summed by the lanes with
// k = (lane index in the group mod SLOTW) + SLOTW * j, j < SL, so each lane finishes SL
// scores instead of every lane finishing all G * kU.  With kU = 4 the four lanes of a quad
// hold one query row's four tokens (their max is two quad permutes) and u = lane & 3.
// Lanes past the G * kU slots repeat slot k mod G * kU.  Groups of 32 lanes are two rows
// of 16 that each hold every slot, so row broadcasts reach every lane that needs a value.
template <typename E, int D, int G>
struct Slots {
  static constexpr int LPT = D / Lanes<E>::EPL;
  static constexpr int NS = G * kU;
  static constexpr int SLOTW = LPT < 16 ? LPT : 16;
  static constexpr int SL = (NS + SLOTW - 1) / SLOTW;
  static constexpr int QPR = SLOTW / kU;   // query rows per slot register
  // LDS floats per slot and per lane group.  Slot stride LPT + 4 puts the slot bases that
  // eight lanes read together (one 128-byte LDS cycle of 16-byte reads) on distinct
  // four-bank groups; a group stride of 16 (LPT 16) or 8 (LPT 8) banks mod 32 keeps the
  // 32 lanes of one 4-byte write cycle on distinct banks.
  static constexpr int SS = LPT + 4;
  static constexpr int kResidue = LPT == 16 ? 16 : LPT == 8 ? 8 : 0;
  static constexpr int GS = NS * SS + ((kResidue - (NS * SS) % 32) + 32) % 32;
  static_assert(kU == 4, "a quad holds one query row's tokens");
};

// Row broadcast of lane `SRC` of this lane's group (row_newbcast: every lane of a row of
// 16 reads lane SRC of that row).  Groups of 8 take lane SRC or 8 + SRC of the row.
template <int LPT, int SRC>
__device__ __forceinline__ float group_bcast(float x) {
  static_assert(SRC >= 0 && SRC < (LPT < 16 ? LPT : 16), "source lane");
  const int xi = __float_as_int(x);
  if constexpr (LPT >= 16) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, xi, 0x150 + SRC, 0xF, 0xF, false));
  } else {
    static_assert(LPT == 8, "lane groups of 8, 16 or 32");
    const int lo = __builtin_amdgcn_update_dpp(0, xi, 0x150 + SRC, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, xi, 0x158 + SRC, 0xF, 0xF, false);
    return __int_as_float((threadIdx.x & 8) ? hi : lo);
  }
}

// Calls f(std::integral_constant<int, I>{}) for I = 0 .. N-1 (indices that must be
// constants, such as DPP controls).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Partial dot product of this lane's 16 bytes of K with one query row's 16 bytes.
__device__ __forceinline__ float lane_dot(const uint4& qv, const uint4& kv, bf16_t*) {
  float acc = 0.0f;
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qv.x),
                                        __builtin_bit_cast(bf16x2_t, kv.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qv.y),
                                        __builtin_bit_cast(bf16x2_t, kv.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qv.z),
                                        __builtin_bit_cast(bf16x2_t, kv.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qv.w),
                                        __builtin_bit_cast(bf16x2_t, kv.w), acc, false);
  return acc;
}
__device__ __forceinline__ float lane_dot(const uint4& qv, const uint4& kv, float*) {
  float acc = __uint_as_float(qv.x) * __uint_as_float(kv.x);
  acc = fmaf(__uint_as_float(qv.y), __uint_as_float(kv.y), acc);
  acc = fmaf(__uint_as_float(qv.z), __uint_as_float(kv.z), acc);
  acc = fmaf(__uint_as_float(qv.w), __uint_as_float(kv.w), acc);
  return acc;
}

__device__ __forceinline__ void unpack(const uint4& v, float* f, float*) {
  f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
}

// o[g][2w], o[g][2w+1] += p_a * v_a + p_b * v_b for one pair of tokens (a, b) of this
// lane, pk[g] holding (p_a, p_b) of query row g as bfloat16: v_perm_b32 pairs the two
// tokens' element of each column into one dword and v_dot2_f32_bf16 does both products
// and the accumulation.
template <int G>
__device__ __forceinline__ void pv_pair(const uint32_t* pk, const uint4& va, const uint4& vb,
                                        float (*o)[8]) {
  const uint32_t a[4] = {va.x, va.y, va.z, va.w};
  const uint32_t b[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const bf16x2_t lo = __builtin_bit_cast(bf16x2_t, __builtin_amdgcn_perm(b[w], a[w], 0x05040100u));
    const bf16x2_t hi = __builtin_bit_cast(bf16x2_t, __builtin_amdgcn_perm(b[w], a[w], 0x07060302u));
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      const bf16x2_t pg = __builtin_bit_cast(bf16x2_t, pk[gg]);
      o[gg][2 * w] = __builtin_amdgcn_fdot2_f32_bf16(pg, lo, o[gg][2 * w], false);
      o[gg][2 * w + 1] = __builtin_amdgcn_fdot2_f32_bf16(pg, hi, o[gg][2 * w + 1], false);
    }
  }
}


// Sequence length and token slots of unit u: N = cnt * g (the masked tail of a partial
// last block included, so no entry of the list has to be read first).  seq_lens and
// sel_cnt outside their ranges are clamped and, when `report`, flagged; a count above the
// unit's n_cap block slots cannot be a valid list (FX_ERR_SEL_INDEX) and is clamped to it,
// which bounds the slots of all units below 2^31 (checked at plan creation).
struct UnitTokens {
  int T, N;
};

__device__ __forceinline__ UnitTokens unit_tokens(const UnitInfo* units, const int32_t* seq_lens,
                                                  const int32_t* sel_cnt, int u, int Hkv,
                                                  int t_cap, int max_sel, bool report,
                                                  uint32_t* err) {
  const int g = units[u].g, n_cap = units[u].n_cap;
  int T = seq_lens[u / Hkv];
  int cnt = sel_cnt[u];
  if (T < 0 || T > t_cap) {
    if (report) atomicOr(err, (uint32_t)FX_ERR_SEQ_LEN);
    T = T < 0 ? 0 : t_cap;
  }
  if (cnt < 0 || cnt > max_sel) {
    if (report) atomicOr(err, (uint32_t)FX_ERR_SEL_COUNT);
    cnt = cnt < 0 ? 0 : max_sel;
  }
  if (cnt > n_cap) {
    if (report) atomicOr(err, (uint32_t)FX_ERR_SEL_INDEX);
    cnt = n_cap;
  }
  return {T, cnt * g};
}

template <typename E, int D, int G, bool ED>
struct DecodeLds {
  using SL = Slots<E, D, G>;
  // Lane groups per wave whose (o, m, l) go to LDS at the end of a piece: as many as fit in
  // the wave's slot area (a power of two); the others are first merged into them in
  // registers.
  static constexpr int keep_groups() {
    int k = 64 / SL::LPT;
    while (k > 1 && k * G * D > (64 / SL::LPT) * SL::GS) k /= 2;
    return k;
  }
  static constexpr int KEEP = keep_groups();
  static constexpr int NG = NWAVES * KEEP;        // partials merged by the workgroup
  // Per wave: its lane groups' partial dot products during the token steps, then, after
  // the wave's last step of a piece, KEEP lane groups' (o) of the query rows.  Only the
  // wave itself writes its area; a barrier separates the merge's reads from the next
  // piece's steps.
  union WaveArea {
    float tr[64 / SL::LPT][SL::GS];
    float og[KEEP][G][D];
  };
  alignas(16) WaveArea wa[NWAVES];
  int blk[kMaxSplit + 1];          // selected block indices of the current token run
  float bias[ED ? kMaxSplit + 1 : 1];   // their eviction logits times log2(e) (ED only)
  float m[NG][G];                  // each lane group's running max and sum per query row
  float l[NG][G];
  int scan[2][NWAVES];
  int scan2[2][NWAVES];
  int cuts[NWAVES];                // per wave: bit 0 the full grid, bit 1 the half grid cuts a unit
  int first_unit, first_pos;       // the unit holding the segment's first token (full grid)
  int first_unit_h, first_pos_h;   // the same on the half grid
  int unit_a, pos_a, piece_a, pieces_a, n_a;   // unit-aligned segments: unit, its first
                                               // token, piece index, piece count, tokens
};

constexpr int kScanKeep = 4;       // unit chunks (NT units each) kept in registers between scans

// Inclusive prefix sum over the workgroup (slot: NWAVES ints, written then read after one
// barrier; alternate slots between consecutive calls).
__device__ __forceinline__ int block_incl_scan(int x, int* slot, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int incl = (int)wave_scan_incl_u32((uint32_t)x);
  if (lane == 63) slot[w] = incl;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NWAVES; ++i) {
    const int v = slot[i];
    off += i < w ? v : 0;
    tot += v;
  }
  *total = tot;
  return off + incl;
}

template <typename E, int D>
__device__ __forceinline__ void write_empty_unit(E* out, float* lse, int u, int Hkv, int G) {
  const int b = u / Hkv, h = u % Hkv;
  for (int gg = 0; gg < G; ++gg) {
    const size_t orow = (size_t)b * Hkv * G + (size_t)h * G + gg;
    for (int c = 0; c < D; ++c) store_elem(out + orow * D + c, 0.0f);
    if (lse) lse[orow] = -__builtin_inff();
  }
}

// At least two waves per SIMD: without the bound the G = 8 instantiation takes 254
// registers and runs at one wave per SIMD (4 registers now spill; the mixed serving batch
// with 64 query heads decodes in 202 us instead of 238 us).  Smaller groups already fit.
template <typename E, int D, int G, int U, bool ED>
__global__ __launch_bounds__(NT, 2) void k_decode(
    const UnitInfo* __restrict__ units, const E* __restrict__ q, const E* __restrict__ K,
    const E* __restrict__ V, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ sel_cnt,
    const float* __restrict__ logits, float scale_log2,
    E* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float2* __restrict__ part_ml, int2* __restrict__ seg_rec, uint32_t* __restrict__ err,
    int Hkv, int t_cap, int max_sel, int n_units, int split) {
  constexpr int EPL = Lanes<E>::EPL;
  constexpr int LPT = D / EPL;        // lanes per token
  constexpr int TPW = 64 / LPT;       // tokens per wave instruction
  constexpr int STEP = TPW * U;       // tokens per wave per step
  static_assert(LPT >= 4 && LPT <= 32 && 64 % LPT == 0, "lane layout");
  __shared__ DecodeLds<E, D, G, ED> L;
  const int seg = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);

  // ---- Scan 1: every unit's token count and the total (errors reported here only).
  int keepN[kScanKeep];
  int mysum = 0;
  for (int c0 = 0; c0 < n_units; c0 += kScanKeep * NT) {
    int Nk[kScanKeep];
#pragma unroll
    for (int k = 0; k < kScanKeep; ++k) {
      const int u = c0 + k * NT + (int)threadIdx.x;
      Nk[k] = u < n_units ? unit_tokens(units, seq_lens, sel_cnt, u, Hkv, t_cap, max_sel, seg == 0,
                                        err).N
                          : 0;
    }
#pragma unroll
    for (int k = 0; k < kScanKeep; ++k) {
      if (c0 == 0) keepN[k] = Nk[k];
      mysum += Nk[k];
    }
  }
  int total = (int)wave_sum_u32((uint32_t)mysum);
  if (lane == 0) L.scan[0][wave] = total;
  __syncthreads();
  total = 0;
#pragma unroll
  for (int i = 0; i < NWAVES; ++i) total += L.scan[0][i];
  total = __builtin_amdgcn_readfirstlane(total);   // uniform: keep what follows scalar
  // Segments: one per workgroup of the grid, or one per workgroup of its first half
  // (dispatched first, so spread over all CUs; the second half exits after the scans)
  // when the full grid's segments would be short, or when the half grid's segments cut
  // no unit while the full grid's cut some (units of equal length, e.g. NOSA heads with a
  // fixed number of blocks: the merge of their pieces then disappears).  Fewer, longer
  // segments amortise each workgroup's fixed costs (scans, first loads, merge).
  const int Pf = gridDim.x;
  const bool can_half = Pf >= 2 * kCUsMin;
  const int Ph = can_half ? Pf >> 1 : Pf;
  const bool short_full = can_half && (total + Pf - 1) / Pf < kShortSegment;
  const int Sf = max((total + Pf - 1) / Pf, split);
  const int Sh = max((total + Ph - 1) / Ph, split);
  // (clamped: a workgroup past the last segment has no first token)
  const int s0f = (int)min((int64_t)seg * Sf, (int64_t)total);
  const int s0h = (int)min((int64_t)seg * Sh, (int64_t)total);

  // Unit-aligned segments, for plans with few units: unit u gets n_u = ceil(N_u / Sa)
  // segments of near-equal length (its pieces), Sa chosen so that the pieces of all units
  // fit the half grid.  No segment then spans two units: a segment that did paid a second
  // unit's start (query rows, block list, first loads) and a second merge after its first
  // piece, and those segments set the kernel's end (16 units over 256 segments: 27 µs
  // against a median segment end of 21.5 µs).
  const bool aligned = can_half && n_units * kAlignedUnitsDiv <= Ph && total > 0;
  const int Sa = aligned ? max((total + (Ph - n_units) - 1) / (Ph - n_units), split) : 1;

  // ---- Scan 2: prefix sums; the unit holding the segment's first token on either grid;
  // whether either grid cuts a unit; units without tokens; the aligned pieces' prefix.
  bool cut_f = false, cut_h = false;
  int running = 0, it = 0, pieces = 0;
  for (int c0 = 0; c0 < n_units; c0 += NT, ++it) {
    const int u = c0 + (int)threadIdx.x;
    int N = 0;
    if (c0 < kScanKeep * NT) {
#pragma unroll
      for (int k = 0; k < kScanKeep; ++k) N = (c0 == k * NT) ? keepN[k] : N;
    } else if (u < n_units) {
      N = unit_tokens(units, seq_lens, sel_cnt, u, Hkv, t_cap, max_sel, false, err).N;
    }
    int chunk_total;
    const int incl = running + block_incl_scan(N, L.scan[(it + 1) & 1], &chunk_total);
    const int excl = incl - N;
    if (N > 0 && excl <= s0f && s0f < incl) {
      L.first_unit = u;
      L.first_pos = excl;
    }
    if (N > 0 && excl <= s0h && s0h < incl) {
      L.first_unit_h = u;
      L.first_pos_h = excl;
    }
    if (N > 0) {
      cut_f |= excl / Sf != (incl - 1) / Sf;
      cut_h |= excl / Sh != (incl - 1) / Sh;
    }
    if (u < n_units && N == 0 && u % Pf == seg) write_empty_unit<E, D>(out, lse, u, Hkv, G);
    if (aligned) {   // workgroup-uniform
      const int na = N > 0 ? (N + Sa - 1) / Sa : 0;
      int na_total;
      const int qincl = pieces + block_incl_scan(na, L.scan2[(it + 1) & 1], &na_total);
      const int qexcl = qincl - na;
      if (na > 0 && qexcl <= seg && seg < qincl) {
        L.unit_a = u;
        L.pos_a = excl;
        L.piece_a = seg - qexcl;
        L.pieces_a = na;
        L.n_a = N;
      }
      pieces += na_total;
    }
    running += chunk_total;
  }
  // One barrier publishes both cut flags and the scan's first-unit records.
  {
    const uint64_t bf = __builtin_amdgcn_ballot_w64(cut_f);
    const uint64_t bh = __builtin_amdgcn_ballot_w64(cut_h);
    if (lane == 0) L.cuts[wave] = (bf != 0 ? 1 : 0) | (bh != 0 ? 2 : 0);
  }
  __syncthreads();
  {
    int cw = 0;
#pragma unroll
    for (int i = 0; i < NWAVES; ++i) cw |= L.cuts[i];
    cut_f = (cw & 1) != 0;
    cut_h = (cw & 2) != 0;
  }
  const bool half = short_full || (can_half && cut_f && !cut_h);
  const int S = half ? Sh : Sf;
  const int nseg = aligned ? pieces : (total + S - 1) / S;
  if (seg >= nseg) {
    if (threadIdx.x == 0) seg_rec[seg] = make_int2(-1, 0);
    return;
  }
  int s0 = half ? s0h : s0f, s1 = min(s0 + S, total);
  int u = __builtin_amdgcn_readfirstlane(half ? L.first_unit_h : L.first_unit);
  int Pu = __builtin_amdgcn_readfirstlane(half ? L.first_pos_h : L.first_pos);
  int pieces_a = 0;   // aligned: the unit's piece count (recorded by its first piece)
  if (aligned) {
    u = __builtin_amdgcn_readfirstlane(L.unit_a);
    Pu = __builtin_amdgcn_readfirstlane(L.pos_a);
    const int j = __builtin_amdgcn_readfirstlane(L.piece_a);
    pieces_a = __builtin_amdgcn_readfirstlane(L.pieces_a);
    const int n = __builtin_amdgcn_readfirstlane(L.n_a);
    s0 = Pu + (int)((int64_t)j * n / pieces_a);
    s1 = Pu + (int)((int64_t)(j + 1) * n / pieces_a);
  }

  const uint32_t lane_off = (uint32_t)(lane % LPT) * 16u;
  const int lg = lane / LPT, li = lane % LPT;
  // This lane's score slots (see Slots): where their partial dot products sit in LDS,
  // and the token u they belong to (the same for every slot of the lane).
  using SLT = Slots<E, D, G>;
  constexpr int SL = SLT::SL, QPR = SLT::QPR, SS = SLT::SS, NS = SLT::NS;
  float* const tr = &L.wa[wave].tr[lg][0];
  int slot_off[SL];
#pragma unroll
  for (int j = 0; j < SL; ++j) {
    const int k = li % SLT::SLOTW + SLT::SLOTW * j;
    slot_off[j] = (k < NS ? k : k % NS) * SS;
  }
  const int usel = lane & (U - 1);
  constexpr uint32_t kRowBytes = D * sizeof(E);
  bool recorded = false;
  int cur = s0;
  while (cur < s1) {
    const UnitTokens ut = unit_tokens(units, seq_lens, sel_cnt, u, Hkv, t_cap, max_sel, false, err);
    const int N = ut.N;
    if (N == 0) {
      ++u;
      continue;
    }
    const int T = ut.T;
    const UnitInfo ui = units[u];
    const int g = ui.g, log2g = ui.log2g;
    const bool biased = ED && ui.mode == FX_NOSA;
    const int b = u / Hkv, h = u % Hkv;
    const int32_t* sel = sel_idx + (size_t)u * max_sel;
    const int a = cur - Pu, e = min(s1, Pu + N) - Pu;   // piece [a, e) of the unit's tokens

    // Query slices: this lane's 16 bytes of each of the G rows.
    const E* qrow = q + ((size_t)b * Hkv * G + (size_t)h * G) * D + li * EPL;
    uint4 qv[G];
#pragma unroll
    for (int gg = 0; gg < G; ++gg) qv[gg] = *reinterpret_cast<const uint4*>(qrow + (size_t)gg * D);
    // Running max and sum of this lane's slots (a quad shares one query row's max; each
    // lane sums its own token u), and the output columns of every query row.
    float m[SL], l[SL], o[G][EPL == 8 ? 8 : EPL];
#pragma unroll
    for (int j = 0; j < SL; ++j) {
      m[j] = kNegBig;
      l[j] = 0.0f;
    }
#pragma unroll
    for (int gg = 0; gg < G; ++gg)
#pragma unroll
      for (int x = 0; x < EPL; ++x) o[gg][x] = 0.0f;
    // The unit's rows [0, T) of K and V as buffer resources: rows past T, and masked
    // token slots (sent to kOutOfRange), read as zeros with no memory access.
    const size_t unit_rows = (size_t)u * t_cap;
    const uint32_t nbytes = (uint32_t)T * kRowBytes;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(K + unit_rows * D), 0, (int)nbytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)(V + unit_rows * D), 0, (int)nbytes, kRsrcWord3);

    for (int c0 = a; c0 < e; c0 += kMaxSplit) {
      const int c1 = min(e, c0 + kMaxSplit);
      // Block indices this run touches; entries that are not valid blocks of the unit,
      // in ascending order, become -1 (their tokens are skipped).
      const int p0 = c0 >> log2g;
      const int np = ((c1 - 1) >> log2g) - p0 + 1;
      __syncthreads();   // the previous run's readers of L.blk are done
      for (int i = threadIdx.x; i < np; i += NT) {
        const int jb = sel[p0 + i];
        const bool ok = jb >= 0 && (int64_t)jb * g < T && (p0 + i == 0 || sel[p0 + i - 1] < jb);
        if (!ok) atomicOr(err, (uint32_t)FX_ERR_SEL_INDEX);
        L.blk[i] = ok ? jb : -1;
        if constexpr (ED) {
          float bj = biased && ok ? logits[ui.block_off + jb] : 0.0f;
          if (!__builtin_isfinite(bj)) {
            atomicOr(err, (uint32_t)FX_ERR_NONFINITE);
            bj = 0.0f;
          }
          L.bias[i] = bj * kLog2e;
        }
      }
      __syncthreads();

      // This wave's share of the run (a multiple of STEP tokens).
      const int per_wave = ((c1 - c0 + NWAVES * STEP - 1) / (NWAVES * STEP)) * STEP;
      const int w0 = c0 + wave * per_wave;
      const int w1 = min(c1, w0 + per_wave);

      auto load_step = [&](int base, uint4* kr, uint4* vr, bool* ok, float* bs) {
        // Block indices first (independent LDS reads), then all 2U buffer loads.
        int jb[U];
#pragma unroll
        for (int uu = 0; uu < U; ++uu) {
          const int i = base + uu * TPW + lg;   // i >= c0, so the slot is never negative
          const int slot = min((i >> log2g) - p0, np - 1);
          jb[uu] = L.blk[slot];
          if constexpr (ED) bs[uu] = L.bias[slot];
        }
#pragma unroll
        for (int uu = 0; uu < U; ++uu) {
          const int i = base + uu * TPW + lg;
          const int row = (jb[uu] << log2g) | (i & (g - 1));
          ok[uu] = (i < w1) & (jb[uu] >= 0) & (row < T);   // no short circuit: no branch
          const uint32_t off = ok[uu] ? (uint32_t)row * kRowBytes + lane_off : kOutOfRange;
          kr[uu] = buffer_load16(rk, off);
          vr[uu] = buffer_load16(rv, off);
        }
      };

      auto compute_step = [&](const uint4* kr, const uint4* vr, const bool* ok, const float* bs) {
        // Partial dot products to LDS (slot k = g * U + u, the group's LPT lanes side by
        // side); each lane then sums the LPT partials of its own slots.
#pragma unroll
        for (int gg = 0; gg < G; ++gg)
#pragma unroll
          for (int uu = 0; uu < U; ++uu)
            tr[(gg * U + uu) * SS + li] = lane_dot(qv[gg], kr[uu], (E*)nullptr);
        // Additive term of the lane's token: its block's eviction bias (ED) or -inf when
        // the token slot is masked.
        float term[U];
#pragma unroll
        for (int uu = 0; uu < U; ++uu) {
          float t = 0.0f;
          if constexpr (ED) t = bs[uu];
          term[uu] = ok[uu] ? t : -__builtin_inff();
        }
        float tsel = term[0];
#pragma unroll
        for (int uu = 1; uu < U; ++uu) tsel = usel == uu ? term[uu] : tsel;
        float sc[SL], mx[SL];
        bool grow = false;
#pragma unroll
        for (int j = 0; j < SL; ++j) {
          const float4* src = reinterpret_cast<const float4*>(tr + slot_off[j]);
          float acc[LPT / 4];
#pragma unroll
          for (int c = 0; c < LPT / 4; ++c) {
            const float4 v = src[c];
            acc[c] = (v.x + v.y) + (v.z + v.w);
          }
#pragma unroll
          for (int w = LPT / 8; w >= 1; w >>= 1)
#pragma unroll
            for (int c = 0; c < w; ++c) acc[c] += acc[c + w];
          sc[j] = acc[0] * scale_log2 + tsel;
          float qm = fmaxf(sc[j], dpp_f<kQuadPerm1032>(sc[j]));
          qm = fmaxf(qm, dpp_f<kQuadPerm2301>(qm));
          mx[j] = fmaxf(m[j], qm);
          grow |= mx[j] > m[j];
        }
        // Rescale o and l only when some running max of the wave grew (a wave-uniform
        // branch); otherwise every alpha would be exactly 1.
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(grow) != 0, 0)) {
          // Keep this a branch: if-converting it would run the rescale every step.
          asm volatile("" ::: "memory");
          float alpha[SL];
#pragma unroll
          for (int j = 0; j < SL; ++j) {
            alpha[j] = __builtin_amdgcn_exp2f(m[j] - mx[j]);
            m[j] = mx[j];
            l[j] *= alpha[j];
          }
          static_for<0, G>([&](auto gc) {
            constexpr int gg = decltype(gc)::value;
            const float al = group_bcast<LPT, (gg % QPR) * U>(alpha[gg / QPR]);
#pragma unroll
            for (int x = 0; x < EPL; ++x) o[gg][x] *= al;
          });
        }
        float p[SL];
#pragma unroll
        for (int j = 0; j < SL; ++j) {
          p[j] = __builtin_amdgcn_exp2f(sc[j] - m[j]);
          l[j] += p[j];
        }
        if constexpr (sizeof(E) == 2) {
          static_assert(U % 2 == 0, "token pairs");
          // bfloat16 pairs (p_u, p_u+1) of the lane's query row, complete in lanes of even u.
          uint32_t pk[SL];
#pragma unroll
          for (int j = 0; j < SL; ++j) {
            const float nb = dpp_f<kQuadPerm1032>(p[j]);
            pk[j] = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)p[j], (__bf16)nb});
          }
          static_for<0, U / 2>([&](auto pc) {
            constexpr int u0 = 2 * decltype(pc)::value;
            uint32_t pb[G];
            static_for<0, G>([&](auto gc) {
              constexpr int gg = decltype(gc)::value;
              pb[gg] = __float_as_uint(
                  group_bcast<LPT, (gg % QPR) * U + u0>(__uint_as_float(pk[gg / QPR])));
            });
            pv_pair<G>(pb, vr[u0], vr[u0 + 1], o);
          });
        } else {
          static_for<0, U>([&](auto uc) {
            constexpr int uu = decltype(uc)::value;
            float vf[EPL];
            unpack(vr[uu], vf, (E*)nullptr);
            static_for<0, G>([&](auto gc) {
              constexpr int gg = decltype(gc)::value;
              const float pb = group_bcast<LPT, (gg % QPR) * U + uu>(p[gg / QPR]);
#pragma unroll
              for (int x = 0; x < EPL; ++x) o[gg][x] = fmaf(pb, vf[x], o[gg][x]);
            });
          });
        }
      };

      // Register double buffering: the loads of step n+1 are in flight while step n
      // computes.  Inside the loop every step's loads are issued unconditionally, so the
      // count of outstanding loads is the same on every path and each compute waits only
      // for its own step's loads; the last one or two steps are peeled, so no load is
      // issued past the run (such loads read nothing, but the epilogue would wait for
      // them: qwen7b_layer's decode 0.5 us longer).
      uint4 kA[U], vA[U], kB[U], vB[U];
      bool okA[U], okB[U];
      float bA[U], bB[U];   // ED only
      if (w0 < w1) {
        load_step(w0, kA, vA, okA, bA);
        int base = w0;
        for (; base + 2 * STEP < w1; base += 2 * STEP) {
          load_step(base + STEP, kB, vB, okB, bB);
          compute_step(kA, vA, okA, bA);
          load_step(base + 2 * STEP, kA, vA, okA, bA);
          compute_step(kB, vB, okB, bB);
        }
        if (base + STEP < w1) {   // two steps left
          load_step(base + STEP, kB, vB, okB, bB);
          compute_step(kA, vA, okA, bA);
          compute_step(kB, vB, okB, bB);
        } else {
          compute_step(kA, vA, okA, bA);
        }
      }
    }

    // Every lane of a group takes the group's (m, l) of each query row: m from the row's
    // quad, l summed over the quad's tokens.
    float mf[G], lf[G];
    {
      float lq[SL];
#pragma unroll
      for (int j = 0; j < SL; ++j) {
        const float t = l[j] + dpp_f<kQuadPerm1032>(l[j]);
        lq[j] = t + dpp_f<kQuadPerm2301>(t);
      }
      static_for<0, G>([&](auto gc) {
        constexpr int gg = decltype(gc)::value;
        mf[gg] = group_bcast<LPT, (gg % QPR) * U>(m[gg / QPR]);
        lf[gg] = group_bcast<LPT, (gg % QPR) * U>(lq[gg / QPR]);
      });
    }
    // Merge the lane groups of the wave down to KEEP (partners differ in the lane bits
    // from LPT * KEEP up).  Those publish their (o, m, l); after the barrier the workgroup
    // merges all NG of them in (wave, group) order, four columns per thread.  Merging all
    // the lane groups in registers took a chain of cross-lane shuffles per query row
    // (1.7 us per wave with seven rows and four groups), every wave of the workgroup then
    // waiting at the barrier.
    constexpr int KEEP = DecodeLds<E, D, G, ED>::KEEP;
#pragma unroll
    for (int off = LPT * KEEP; off < 64; off <<= 1) {
#pragma unroll
      for (int gg = 0; gg < G; ++gg) {
        const float m2 = __shfl_xor(mf[gg], off);
        const float l2 = __shfl_xor(lf[gg], off);
        const float M = fmaxf(mf[gg], m2);
        const float x = __builtin_amdgcn_exp2f(mf[gg] - M);
        const float y = __builtin_amdgcn_exp2f(m2 - M);
        lf[gg] = lf[gg] * x + l2 * y;
#pragma unroll
        for (int z = 0; z < EPL; ++z) {
          const float o2 = __shfl_xor(o[gg][z], off);
          o[gg][z] = o[gg][z] * x + o2 * y;
        }
        mf[gg] = M;
      }
    }
    if (lg < KEEP) {
      float* og = &L.wa[wave].og[lg][0][0];
#pragma unroll
      for (int gg = 0; gg < G; ++gg)
#pragma unroll
        for (int z = 0; z < EPL; z += 4)
          *reinterpret_cast<float4*>(og + gg * D + li * EPL + z) =
              make_float4(o[gg][z], o[gg][z + 1], o[gg][z + 2], o[gg][z + 3]);
      if (li == 0) {
#pragma unroll
        for (int gg = 0; gg < G; ++gg) {
          L.m[wave * KEEP + lg][gg] = mf[gg];
          L.l[wave * KEEP + lg][gg] = lf[gg];
        }
      }
    }
    __syncthreads();

    // Finish the unit or publish a partial.
    const bool whole = a == 0 && e == N;
    const size_t pbase = (size_t)seg * 2 + (a == 0 ? 1 : 0);
    for (int idx = threadIdx.x; idx < G * D / 4; idx += NT) {
      constexpr int NG = DecodeLds<E, D, G, ED>::NG;
      const int gg = idx / (D / 4), c = (idx % (D / 4)) * 4;
      float M = L.m[0][gg];
#pragma unroll
      for (int k = 1; k < NG; ++k) M = fmaxf(M, L.m[k][gg]);
      float Ls = 0.0f;
      float4 Os = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
      for (int k = 0; k < NG; ++k) {
        const float x = __builtin_amdgcn_exp2f(L.m[k][gg] - M);
        const float4 ov = *reinterpret_cast<const float4*>(&L.wa[k / KEEP].og[k % KEEP][gg][c]);
        Ls = fmaf(L.l[k][gg], x, Ls);
        Os.x = fmaf(ov.x, x, Os.x);
        Os.y = fmaf(ov.y, x, Os.y);
        Os.z = fmaf(ov.z, x, Os.z);
        Os.w = fmaf(ov.w, x, Os.w);
      }
      if (whole) {
        const size_t orow = (size_t)b * Hkv * G + (size_t)h * G + gg;
        E* dst = out + orow * D + c;
        store_elem(dst + 0, Ls > 0.0f ? Os.x / Ls : 0.0f);
        store_elem(dst + 1, Ls > 0.0f ? Os.y / Ls : 0.0f);
        store_elem(dst + 2, Ls > 0.0f ? Os.z / Ls : 0.0f);
        store_elem(dst + 3, Ls > 0.0f ? Os.w / Ls : 0.0f);
        if (lse && c == 0) lse[orow] = Ls > 0.0f ? (M + __log2f(Ls)) * kLn2 : -__builtin_inff();
      } else {
        *reinterpret_cast<float4*>(&part_o[(pbase * G + gg) * D + c]) = Os;
        if (c == 0) part_ml[pbase * G + gg] = make_float2(M, Ls);
      }
    }
    if (a == 0 && e < N) {
      // The unit continues in the following segments: its pieces are this segment's
      // tail slot and the head slots of segments seg+1 .. seg+n-1.
      if (threadIdx.x == 0)
        seg_rec[seg] = make_int2(u, aligned ? pieces_a : (Pu + N - 1) / S - seg + 1);
      recorded = true;
    }
    cur = Pu + e;
    Pu += N;
    ++u;
  }
  if (!recorded && threadIdx.x == 0) seg_rec[seg] = make_int2(-1, 0);
}

// Partial slot of piece k of the unit recorded by segment s.
__device__ __forceinline__ size_t piece_slot(int s, int k) {
  return k == 0 ? (size_t)s * 2 + 1 : (size_t)(s + k) * 2;
}

// One workgroup per segment with one thread per output (query row, column); each thread
// merges its own pieces in piece order, eight at a time (all sixteen loads in flight), with a
// running max: M = max m_k, L = sum l_k 2^(m_k - M), out = sum o_k 2^(m_k - M) / L.
// No LDS and no barriers; the (m, l) loads repeat across a row's threads and hit the
// cache.
constexpr int kMergeBatch = 8;

template <typename E, int D, int G>
__global__ __launch_bounds__(1024) void k_combine(
    const int2* __restrict__ seg_rec, E* __restrict__ out, float* __restrict__ lse,
    const float* __restrict__ part_o, const float2* __restrict__ part_ml, int Hkv) {
  const int s = blockIdx.x;
  const int2 rec = seg_rec[s];
  if (rec.x < 0) return;
  const int u = rec.x, nk = min(rec.y, (int)gridDim.x - s);
  const int b = u / Hkv, h = u % Hkv;
  for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
    const int gg = idx / D, c = idx % D;
    float M = kNegBig, Lt = 0.0f, acc = 0.0f;
    for (int k0 = 0; k0 < nk; k0 += kMergeBatch) {
      float2 ml[kMergeBatch];
      float ov[kMergeBatch];
#pragma unroll
      for (int j = 0; j < kMergeBatch; ++j) {
        const int k = k0 + j;
        if (k < nk) {
          const size_t slot = piece_slot(s, k);
          ml[j] = part_ml[slot * G + gg];
          ov[j] = part_o[slot * G * D + idx];
        } else {
          ml[j] = make_float2(kNegBig, 0.0f);
          ov[j] = 0.0f;
        }
      }
      float Mn = M;
#pragma unroll
      for (int j = 0; j < kMergeBatch; ++j) Mn = fmaxf(Mn, ml[j].x);
      const float r = __builtin_amdgcn_exp2f(M - Mn);
      Lt *= r;
      acc *= r;
      M = Mn;
#pragma unroll
      for (int j = 0; j < kMergeBatch; ++j) {
        const float wgt = __builtin_amdgcn_exp2f(ml[j].x - M);
        Lt = fmaf(ml[j].y, wgt, Lt);
        acc = fmaf(ov[j], wgt, acc);
      }
    }
    const size_t orow = (size_t)b * Hkv * G + (size_t)h * G + gg;
    store_elem(out + orow * D + c, Lt > 0.0f ? acc / Lt : 0.0f);
    if (lse && c == 0) lse[orow] = Lt > 0.0f ? (M + __log2f(Lt)) * kLn2 : -__builtin_inff();
  }
}

template <typename E, int D, int G>
int launch_t(const fx_plan* p, const void* q, const void* K, const void* V,
             const int32_t* seq_lens, const int32_t* sel_idx, const int32_t* sel_cnt,
             const float* logits, float softmax_scale, void* out, float* lse, void* scratch,
             hipStream_t stream) {
  const int Hkv = p->desc.num_kv_heads, t_cap = p->desc.t_cap;
  const dim3 grid((unsigned)(logits ? p->decode_grid_ed : p->decode_grid));
  char* base = static_cast<char*>(scratch);
  float* part_o = reinterpret_cast<float*>(base + p->ws_decode.part_o);
  float2* part_ml = reinterpret_cast<float2*>(base + p->ws_decode.part_ml);
  int2* seg_rec = reinterpret_cast<int2*>(base + p->ws_decode.seg);
  // Every argument but the logits is the same for both instantiations.
  auto args = [&](auto kernel) {
    kernel<<<grid, NT, 0, stream>>>(
        p->d_units, static_cast<const E*>(q), static_cast<const E*>(K),
        static_cast<const E*>(V), seq_lens, sel_idx, sel_cnt, logits, softmax_scale * kLog2e,
        static_cast<E*>(out), lse, part_o, part_ml, seg_rec, p->d_error, Hkv, t_cap, p->max_sel,
        p->units, p->decode_split);
  };
  if (logits)
    args(k_decode<E, D, G, kU, true>);
  else
    args(k_decode<E, D, G, kU, false>);
  const int e = hipGetLastError();
  if (e != 0 || p->decode_uncut) return e;   // uncut plans finish every unit in place
  // One thread per output (query row, column).
  constexpr int kCombineThreads = G * D < 1024 ? G * D : 1024;
  k_combine<E, D, G><<<grid, kCombineThreads, 0, stream>>>(
      seg_rec, static_cast<E*>(out), lse, part_o, part_ml, Hkv);
  return hipGetLastError();
}

// Resident decode workgroups per CU, at most: small groups fit three, but the mixed
// serving batch (G = 4) decodes in 141 us with two per CU against 143 us with three, and
// the NOSA batch in 95 us against 100 us (three cut its equal units into pieces).
constexpr int kMaxDecodeWgsPerCu = 2;

template <typename E, int D, int G, bool ED>
int grid_t() {
  int per_cu = 0, cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(&k_decode<E, D, G, kU, ED>), NT, 0) !=
          hipSuccess)
    return 0;
  return (per_cu < kMaxDecodeWgsPerCu ? per_cu : kMaxDecodeWgsPerCu) * cus;
}

// Calls f.template operator()<E, D, G>() for the plan's element type, head dim and group.
template <typename F>
auto with_shape(const fx_plan* p, F&& f) {
  auto by_g = [&](auto e_tag, auto d_tag) {
    using E = typename decltype(e_tag)::type;
    constexpr int D = decltype(d_tag)::value;
    switch (p->G) {
      case 1: return f.template operator()<E, D, 1>();
      case 2: return f.template operator()<E, D, 2>();
      case 3: return f.template operator()<E, D, 3>();
      case 4: return f.template operator()<E, D, 4>();
      case 5: return f.template operator()<E, D, 5>();
      case 6: return f.template operator()<E, D, 6>();
      case 7: return f.template operator()<E, D, 7>();
      default: return f.template operator()<E, D, 8>();
    }
  };
  struct Bf { using type = bf16_t; };
  struct Fl { using type = float; };
  if (p->desc.dtype == FX_BF16)
    return p->desc.head_dim == 128 ? by_g(Bf{}, std::integral_constant<int, 128>{})
                                   : by_g(Bf{}, std::integral_constant<int, 64>{});
  return p->desc.head_dim == 128 ? by_g(Fl{}, std::integral_constant<int, 128>{})
                                 : by_g(Fl{}, std::integral_constant<int, 64>{});
}

struct GridFn {
  bool ed;
  template <typename E, int D, int G>
  int operator()() const { return ed ? grid_t<E, D, G, true>() : grid_t<E, D, G, false>(); }
};

struct LaunchFn {
  const fx_plan* p;
  const void *q, *K, *V;
  const int32_t *seq_lens, *sel_idx, *sel_cnt;
  const float* logits;
  float softmax_scale;
  void* out;
  float* lse;
  void* scratch;
  hipStream_t stream;
  template <typename E, int D, int G>
  int operator()() const {
    return launch_t<E, D, G>(p, q, K, V, seq_lens, sel_idx, sel_cnt, logits, softmax_scale, out,
                             lse, scratch, stream);
  }
};

}  // namespace

// Decode scratch for the entry point that allocates nothing (fx_sparse_decode_noalloc):
// one array per GPU in the library's code object, shared by every call on that GPU.
// Host code never uses the array's name as an address: the device address comes from
// hipGetSymbolAddress, once per device, at plan creation (dev_static_scratch).
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

int decode_grid(const fx_plan* p, bool ed) { return with_shape(p, GridFn{ed}); }

int launch_decode(const fx_plan* p, const void* q, const void* K, const void* V,
                  const int32_t* seq_lens, const int32_t* sel_idx, const int32_t* sel_cnt,
                  const float* logits, float softmax_scale, void* out, float* lse, void* scratch,
                  hipStream_t stream) {
  if (p->G < 1 || p->G > kMaxGroup) return hipErrorInvalidValue;
  return with_shape(p, LaunchFn{p, q, K, V, seq_lens, sel_idx, sel_cnt, logits, softmax_scale,
                                out, lse, scratch, stream});
}

void* dev_static_scratch(size_t* bytes) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  *bytes = kStaticScratchBytes;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    addr[dev] = ptr;
  }
  return addr[dev];
}

}  // namespace fx
