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
// The selected tokens of a unit are numbered i = 0 .. N-1 in ascending order; because
// only the last block of a unit can be partial and selections are ascending, token i
// lives in selected block i / g at offset i % g.  A unit's N tokens are cut into
// nchunks = ceil(N / split) chunks of equal length (rounded up to 16 tokens), one
// workgroup each (grid = units x stride, stride = max_chunks rounded up to an odd
// number; chunks past the unit's count exit at once).  A unit's chunks are adjacent
// workgroups, so the machine sweeps the K/V cache roughly unit by unit.  Workgroup i
// runs on XCD i mod 8; with an odd stride the first chunk of unit u (present for every
// unit) lands on XCD (u * stride) mod 8, which cycles through all eight XCDs, where an
// even stride would pile the first chunks onto a few of them.
//
// k_decode (4 waves per chunk): a token's d-vector is spread over LPT lanes, each lane
// holding 16 bytes (8 bfloat16 / 4 float32) of the K and V rows, so every load is a
// 128-bit load and each wave instruction reads 64/LPT whole rows.  K and V are read
// through raw buffer resources bounded to the unit's T valid rows: masked token slots
// get an out-of-range offset and read zeros without a branch or a memory access.
// Loads for the next step of U tokens per lane group are issued before the current
// step is computed (register double buffering), so two steps are in flight per wave.
// Each lane keeps the G query rows' matching 16 bytes in registers, forms G partial
// dot products (v_dot2_f32_bf16 for bfloat16) and DPP-reduces them across its LPT
// lanes.  The online softmax runs in base 2 (scores pre-multiplied by scale*log2(e))
// per lane group, rescaling o and l only in steps where some running max grew.  For
// bfloat16 the P.V update takes tokens in pairs: p is rounded to bfloat16 and one
// v_dot2_f32_bf16 per (row, column) accumulates both tokens.  Lane groups, then waves,
// merge with the log-sum-exp rule.  A unit with one chunk writes `out` directly;
// otherwise each chunk writes its unnormalised (o, m, l).
//
// k_combine (one workgroup per unit with more than one chunk) merges the chunk
// partials: per query row the max M and the weighted sum L come from workgroup
// reductions in a fixed order, the per-chunk weights 2^(m_k - M) sit in LDS, and each
// output sums its chunks in chunk order, so results do not depend on scheduling.  The kernel
// boundary makes every chunk's partial visible to it; no fence is needed inside
// k_decode (an agent-scope fence per workgroup would write back the L2 each time).
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
// lane, with p rounded to bfloat16: v_perm_b32 pairs the two tokens' element of each
// column into one dword and v_dot2_f32_bf16 does both products and the accumulation.
template <int G>
__device__ __forceinline__ void pv_pair(const float* pa, const float* pb, const uint4& va,
                                        const uint4& vb, float (*o)[8]) {
  bf16x2_t pk[G];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) pk[gg] = bf16x2_t{(__bf16)pa[gg], (__bf16)pb[gg]};
  const uint32_t a[4] = {va.x, va.y, va.z, va.w};
  const uint32_t b[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const bf16x2_t lo = __builtin_bit_cast(bf16x2_t, __builtin_amdgcn_perm(b[w], a[w], 0x05040100u));
    const bf16x2_t hi = __builtin_bit_cast(bf16x2_t, __builtin_amdgcn_perm(b[w], a[w], 0x07060302u));
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      o[gg][2 * w] = __builtin_amdgcn_fdot2_f32_bf16(pk[gg], lo, o[gg][2 * w], false);
      o[gg][2 * w + 1] = __builtin_amdgcn_fdot2_f32_bf16(pk[gg], hi, o[gg][2 * w + 1], false);
    }
  }
}


// Selected-token count of a unit and its chunk count (identical in both kernels).
struct UnitSpan {
  int T, cnt, N, nchunks;
  int clen;    // tokens per chunk: N split evenly, rounded up to 16; the last chunk is shorter
};

__device__ __forceinline__ UnitSpan unit_span(const UnitInfo& ui, const int32_t* seq_lens,
                                              const int32_t* sel, const int32_t* sel_cnt, int u,
                                              int b, int t_cap, int max_sel, int split,
                                              int log2split, int max_chunks, uint32_t* err) {
  UnitSpan s;
  s.T = load_seq_len(seq_lens, b, t_cap, err);
  int cnt = sel_cnt[u];
  if (cnt < 0 || cnt > max_sel) {
    if (threadIdx.x == 0) atomicOr(err, (uint32_t)FX_ERR_SEL_COUNT);
    cnt = cnt < 0 ? 0 : max_sel;
  }
  s.cnt = cnt;
  int N = 0;
  if (cnt > 0) {
    const int last = sel[cnt - 1];
    const int valid_last = min(max(s.T - last * ui.g, 0), ui.g);
    N = (cnt - 1) * ui.g + valid_last;
  }
  if (N > max_chunks * split) {   // only for selections that are not valid for this unit
    if (threadIdx.x == 0) atomicOr(err, (uint32_t)FX_ERR_SEL_INDEX);
    N = max_chunks * split;
  }
  s.N = N;
  s.nchunks = N > 0 ? ((N + split - 1) >> log2split) : 1;
  s.clen = min(split, ((N + s.nchunks - 1) / s.nchunks + 15) & ~15);
  return s;
}

template <typename E, int D, int G>
struct DecodeLds {
  int blk[kMaxSplit + 1];          // selected block indices covering this chunk
  float o[NWAVES][G][D];
  float m[NWAVES][G];
  float l[NWAVES][G];
};

template <typename E, int D, int G, int U>
__global__ __launch_bounds__(NT) void k_decode(
    const UnitInfo* __restrict__ units, const E* __restrict__ q, const E* __restrict__ K,
    const E* __restrict__ V, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ sel_cnt, float scale_log2,
    E* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float2* __restrict__ part_ml, uint32_t* __restrict__ err, int Hkv, int t_cap, int max_sel,
    int split, int log2split, int max_chunks) {
  constexpr int EPL = Lanes<E>::EPL;
  constexpr int LPT = D / EPL;        // lanes per token
  constexpr int TPW = 64 / LPT;       // tokens per wave instruction
  constexpr int STEP = TPW * U;       // tokens per wave per step
  static_assert(LPT >= 4 && LPT <= 32 && 64 % LPT == 0, "lane layout");
  __shared__ DecodeLds<E, D, G> L;

  const int stride = max_chunks | 1;
  const int u = blockIdx.x / stride;
  const int chunk = blockIdx.x % stride;
  const UnitInfo ui = units[u];
  const int b = u / Hkv, h = u % Hkv;
  const int32_t* sel = sel_idx + (size_t)u * max_sel;
  const UnitSpan sp = unit_span(ui, seq_lens, sel, sel_cnt, u, b, t_cap, max_sel, split,
                                log2split, max_chunks, err);
  if (chunk >= sp.nchunks) return;
  const int T = sp.T, g = ui.g, log2g = ui.log2g;

  const int i0 = chunk * sp.clen;
  const int i1 = min(sp.N, i0 + sp.clen);
  // Block indices this chunk touches; entries that are not valid blocks of the unit, in
  // ascending order, become -1 (their tokens are skipped).
  const int p0 = i0 >> log2g;
  const int np = i1 > i0 ? ((i1 - 1) >> log2g) - p0 + 1 : 0;
  for (int i = threadIdx.x; i < np; i += NT) {
    const int jb = sel[p0 + i];
    const bool ok = jb >= 0 && (int64_t)jb * g < T && (p0 + i == 0 || sel[p0 + i - 1] < jb);
    if (!ok) atomicOr(err, (uint32_t)FX_ERR_SEL_INDEX);
    L.blk[i] = ok ? jb : -1;
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lg = lane / LPT, li = lane % LPT;

  // Query slices: this lane's 16 bytes of each of the G rows.
  const size_t unit_rows = (size_t)u * t_cap;
  const E* qrow = q + ((size_t)b * Hkv * G + (size_t)h * G) * D + li * EPL;
  uint4 qv[G];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) qv[gg] = *reinterpret_cast<const uint4*>(qrow + (size_t)gg * D);

  float m[G], l[G], o[G][EPL == 8 ? 8 : EPL];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    m[gg] = kNegBig;
    l[gg] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[gg][e] = 0.0f;
  }

  // This wave's share of the chunk (a multiple of STEP tokens).
  const int per_wave = ((sp.clen + NWAVES * STEP - 1) / (NWAVES * STEP)) * STEP;
  const int w0 = i0 + wave * per_wave;
  const int w1 = min(i1, w0 + per_wave);
  // The unit's rows [0, T) of K and V as buffer resources: rows past T, and masked
  // token slots (sent to kOutOfRange), read as zeros with no memory access.
  constexpr uint32_t kRowBytes = D * sizeof(E);
  const uint32_t nbytes = (uint32_t)T * kRowBytes;
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)(K + unit_rows * D), 0, (int)nbytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void*)(V + unit_rows * D), 0, (int)nbytes, kRsrcWord3);
  const uint32_t lane_off = (uint32_t)li * 16u;

  auto load_step = [&](int base, uint4* kr, uint4* vr, bool* ok) {
    // Block indices first (independent LDS reads), then all 2U buffer loads.
    int jb[U];
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      const int i = base + uu * TPW + lg;
      jb[uu] = L.blk[max(0, min((i >> log2g) - p0, np - 1))];
    }
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      const int i = base + uu * TPW + lg;
      const int row = jb[uu] * g + (i & (g - 1));
      ok[uu] = i < w1 && jb[uu] >= 0 && row < T;
      const uint32_t off = ok[uu] ? (uint32_t)row * kRowBytes + lane_off : kOutOfRange;
      kr[uu] = buffer_load16(rk, off);
      vr[uu] = buffer_load16(rv, off);
    }
  };

  auto compute_step = [&](const uint4* kr, const uint4* vr, const bool* ok) {
    float s[U][G];
#pragma unroll
    for (int uu = 0; uu < U; ++uu)
#pragma unroll
      for (int gg = 0; gg < G; ++gg) s[uu][gg] = lane_dot(qv[gg], kr[uu], (E*)nullptr);
#pragma unroll
    for (int uu = 0; uu < U; ++uu)
#pragma unroll
      for (int gg = 0; gg < G; ++gg) {
        const float t = group_sum<LPT>(s[uu][gg]) * scale_log2;
        s[uu][gg] = ok[uu] ? t : -__builtin_inff();
      }
    // Rescale o and l only when some running max of the wave grew (a wave-uniform
    // branch); otherwise every alpha would be exactly 1.
    float mx[G];
    bool grow = false;
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      mx[gg] = m[gg];
#pragma unroll
      for (int uu = 0; uu < U; ++uu) mx[gg] = fmaxf(mx[gg], s[uu][gg]);
      grow |= mx[gg] > m[gg];
    }
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(grow) != 0, 0)) {
      // Keep this a branch: if-converting it would run the rescale every step.
      asm volatile("" ::: "memory");
#pragma unroll
      for (int gg = 0; gg < G; ++gg) {
        const float alpha = __builtin_amdgcn_exp2f(m[gg] - mx[gg]);
        m[gg] = mx[gg];
        l[gg] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[gg][e] *= alpha;
      }
    }
    float p[U][G];
#pragma unroll
    for (int uu = 0; uu < U; ++uu)
#pragma unroll
      for (int gg = 0; gg < G; ++gg) {
        p[uu][gg] = __builtin_amdgcn_exp2f(s[uu][gg] - m[gg]);
        l[gg] += p[uu][gg];
      }
    if constexpr (sizeof(E) == 2) {
      static_assert(U % 2 == 0, "token pairs");
#pragma unroll
      for (int uu = 0; uu < U; uu += 2) pv_pair<G>(p[uu], p[uu + 1], vr[uu], vr[uu + 1], o);
    } else {
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        float vf[EPL];
        unpack(vr[uu], vf, (E*)nullptr);
#pragma unroll
        for (int gg = 0; gg < G; ++gg)
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[gg][e] = fmaf(p[uu][gg], vf[e], o[gg][e]);
      }
    }
  };

  // Register double buffering: the loads of step n+1 are in flight while step n
  // computes.  The loads are issued unconditionally (slots past w1 are out of range and
  // cost no memory traffic) so the count of outstanding loads is the same on every path
  // and each compute waits only for its own step's loads.
  uint4 kA[U], vA[U], kB[U], vB[U];
  bool okA[U], okB[U];
  if (w0 < w1) {
    load_step(w0, kA, vA, okA);
    for (int base = w0; base < w1; base += 2 * STEP) {
      load_step(base + STEP, kB, vB, okB);
      compute_step(kA, vA, okA);
      load_step(base + 2 * STEP, kA, vA, okA);
      if (base + STEP < w1) compute_step(kB, vB, okB);
    }
  }

  // Merge the lane groups of the wave (partners differ in the lane bits above LPT).
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      const float m2 = __shfl_xor(m[gg], off);
      const float l2 = __shfl_xor(l[gg], off);
      const float M = fmaxf(m[gg], m2);
      const float a = __builtin_amdgcn_exp2f(m[gg] - M);
      const float c = __builtin_amdgcn_exp2f(m2 - M);
      l[gg] = l[gg] * a + l2 * c;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float o2 = __shfl_xor(o[gg][e], off);
        o[gg][e] = o[gg][e] * a + o2 * c;
      }
      m[gg] = M;
    }
  }
  if (lg == 0) {
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) L.o[wave][gg][li * EPL + e] = o[gg][e];
      if (li == 0) {
        L.m[wave][gg] = m[gg];
        L.l[wave][gg] = l[gg];
      }
    }
  }
  __syncthreads();

  // Merge the waves in wave order; then either finish the unit or publish a partial.
  const bool single = sp.nchunks == 1;
  const size_t pbase = (size_t)u * max_chunks + chunk;
  for (int idx = threadIdx.x; idx < G * D; idx += NT) {
    const int gg = idx / D, c = idx % D;
    float M = L.m[0][gg];
#pragma unroll
    for (int w = 1; w < NWAVES; ++w) M = fmaxf(M, L.m[w][gg]);
    float Ls = 0.0f, Os = 0.0f;
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) {
      const float a = __builtin_amdgcn_exp2f(L.m[w][gg] - M);
      Ls = fmaf(L.l[w][gg], a, Ls);
      Os = fmaf(L.o[w][gg][c], a, Os);
    }
    if (single) {
      const size_t orow = (size_t)b * Hkv * G + (size_t)h * G + gg;
      store_elem(out + orow * D + c, Ls > 0.0f ? Os / Ls : 0.0f);
      if (lse && c == 0) lse[orow] = Ls > 0.0f ? (M + __log2f(Ls)) * kLn2 : -__builtin_inff();
    } else {
      part_o[(pbase * G + gg) * D + c] = Os;
      if (c == 0) part_ml[pbase * G + gg] = make_float2(M, Ls);
    }
  }
}

// Reductions over the 256 threads of a workgroup (lds: NWAVES floats).
__device__ __forceinline__ float block_max(float x, float* lds) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = lds[0];
#pragma unroll
  for (int w = 1; w < NWAVES; ++w) r = fmaxf(r, lds[w]);
  __syncthreads();
  return r;
}
__device__ __forceinline__ float block_sum_f(float x, float* lds) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = 0.0f;
#pragma unroll
  for (int w = 0; w < NWAVES; ++w) r += lds[w];   // fixed order: deterministic
  __syncthreads();
  return r;
}

constexpr int kCombineTile = 256;   // chunks whose weights sit in LDS at a time

template <typename E, int D, int G>
__global__ __launch_bounds__(NT) void k_combine(
    const UnitInfo* __restrict__ units, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ sel_cnt,
    E* __restrict__ out, float* __restrict__ lse, const float* __restrict__ part_o,
    const float2* __restrict__ part_ml, uint32_t* __restrict__ err, int Hkv, int t_cap,
    int max_sel, int split, int log2split, int max_chunks) {
  constexpr int OUTS = (G * D + NT - 1) / NT;   // outputs per thread
  __shared__ float red[NWAVES];
  __shared__ float Mg[G], Lg[G];
  __shared__ float wts[kCombineTile][G];
  const int u = blockIdx.x;
  const UnitInfo ui = units[u];
  const int b = u / Hkv, h = u % Hkv;
  const UnitSpan sp = unit_span(ui, seq_lens, sel_idx + (size_t)u * max_sel, sel_cnt, u, b,
                                t_cap, max_sel, split, log2split, max_chunks, err);
  if (sp.nchunks == 1) return;   // k_decode already wrote this unit
  const int nk = sp.nchunks;
  const float2* ml = part_ml + (size_t)u * max_chunks * G;
  const float* po = part_o + (size_t)u * max_chunks * G * D;

  // Per query row: M = max over chunks of m, L = sum over chunks of l * 2^(m - M).
  for (int gg = 0; gg < G; ++gg) {
    float mx = kNegBig;
    for (int k = threadIdx.x; k < nk; k += NT) mx = fmaxf(mx, ml[(size_t)k * G + gg].x);
    const float M = block_max(mx, red);
    float ls = 0.0f;
    for (int k = threadIdx.x; k < nk; k += NT) {
      const float2 v = ml[(size_t)k * G + gg];
      ls += v.y * __builtin_amdgcn_exp2f(v.x - M);
    }
    const float L = block_sum_f(ls, red);
    if (threadIdx.x == 0) {
      Mg[gg] = M;
      Lg[gg] = L;
    }
  }
  __syncthreads();

  // out = sum over chunks of o_k * 2^(m_k - M) / L, chunks taken in order.
  float acc[OUTS];
#pragma unroll
  for (int j = 0; j < OUTS; ++j) acc[j] = 0.0f;
  for (int k0 = 0; k0 < nk; k0 += kCombineTile) {
    const int kt = min(kCombineTile, nk - k0);
    for (int i = threadIdx.x; i < kt * G; i += NT) {
      const int k = i / G, gg = i % G;
      wts[k][gg] = __builtin_amdgcn_exp2f(ml[(size_t)(k0 + k) * G + gg].x - Mg[gg]);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < OUTS; ++j) {
      const int idx = threadIdx.x + j * NT;
      if (idx < G * D) {
        const int gg = idx / D;
        const float* src = po + (size_t)k0 * G * D + idx;
        float a = acc[j];
#pragma unroll 8
        for (int k = 0; k < kt; ++k) a = fmaf(src[(size_t)k * G * D], wts[k][gg], a);
        acc[j] = a;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < OUTS; ++j) {
    const int idx = threadIdx.x + j * NT;
    if (idx < G * D) {
      const int gg = idx / D, c = idx % D;
      const float L = Lg[gg];
      const size_t orow = (size_t)b * Hkv * G + (size_t)h * G + gg;
      store_elem(out + orow * D + c, L > 0.0f ? acc[j] / L : 0.0f);
      if (lse && c == 0) lse[orow] = L > 0.0f ? (Mg[gg] + __log2f(L)) * kLn2 : -__builtin_inff();
    }
  }
}

template <typename E, int D, int G>
hipError_t launch_t(const fx_plan* p, const void* q, const void* K, const void* V,
                    const int32_t* seq_lens, const int32_t* sel_idx, const int32_t* sel_cnt,
                    float softmax_scale, void* out, float* lse, float* part_o, float* part_ml,
                    hipStream_t stream) {
  constexpr int U = 4;
  const int Hkv = p->desc.num_kv_heads, t_cap = p->desc.t_cap;
  const dim3 grid((unsigned)((int64_t)p->units * (p->max_chunks | 1)));
  k_decode<E, D, G, U><<<grid, NT, 0, stream>>>(
      p->d_units, static_cast<const E*>(q), static_cast<const E*>(K), static_cast<const E*>(V),
      seq_lens, sel_idx, sel_cnt, softmax_scale * kLog2e, static_cast<E*>(out), lse, part_o,
      reinterpret_cast<float2*>(part_ml), p->d_error, Hkv, t_cap, p->max_sel, p->split,
      p->log2split, p->max_chunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p->max_chunks == 1) return e;
  k_combine<E, D, G><<<dim3((unsigned)p->units), NT, 0, stream>>>(
      p->d_units, seq_lens, sel_idx, sel_cnt, static_cast<E*>(out), lse, part_o,
      reinterpret_cast<const float2*>(part_ml), p->d_error, Hkv, t_cap, p->max_sel, p->split,
      p->log2split, p->max_chunks);
  return hipGetLastError();
}

template <typename E, int D>
hipError_t dispatch_g(const fx_plan* p, const void* q, const void* K, const void* V,
                      const int32_t* seq_lens, const int32_t* sel_idx, const int32_t* sel_cnt,
                      float scale, void* out, float* lse, float* po, float* pml,
                      hipStream_t s) {
  switch (p->G) {
    case 1: return launch_t<E, D, 1>(p, q, K, V, seq_lens, sel_idx, sel_cnt, scale, out, lse, po, pml, s);
    case 2: return launch_t<E, D, 2>(p, q, K, V, seq_lens, sel_idx, sel_cnt, scale, out, lse, po, pml, s);
    case 3: return launch_t<E, D, 3>(p, q, K, V, seq_lens, sel_idx, sel_cnt, scale, out, lse, po, pml, s);
    case 4: return launch_t<E, D, 4>(p, q, K, V, seq_lens, sel_idx, sel_cnt, scale, out, lse, po, pml, s);
    case 5: return launch_t<E, D, 5>(p, q, K, V, seq_lens, sel_idx, sel_cnt, scale, out, lse, po, pml, s);
    case 6: return launch_t<E, D, 6>(p, q, K, V, seq_lens, sel_idx, sel_cnt, scale, out, lse, po, pml, s);
    case 7: return launch_t<E, D, 7>(p, q, K, V, seq_lens, sel_idx, sel_cnt, scale, out, lse, po, pml, s);
    case 8: return launch_t<E, D, 8>(p, q, K, V, seq_lens, sel_idx, sel_cnt, scale, out, lse, po, pml, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const fx_plan* p, const void* q, const void* K, const void* V,
                         const int32_t* seq_lens, const int32_t* sel_idx, const int32_t* sel_cnt,
                         float softmax_scale, void* out, float* lse, float* part_o,
                         float* part_ml, hipStream_t stream) {
  const int d = p->desc.head_dim;
  if (p->desc.dtype == FX_BF16)
    return d == 128 ? dispatch_g<bf16_t, 128>(p, q, K, V, seq_lens, sel_idx, sel_cnt,
                                              softmax_scale, out, lse, part_o, part_ml, stream)
                    : dispatch_g<bf16_t, 64>(p, q, K, V, seq_lens, sel_idx, sel_cnt,
                                             softmax_scale, out, lse, part_o, part_ml, stream);
  return d == 128 ? dispatch_g<float, 128>(p, q, K, V, seq_lens, sel_idx, sel_cnt, softmax_scale,
                                           out, lse, part_o, part_ml, stream)
                  : dispatch_g<float, 64>(p, q, K, V, seq_lens, sel_idx, sel_cnt, softmax_scale,
                                          out, lse, part_o, part_ml, stream);
}

}  // namespace fx
