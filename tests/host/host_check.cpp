// The host path of libfx (plan creation, validation, layouts, entry points) on the CPU,
// with the device stand-ins of dev_stub.cpp.  Built with the address and
// undefined-behaviour sanitizers by tests/test_host_sanitized.py; every fx_status code is
// forced at least once.  Prints one line per failed check and exits nonzero if any failed.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <vector>

#include "dev_stub.h"
#include "fx.h"
#include "fx_plan.h"

static int failures = 0;
static int checks = 0;
#define CHECK(cond)                                                        \
  do {                                                                     \
    ++checks;                                                              \
    if (!(cond)) {                                                         \
      ++failures;                                                          \
      std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);          \
    }                                                                      \
  } while (0)

static fx_plan_desc desc(int B, int Hq, int Hkv, int d, int t_cap, int dtype) {
  fx_plan_desc x;
  x.batch = B;
  x.num_q_heads = Hq;
  x.num_kv_heads = Hkv;
  x.head_dim = d;
  x.t_cap = t_cap;
  x.dtype = dtype;
  x.split_tokens = 0;
  x.pooling = FX_POOL_KEY;
  return x;
}

static fx_head_policy retrieval(int block, int top_k) {
  fx_head_policy p;
  std::memset(&p, 0, sizeof p);
  p.mode = FX_RETRIEVAL;
  p.block = block;
  p.sub_block = block < 16 ? block : 16;
  p.top_k = top_k;
  p.force_sink = 1;
  p.force_last = 1;
  return p;
}
static fx_head_policy streaming(int block) {
  fx_head_policy p = retrieval(block, 0);
  p.mode = FX_STREAMING;
  p.sink_tokens = 64;
  p.local_tokens = 1024;
  p.force_sink = p.force_last = 0;
  return p;
}
static fx_head_policy nosa(int block, int kq, int ke) {
  fx_head_policy p = retrieval(block, kq);
  p.mode = FX_NOSA;
  p.k_evict = ke;
  p.force_sink = p.force_last = 0;
  return p;
}

static size_t up256(size_t x) { return (x + 255) / 256 * 256; }

// Host buffers standing in for device buffers (16-byte aligned at offset 0).
struct Buf {
  std::vector<uint64_t> v;
  explicit Buf(size_t bytes) : v(bytes / 8 + 4, 0) {}
  void* p(size_t off = 0) { return reinterpret_cast<char*>(v.data()) + off; }
  template <class T>
  T* as(size_t off = 0) { return reinterpret_cast<T*>(p(off)); }
};

static void test_descriptions() {
  fx_head_policy pol[8];
  for (auto& p : pol) p = retrieval(64, 8);
  fx_plan_t plan = nullptr;
  fx_plan_desc d = desc(1, 4, 2, 128, 4096, FX_BF16);
  CHECK(fx_plan_create(nullptr, pol, &plan) == FX_E_INVALID);
  CHECK(fx_plan_create(&d, nullptr, &plan) == FX_E_INVALID);
  CHECK(fx_plan_create(&d, pol, nullptr) == FX_E_INVALID);
  const fx_plan_desc bad[] = {
      desc(0, 4, 2, 128, 4096, FX_BF16),  desc(1, 4, 0, 128, 4096, FX_BF16),
      desc(1, 6, 4, 128, 4096, FX_BF16),  desc(1, 18, 2, 128, 4096, FX_BF16),
      desc(1, 4, 2, 96, 4096, FX_BF16),   desc(1, 4, 2, 128, 0, FX_BF16),
      desc(1, 4, 2, 128, (1 << 24) + 1, FX_BF16), desc(1, 4, 2, 128, 4096, 7)};
  for (const auto& b : bad) CHECK(fx_plan_create(&b, pol, &plan) == FX_E_INVALID);
  fx_plan_desc s = d;
  s.split_tokens = 100;
  CHECK(fx_plan_create(&s, pol, &plan) == FX_E_INVALID);
  s.split_tokens = 4096;
  CHECK(fx_plan_create(&s, pol, &plan) == FX_E_INVALID);
  s = d;
  s.pooling = 3;
  CHECK(fx_plan_create(&s, pol, &plan) == FX_E_INVALID);
  // One unit's K rows need 32-bit byte offsets: t_cap * d * 4 >= 2^31 is unsupported.
  fx_plan_desc big = desc(1, 4, 2, 128, 1 << 22, FX_F32);
  CHECK(fx_plan_create(&big, pol, &plan) == FX_E_UNSUPPORTED);
  // Score-side pooling keeps block / sub_block rows per block, at most 64.
  fx_head_policy wide[2] = {retrieval(256, 8), retrieval(256, 8)};
  wide[0].sub_block = wide[1].sub_block = 2;
  s = d;
  s.pooling = FX_POOL_SCORE_SUM;
  CHECK(fx_plan_create(&s, wide, &plan) == FX_E_UNSUPPORTED);
  CHECK(plan == nullptr);
}

static void test_policies() {
  fx_plan_desc d = desc(1, 4, 2, 128, 4096, FX_BF16);
  fx_plan_t plan = nullptr;
  auto bad = [&](fx_head_policy p) {
    fx_head_policy two[2] = {retrieval(64, 8), p};
    return fx_plan_create(&d, two, &plan);
  };
  fx_head_policy p = retrieval(64, 8);
  p.mode = 5;
  CHECK(bad(p) == FX_E_INVALID);
  p = retrieval(48, 8);
  CHECK(bad(p) == FX_E_INVALID);
  p = retrieval(512, 8);
  CHECK(bad(p) == FX_E_INVALID);
  p = retrieval(64, 8);
  p.sub_block = 3;
  CHECK(bad(p) == FX_E_INVALID);
  p = retrieval(64, 8);
  p.force_sink = 2;
  CHECK(bad(p) == FX_E_INVALID);
  p = retrieval(64, 0);
  p.budget = 0.0f;
  CHECK(bad(p) == FX_E_INVALID);
  p.budget = 1.5f;
  CHECK(bad(p) == FX_E_INVALID);
  p.budget = std::numeric_limits<float>::quiet_NaN();
  CHECK(bad(p) == FX_E_INVALID);
  p = streaming(64);
  p.local_tokens = -1;
  CHECK(bad(p) == FX_E_INVALID);
  p = nosa(64, 0, 0);
  CHECK(bad(p) == FX_E_INVALID);
  p = nosa(64, 4, -1);
  CHECK(bad(p) == FX_E_INVALID);
}

static void test_layout_and_sizes() {
  // Two sequences, four kv heads of different block sizes and modes, t_cap 1000.
  fx_plan_desc d = desc(2, 8, 4, 64, 1000, FX_BF16);
  fx_head_policy pol[8] = {retrieval(16, 8), streaming(32), nosa(64, 4, 12), retrieval(128, 0),
                           retrieval(16, 8), streaming(32), nosa(64, 4, 12), retrieval(128, 0)};
  pol[3].budget = 0.05f;
  pol[7].budget = 0.05f;
  fx_plan_t plan = nullptr;
  CHECK(fx_plan_create(&d, pol, &plan) == FX_OK);
  if (!plan) return;
  // n_cap = ceil(1000 / g): 63, 32, 16, 8 per sequence.
  const int64_t ncap[4] = {63, 32, 16, 8};
  int64_t off = 0, words = 0;
  for (int u = 0; u < 8; ++u) {
    CHECK(fx_unit_block_offset(plan, u) == off);
    CHECK(fx_unit_summary_offset(plan, u) == off);
    off += ncap[u % 4];
    words += (ncap[u % 4] + 31) / 32;
  }
  CHECK(fx_unit_block_offset(plan, 8) == -1 && fx_unit_block_offset(plan, -1) == -1);
  CHECK(fx_logits_bytes(plan) == (size_t)off * 4);
  CHECK(fx_summary_bytes(plan) == (size_t)off * 64 * 2);
  CHECK(fx_evict_mask_bytes(plan) == (size_t)words * 4);
  // Selection bounds: retrieval top-k 8 + 2; streaming ceil(64/32) + ceil(1024/32) + 2 = 36
  // clamped to n_cap 32; NOSA 4 + 12 + 2; budget ceil(0.05 * 8) + 2 = 3.
  CHECK(fx_unit_max_selected(plan, 0) == 10);
  CHECK(fx_unit_max_selected(plan, 1) == 32);
  CHECK(fx_unit_max_selected(plan, 2) == 16);
  CHECK(fx_unit_max_selected(plan, 3) == 3);
  CHECK(fx_max_selected(plan) == 32);
  CHECK(fx_split_tokens(plan) == 256);
  // Compaction slots: max_sel * g rows per unit.
  const int64_t wrows = 10 * 16 + 32 * 32 + 16 * 64 + 3 * 128;
  CHECK(fx_unit_work_offset(plan, 1) == 10 * 16);
  CHECK(fx_work_bytes(plan) == (size_t)(2 * wrows) * 64 * 2);
  // Workspace: scores | (no top-k keys / bits: registers) | decode partials | moves.
  const size_t G = 2, grid = (size_t)stub::decode_grid;
  const size_t expect = up256(off * 4) + up256(grid * 2 * G * 64 * 4) + up256(grid * 2 * G * 8) +
                        up256(grid * 8) + up256(8 * 32 * 8) + up256(8 * 4);
  CHECK(fx_workspace_bytes(plan) == expect);
  CHECK(fx_noalloc_scratch_bytes(plan) ==
        up256(grid * 2 * G * 64 * 4) + up256(grid * 2 * G * 8) + up256(grid * 8));
  CHECK(fx_plan_destroy(plan) == FX_OK);
  CHECK(fx_plan_destroy(nullptr) == FX_OK);
  CHECK(fx_summary_bytes(nullptr) == 0 && fx_max_selected(nullptr) == -1);
  CHECK(fx_noalloc_scratch_bytes(nullptr) == 0);
}

static void test_create_failures() {
  fx_plan_desc d = desc(1, 4, 2, 128, 4096, FX_BF16);
  fx_head_policy pol[2] = {retrieval(64, 8), retrieval(64, 8)};
  fx_plan_t plan = nullptr;
  stub::alloc_fails = 1;
  CHECK(fx_plan_create(&d, pol, &plan) == FX_E_HIP);
  stub::alloc_fails = 0;
  stub::decode_grid = 0;   // the occupancy query failed
  CHECK(fx_plan_create(&d, pol, &plan) == FX_E_HIP);
  stub::decode_grid = 512;
  CHECK(plan == nullptr);
  // Selected tokens of all units laid end to end must index with int32.
  fx_plan_desc many = desc(1024, 8, 8, 64, 1 << 21, FX_BF16);
  std::vector<fx_head_policy> all(8192, retrieval(256, 8192));
  CHECK(fx_plan_create(&many, all.data(), &plan) == FX_E_UNSUPPORTED);
}

static void test_select() {
  fx_plan_desc d = desc(2, 8, 2, 128, 4096, FX_BF16);
  fx_head_policy pol[4] = {retrieval(64, 8), nosa(64, 4, 12), streaming(64), nosa(64, 4, 12)};
  fx_plan_t plan = nullptr;
  CHECK(fx_plan_create(&d, pol, &plan) == FX_OK);
  if (!plan) return;
  const size_t ws_bytes = fx_workspace_bytes(plan);
  Buf q(4096), S(fx_summary_bytes(plan)), lg(fx_logits_bytes(plan) + 16),
      mk(fx_evict_mask_bytes(plan) + 16), lens(64), sel(4096), cnt(64), ws(ws_bytes + 64),
      prev(4096), pcnt(64), add(4096), acnt(64), rem(4096), rcnt(64);
  auto sel_call = [&](const void* qq, const void* ss, const float* l, uint32_t* m, void* w,
                      size_t wb) {
    return fx_select(plan, qq, ss, l, m, lens.as<int32_t>(), sel.as<int32_t>(),
                     cnt.as<int32_t>(), w, wb, nullptr);
  };
  CHECK(sel_call(q.p(), S.p(), lg.as<float>(), mk.as<uint32_t>(), ws.p(), ws_bytes) == FX_OK);
  // 256 block slots per unit: the selection forms its own scores.
  CHECK(std::strcmp(stub::last.name, "select_fused") == 0 && stub::last.a == q.p());
  CHECK(sel_call(nullptr, S.p(), lg.as<float>(), mk.as<uint32_t>(), ws.p(), ws_bytes) ==
        FX_E_INVALID);
  CHECK(sel_call(q.p(8), S.p(), lg.as<float>(), mk.as<uint32_t>(), ws.p(), ws_bytes) ==
        FX_E_INVALID);   // q not 16-byte aligned
  CHECK(sel_call(q.p(), nullptr, lg.as<float>(), mk.as<uint32_t>(), ws.p(), ws_bytes) ==
        FX_E_INVALID);   // scored units need summaries
  CHECK(sel_call(q.p(), S.p(), nullptr, mk.as<uint32_t>(), ws.p(), ws_bytes) ==
        FX_E_INVALID);   // NOSA with k_evict > 0 needs logits
  CHECK(sel_call(q.p(), S.p(), lg.as<float>(), nullptr, ws.p(), ws_bytes) ==
        FX_E_INVALID);   // ... and the eviction mask
  CHECK(sel_call(q.p(), S.p(), lg.as<float>(2), mk.as<uint32_t>(), ws.p(), ws_bytes) ==
        FX_E_INVALID);   // logits not 4-byte aligned
  CHECK(sel_call(q.p(), S.p(), lg.as<float>(), mk.as<uint32_t>(), ws.p(), ws_bytes - 1) ==
        FX_E_WORKSPACE);
  CHECK(sel_call(q.p(), S.p(), lg.as<float>(), mk.as<uint32_t>(), ws.p(4), ws_bytes) ==
        FX_E_INVALID);   // workspace not 16-byte aligned
  CHECK(fx_select(nullptr, q.p(), S.p(), nullptr, nullptr, lens.as<int32_t>(), sel.as<int32_t>(),
                  cnt.as<int32_t>(), ws.p(), ws_bytes, nullptr) == FX_E_INVALID);
  stub::launch_fails = 98;   // hipErrorInvalidValue
  CHECK(sel_call(q.p(), S.p(), lg.as<float>(), mk.as<uint32_t>(), ws.p(), ws_bytes) == FX_E_HIP);
  stub::launch_fails = 0;
  // fx_select_delta: the previous selection must not alias the new one.
  auto sd = [&](int32_t* pi, int32_t* pc) {
    return fx_select_delta(plan, q.p(), S.p(), lg.as<float>(), mk.as<uint32_t>(),
                           lens.as<int32_t>(), pi, pc, sel.as<int32_t>(), cnt.as<int32_t>(),
                           add.as<int32_t>(), acnt.as<int32_t>(), rem.as<int32_t>(),
                           rcnt.as<int32_t>(), ws.p(), ws_bytes, nullptr);
  };
  CHECK(sd(prev.as<int32_t>(), pcnt.as<int32_t>()) == FX_OK);
  CHECK(sd(sel.as<int32_t>(), pcnt.as<int32_t>()) == FX_E_INVALID);
  CHECK(sd(prev.as<int32_t>(), cnt.as<int32_t>()) == FX_E_INVALID);
  CHECK(sd(nullptr, pcnt.as<int32_t>()) == FX_E_INVALID);
  fx_plan_destroy(plan);

  // A plan of streaming units only: no summaries, logits or mask needed.
  fx_head_policy st[4] = {streaming(64), streaming(64), streaming(64), streaming(64)};
  CHECK(fx_plan_create(&d, st, &plan) == FX_OK);
  if (!plan) return;
  CHECK(sel_call(q.p(), nullptr, nullptr, nullptr, ws.p(), fx_workspace_bytes(plan)) == FX_OK);
  CHECK(std::strcmp(stub::last.name, "topk") == 0);
  fx_plan_destroy(plan);

  // Large units: separate scoring kernel, then the top-k kernel reading the scores at the
  // start of the workspace; more than 8192 slots: keys and bitmaps in the workspace.
  fx_plan_desc dl = desc(1, 4, 2, 128, 1 << 18, FX_BF16);
  fx_head_policy big[2] = {retrieval(16, 64), retrieval(16, 64)};
  CHECK(fx_plan_create(&dl, big, &plan) == FX_OK);
  if (!plan) return;
  Buf S2(fx_summary_bytes(plan)), ws2(fx_workspace_bytes(plan) + 64);
  CHECK(fx_select(plan, q.p(), S2.p(), nullptr, nullptr, lens.as<int32_t>(), sel.as<int32_t>(),
                  cnt.as<int32_t>(), ws2.p(), fx_workspace_bytes(plan), nullptr) == FX_OK);
  CHECK(std::strcmp(stub::last.name, "topk") == 0 && stub::last.a == ws2.p());
  // 2 x 16384 slots of float scores and 32-bit keys, 3 bitmaps of 2 x 512 words.
  const size_t grid = (size_t)stub::decode_grid;
  CHECK(fx_workspace_bytes(plan) == up256(32768 * 4) + up256(32768 * 4) + up256(3 * 1024 * 4) +
                                        up256(grid * 2 * 2 * 128 * 4) + up256(grid * 2 * 2 * 8) +
                                        up256(grid * 8) + up256(2 * 66 * 8) + up256(2 * 4));
  fx_plan_destroy(plan);
}

static void test_decode() {
  fx_plan_desc d = desc(1, 8, 2, 64, 2048, FX_F32);
  fx_head_policy pol[2] = {retrieval(32, 8), nosa(32, 4, 4)};
  fx_plan_t plan = nullptr;
  CHECK(fx_plan_create(&d, pol, &plan) == FX_OK);
  if (!plan) return;
  const size_t ws_bytes = fx_workspace_bytes(plan);
  Buf q(4096), K(2 * 2048 * 64 * 4), V(2 * 2048 * 64 * 4), lens(16), sel(4096), cnt(16),
      out(4096), lse(64), ws(ws_bytes + 64), lg(fx_logits_bytes(plan) + 16);
  auto dec = [&](float scale, void* o, float* l, void* w, size_t wb) {
    return fx_sparse_decode(plan, q.p(), K.p(), V.p(), lens.as<int32_t>(), sel.as<int32_t>(),
                            cnt.as<int32_t>(), scale, o, l, w, wb, nullptr);
  };
  CHECK(dec(0.125f, out.p(), lse.as<float>(), ws.p(), ws_bytes) == FX_OK);
  CHECK(std::strcmp(stub::last.name, "decode") == 0 && stub::last.b == nullptr);
  // The partials follow the scores in the workspace.
  CHECK(stub::last.c == ws.as<char>() + up256(fx_logits_bytes(plan)));
  CHECK(dec(0.125f, out.p(), nullptr, ws.p(), ws_bytes) == FX_OK);   // lse is optional
  CHECK(dec(0.0f, out.p(), lse.as<float>(), ws.p(), ws_bytes) == FX_E_INVALID);
  CHECK(dec(-1.0f, out.p(), lse.as<float>(), ws.p(), ws_bytes) == FX_E_INVALID);
  CHECK(dec(std::numeric_limits<float>::infinity(), out.p(), lse.as<float>(), ws.p(), ws_bytes) ==
        FX_E_INVALID);
  CHECK(dec(std::numeric_limits<float>::quiet_NaN(), out.p(), lse.as<float>(), ws.p(),
            ws_bytes) == FX_E_INVALID);
  CHECK(dec(0.125f, out.p(8), lse.as<float>(), ws.p(), ws_bytes) == FX_E_INVALID);
  CHECK(dec(0.125f, out.p(), lse.as<float>(1) , ws.p(), ws_bytes) == FX_E_INVALID);
  CHECK(dec(0.125f, out.p(), lse.as<float>(), ws.p(), ws_bytes - 256) == FX_E_WORKSPACE);
  CHECK(dec(0.125f, out.p(), lse.as<float>(), nullptr, ws_bytes) == FX_E_INVALID);
  CHECK(fx_sparse_decode(plan, q.p(), K.p(4), V.p(), lens.as<int32_t>(), sel.as<int32_t>(),
                         cnt.as<int32_t>(), 0.125f, out.p(), nullptr, ws.p(), ws_bytes,
                         nullptr) == FX_E_INVALID);   // K not 16-byte aligned
  stub::launch_fails = 98;
  CHECK(dec(0.125f, out.p(), lse.as<float>(), ws.p(), ws_bytes) == FX_E_HIP);
  stub::launch_fails = 0;

  // The eviction-logit decode: a plan with a NOSA unit needs the logits.
  auto ed = [&](const float* l) {
    return fx_sparse_decode_ed(plan, q.p(), K.p(), V.p(), lens.as<int32_t>(), sel.as<int32_t>(),
                               cnt.as<int32_t>(), l, 0.125f, out.p(), nullptr, ws.p(), ws_bytes,
                               nullptr);
  };
  CHECK(ed(nullptr) == FX_E_INVALID);
  CHECK(ed(lg.as<float>()) == FX_OK && stub::last.b == lg.p());

  // The no-allocation decode: partials in the static array, never in a workspace.
  auto na = [&](void* o) {
    return fx_sparse_decode_noalloc(plan, q.p(), K.p(), V.p(), lens.as<int32_t>(),
                                    sel.as<int32_t>(), cnt.as<int32_t>(), 0.125f, o, nullptr,
                                    nullptr);
  };
  size_t sb = 0;
  void* static_array = fx::dev_static_scratch(&sb);
  CHECK(na(out.p()) == FX_OK && stub::last.c == static_array);
  CHECK(na(out.p(4)) == FX_E_INVALID);
  fx_plan_destroy(plan);
  // Partials larger than the array: refused with FX_E_WORKSPACE.
  stub::decode_grid = 40000;
  CHECK(fx_plan_create(&d, pol, &plan) == FX_OK);
  if (plan) {
    CHECK(fx_noalloc_scratch_bytes(plan) > fx::kStaticScratchBytes);
    CHECK(na(out.p()) == FX_E_WORKSPACE);
    fx_plan_destroy(plan);
  }
  stub::decode_grid = 512;
  // No array address found on the device: FX_E_HIP.
  stub::scratch_missing = true;
  CHECK(fx_plan_create(&d, pol, &plan) == FX_OK);
  if (plan) {
    CHECK(na(out.p()) == FX_E_HIP);
    fx_plan_destroy(plan);
  }
  stub::scratch_missing = false;
}

static void test_other_calls() {
  fx_plan_desc d = desc(1, 4, 2, 128, 8192, FX_BF16);
  fx_head_policy pol[2] = {retrieval(64, 8), retrieval(64, 8)};
  fx_plan_t plan = nullptr;
  CHECK(fx_plan_create(&d, pol, &plan) == FX_OK);
  if (!plan) return;
  const size_t ws_bytes = fx_workspace_bytes(plan);
  Buf K(2 * 8192 * 256), V(2 * 8192 * 256), lens(16), S(fx_summary_bytes(plan)), sel(4096),
      cnt(16), slots(4096), wk(fx_work_bytes(plan)), wv(fx_work_bytes(plan)), moved(16),
      ws(ws_bytes + 64), a(4096), b(4096), c(4096), e(4096), f(4096), g(4096), h(4096), i(4096);
  CHECK(fx_build_summaries(plan, K.p(), lens.as<int32_t>(), 0, 1 << 30, S.p(), nullptr) == FX_OK);
  CHECK(fx_build_summaries(plan, K.p(2), lens.as<int32_t>(), 0, 1, S.p(), nullptr) ==
        FX_E_INVALID);
  CHECK(fx_build_summaries(plan, K.p(), lens.as<int32_t>(1), 0, 1, S.p(), nullptr) ==
        FX_E_INVALID);
  auto cu = [&](int32_t* sm, size_t wb) {
    return fx_compact_update(plan, K.p(), V.p(), lens.as<int32_t>(), sel.as<int32_t>(),
                             cnt.as<int32_t>(), sm, wk.p(), wv.p(), moved.as<int32_t>(), ws.p(),
                             wb, nullptr);
  };
  CHECK(cu(slots.as<int32_t>(), ws_bytes) == FX_OK);
  CHECK(std::strcmp(stub::last.name, "compact") == 0);
  CHECK(cu(nullptr, ws_bytes) == FX_E_INVALID);
  CHECK(cu(slots.as<int32_t>(), ws_bytes - 1) == FX_E_WORKSPACE);
  auto dl = [&](int32_t* prev) {
    return fx_selection_delta(plan, prev, b.as<int32_t>(), c.as<int32_t>(), e.as<int32_t>(),
                              f.as<int32_t>(), g.as<int32_t>(), h.as<int32_t>(), i.as<int32_t>(),
                              nullptr);
  };
  CHECK(dl(a.as<int32_t>()) == FX_OK && std::strcmp(stub::last.name, "delta") == 0);
  CHECK(dl(nullptr) == FX_E_INVALID);
  CHECK(dl(a.as<int32_t>(2)) == FX_E_INVALID);
  uint32_t word = 7;
  CHECK(fx_read_error(plan, &word) == FX_OK && word == 0);
  CHECK(fx_read_error(plan, nullptr) == FX_E_INVALID);
  CHECK(fx_read_error(nullptr, &word) == FX_E_INVALID);
  fx_plan_destroy(plan);

  // A selection bound above the compaction slot limit.
  fx_head_policy wide[2] = {retrieval(1, 3000), retrieval(1, 3000)};
  fx_plan_desc dw = desc(1, 4, 2, 64, 4096, FX_BF16);
  CHECK(fx_plan_create(&dw, wide, &plan) == FX_OK);
  if (plan) {
    Buf ws3(fx_workspace_bytes(plan) + 64), wk3(fx_work_bytes(plan)), wv3(fx_work_bytes(plan));
    CHECK(fx_compact_update(plan, K.p(), V.p(), lens.as<int32_t>(), sel.as<int32_t>(),
                            cnt.as<int32_t>(), slots.as<int32_t>(), wk3.p(), wv3.p(), nullptr,
                            ws3.p(), fx_workspace_bytes(plan), nullptr) == FX_E_UNSUPPORTED);
    fx_plan_destroy(plan);
  }

  Buf src(4096), sink(64);
  CHECK(fx_stream_read(src.p(), 4096, sink.as<uint32_t>(), nullptr) == FX_OK);
  CHECK(fx_stream_read(src.p(), 4000 + 8, sink.as<uint32_t>(), nullptr) == FX_E_INVALID);
  CHECK(fx_stream_read(src.p(), 0, sink.as<uint32_t>(), nullptr) == FX_E_INVALID);
  CHECK(fx_stream_read_sink_words((3u << 20) + 1) == 4);

  // Every status has its own string.
  for (int st = FX_OK; st <= FX_E_HIP; ++st) CHECK(std::strncmp(fx_status_string(st), "FX_", 3) == 0);
  CHECK(std::strstr(fx_status_string(42), "unknown") != nullptr);
}

// The automatic split keeps every unit whole (and the decode launches no merge kernel)
// only when the decode cuts units into their own pieces (at most half grid / 8 units on
// a grid of at least 128 workgroups) and no unit can hold more than 512 token slots.
static void test_uncut_plans() {
  fx_plan_t plan = nullptr;
  // Two units of at most 10 blocks of 32 tokens: 320 slots.
  fx_plan_desc d = desc(1, 4, 2, 64, 2048, FX_F32);
  fx_head_policy small[2] = {retrieval(32, 8), retrieval(32, 8)};
  CHECK(fx_plan_create(&d, small, &plan) == FX_OK);
  CHECK(plan->decode_uncut && plan->decode_split == 320);
  CHECK(fx_split_tokens(plan) == 256);
  CHECK(fx_plan_destroy(plan) == FX_OK);
  // An explicit split is kept as given.
  d.split_tokens = 128;
  CHECK(fx_plan_create(&d, small, &plan) == FX_OK);
  CHECK(!plan->decode_uncut && plan->decode_split == 128);
  CHECK(fx_plan_destroy(plan) == FX_OK);
  d.split_tokens = 0;
  // Units of up to 28 blocks of 64 tokens (1792 slots) are cut into pieces.
  fx_plan_desc d8 = desc(1, 32, 8, 128, 32768, FX_BF16);
  std::vector<fx_head_policy> big(8, retrieval(64, 26));
  CHECK(fx_plan_create(&d8, big.data(), &plan) == FX_OK);
  CHECK(!plan->decode_uncut && plan->decode_split == 256);
  CHECK(fx_plan_destroy(plan) == FX_OK);
  // 40 small units on a 512-workgroup grid: more than 256 / 8, so stream-K, which may cut.
  fx_plan_desc d40 = desc(20, 4, 2, 64, 2048, FX_F32);
  std::vector<fx_head_policy> many(40, retrieval(32, 8));
  CHECK(fx_plan_create(&d40, many.data(), &plan) == FX_OK);
  CHECK(!plan->decode_uncut);
  CHECK(fx_plan_destroy(plan) == FX_OK);
  // A grid below 128 workgroups has no half grid and no unit-aligned pieces.
  stub::decode_grid = 100;
  CHECK(fx_plan_create(&d, small, &plan) == FX_OK);
  CHECK(!plan->decode_uncut && plan->decode_split == 256);
  CHECK(fx_plan_destroy(plan) == FX_OK);
  stub::decode_grid = 512;
}

int main() {
  test_descriptions();
  test_policies();
  test_layout_and_sizes();
  test_create_failures();
  test_uncut_plans();
  test_select();
  test_decode();
  test_other_calls();
  std::printf("%d checks, %d failed\n", checks, failures);
  return failures == 0 ? 0 : 1;
}
