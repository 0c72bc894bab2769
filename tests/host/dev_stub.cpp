// Stand-ins for the device side of libfx, so that the host code (fx_api.cpp) runs on a
// machine without a GPU: device memory is host memory, kernel launchers record their
// arguments instead of launching, and the decode grid is a settable number.
#include <cstdlib>
#include <cstring>
#include <new>

#include "dev_stub.h"

namespace stub {
int alloc_fails = 0;
int launch_fails = 0;
int decode_grid = 512;
bool scratch_missing = false;
Launch last;
int launches = 0;
static unsigned char scratch[fx::kStaticScratchBytes];

static int record(const char* name, const void* a = nullptr, const void* b = nullptr,
                  const void* c = nullptr) {
  last = Launch{name, a, b, c};
  ++launches;
  return launch_fails;
}
}  // namespace stub

namespace fx {

int dev_current(int* device) {
  *device = 0;
  return 0;
}
int dev_alloc(void** ptr, size_t bytes) {
  if (stub::alloc_fails) return 2;   // hipErrorOutOfMemory
  *ptr = std::malloc(bytes);
  return *ptr ? 0 : 2;
}
int dev_free(void* ptr) {
  std::free(ptr);
  return 0;
}
int dev_upload(void* dst, const void* src, size_t bytes) {
  std::memcpy(dst, src, bytes);
  return 0;
}
int dev_zero(void* dst, size_t bytes) {
  std::memset(dst, 0, bytes);
  return 0;
}
int dev_take_error(uint32_t* dev_word, uint32_t* host_word) {
  *host_word = *dev_word;
  *dev_word = 0;
  return 0;
}
void* dev_static_scratch(size_t* bytes) {
  *bytes = sizeof(stub::scratch);
  return stub::scratch_missing ? nullptr : stub::scratch;
}
int decode_grid(const fx_plan*, bool) { return stub::decode_grid; }

int launch_build_summaries(const fx_plan*, const void* K, const int32_t*, int32_t, int32_t,
                           void* S, hipStream_t) {
  return stub::record("build", K, S);
}
int launch_score(const fx_plan*, const void* q, const void* S, const int32_t*, float* scores,
                 hipStream_t) {
  return stub::record("score", q, S, scores);
}
int launch_topk(const fx_plan*, const float* scores, const float* logits, uint32_t*,
                const int32_t*, int32_t* sel_idx, int32_t*, uint32_t*, uint32_t*,
                const int32_t*, const int32_t*, int32_t*, int32_t*, int32_t*, int32_t*,
                hipStream_t) {
  return stub::record("topk", scores, logits, sel_idx);
}
int launch_select_fused(const fx_plan*, const void* q, const void* S, float* scores,
                        const float*, uint32_t*, const int32_t*, int32_t*, int32_t*,
                        const int32_t*, const int32_t*, int32_t*, int32_t*, int32_t*, int32_t*,
                        hipStream_t) {
  return stub::record("select_fused", q, S, scores);
}
int launch_decode(const fx_plan*, const void* q, const void*, const void*, const int32_t*,
                  const int32_t*, const int32_t*, const float* logits, float, void*, float*,
                  void* scratch, hipStream_t) {
  return stub::record("decode", q, logits, scratch);
}
int launch_stream_read(const void* src, size_t, uint32_t* sink, hipStream_t) {
  return stub::record("stream_read", src, sink);
}
int launch_compact(const fx_plan*, const void* K, const void*, const int32_t*, const int32_t*,
                   const int32_t*, int32_t* slot_map, void*, void*, int32_t*, void* moves,
                   int32_t*, hipStream_t) {
  return stub::record("compact", K, slot_map, moves);
}
int launch_delta(const fx_plan*, const int32_t* prev, const int32_t*, const int32_t* cur,
                 const int32_t*, int32_t* added, int32_t*, int32_t*, int32_t*, hipStream_t) {
  return stub::record("delta", prev, cur, added);
}

}  // namespace fx
