// Attainable-bandwidth reference: a plain streaming read (measurement utility; not part
// of the decode path).
//
// Each workgroup reads one contiguous span of the buffer with 16-byte nontemporal buffer
// loads, four per thread in flight, and writes the XOR of what it read to one sink word
// so the loads cannot be removed.  Spans past the end of the buffer read as zero without
// a memory access (buffer resource bound), so the grid needs no tail handling.
#include "fx_device.h"

namespace fx {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;

__global__ __launch_bounds__(kProbeThreads) void k_stream_read(const uint8_t* __restrict__ src,
                                                               uint64_t bytes, uint64_t span,
                                                               uint32_t* __restrict__ sink) {
  const uint64_t begin = (uint64_t)blockIdx.x * span;
  const uint64_t len = begin < bytes ? min(span, bytes - begin) : 0;
  // One resource per workgroup span (spans are below 2^31 bytes).
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)(src + begin), 0, (int)len, kRsrcWord3);
  uint32_t acc = 0;
  for (uint32_t off = threadIdx.x * 16u; off < (uint32_t)span;
       off += kProbeThreads * 16u * kProbeUnroll) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int k = 0; k < kProbeUnroll; ++k) v[k] = buffer_load16(r, off + k * kProbeThreads * 16u);
#pragma unroll
    for (int k = 0; k < kProbeUnroll; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  __shared__ uint32_t red[kProbeThreads / 64];
  for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < kProbeThreads / 64; ++i) x ^= red[i];
    sink[blockIdx.x] = x;
  }
}

}  // namespace

int launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  const uint64_t span = kStreamReadSpan;
  const uint64_t grid = (bytes + span - 1) / span;
  if (grid == 0) return hipSuccess;
  k_stream_read<<<dim3((unsigned)grid), kProbeThreads, 0, stream>>>(
      static_cast<const uint8_t*>(src), bytes, span, sink);
  return hipGetLastError();
}

}  // namespace fx
