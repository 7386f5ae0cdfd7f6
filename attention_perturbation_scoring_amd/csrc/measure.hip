// Streaming-read reference kernel: the read bandwidth a plain, perfectly
// coalesced scan of one large buffer reaches on this device.  It is the
// "achievable" denominator next to the 8 TB/s data-sheet peak when the two
// score passes (each a single streaming read of K and V) are judged.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.h"

namespace dropkv {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;
constexpr int kReadBlocks = 2048;   // eight workgroups per CU on 256 CUs

// Each workgroup scans one contiguous slice of the buffer, eight 16-byte loads
// per thread in flight per step, non-temporal like the K/V streams of the
// score passes (on MI355X the faster form: ~6.9 against ~6.1 TB/s).  The XOR of everything it read is stored only
// if it equals a fixed constant, so the loads cannot be dropped while nothing
// is written in practice.
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4* __restrict__ p,
                                                                   int64_t units, uint32_t* sink) {
  const int64_t per = (units + kReadBlocks - 1) / kReadBlocks;
  const int64_t b0 = (int64_t)blockIdx.x * per;
  const int64_t b1 = b0 + per < units ? b0 + per : units;
  uint32_t acc = 0;
  constexpr int64_t kStep = (int64_t)kReadThreads * kReadUnroll;
  int64_t i = b0;
  for (; i + kStep <= b1; i += kStep) {
    u32x4 x[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const u32x4* a = p + i + (int64_t)u * kReadThreads + threadIdx.x;
      if constexpr (kNTStream) x[u] = __builtin_nontemporal_load(a);
      else x[u] = *a;
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
  }
  for (int64_t j = i + threadIdx.x; j < b1; j += kReadThreads) {
    const u32x4 x = p[j];
    acc ^= x.x ^ x.y ^ x.z ^ x.w;
  }
  if (acc == 0x9E3779B9u) sink[threadIdx.x & 7] = acc;
}

}  // namespace

hipError_t launch_stream_read(void* ctx, const void* p, int64_t bytes, uint32_t* sink,
                              hipStream_t s) {
  prof_begin(ctx, "stream_read", s);
  hipLaunchKernelGGL(stream_read_kernel, dim3(kReadBlocks), dim3(kReadThreads), 0, s,
                     static_cast<const u32x4*>(p), bytes / 16, sink);
  prof_end(ctx, "stream_read", s);
  return hipGetLastError();
}

}  // namespace dropkv
