// Streaming-read calibration (a measurement utility, not a step of the round): reads a
// device buffer once the way a well-formed memory-bound kernel does -- many workgroups,
// every thread with eight 16-byte loads in flight -- and stores one word per workgroup so
// that the loads are kept.  Its bandwidth on a buffer larger than the Infinity Cache is the
// practical read ceiling the round's kernels are compared with, measured on the same chip
// in the same run.

#include "common.h"

namespace medusa {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;
constexpr int kProbeBlocks = 4096;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* __restrict__ p, int64_t n16,
                                                                    uint32_t* sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const int64_t stride = int64_t(gridDim.x) * kProbeThreads * kProbeUnroll;
  for (int64_t base = int64_t(blockIdx.x) * kProbeThreads * kProbeUnroll + threadIdx.x; base < n16;
       base += stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {  // all loads first; past the end re-read the last piece
      const int64_t i = base + int64_t(u) * kProbeThreads;
      v[u] = __builtin_nontemporal_load(p + (i < n16 ? i : n16 - 1));
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
  }
  const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  const uint32_t y = __reduce_or_sync(~0ull, x);  // one word per workgroup: wave 0's lanes
  if (threadIdx.x == 0) sink[blockIdx.x] = y;
}

}  // namespace
}  // namespace medusa

using namespace medusa;

extern "C" size_t medusa_read_probe_sink_size(void) { return size_t(kProbeBlocks) * sizeof(uint32_t); }

extern "C" medusa_status medusa_read_probe(void* stream, const void* src, size_t bytes, uint32_t* sink,
                                           void* ev_start, void* ev_stop) {
  if (!src || !sink || bytes < 16 || bytes % 16 != 0) return MEDUSA_EINVAL;
  if ((reinterpret_cast<uintptr_t>(src) & 15) != 0) return MEDUSA_EINVAL;
  const int64_t n16 = int64_t(bytes / 16);
  const int64_t per_block = int64_t(kProbeThreads) * kProbeUnroll;
  const int64_t blocks = (n16 + per_block - 1) / per_block < kProbeBlocks ? (n16 + per_block - 1) / per_block
                                                                          : kProbeBlocks;
  const u32x4* p = static_cast<const u32x4*>(src);
  void* kargs[] = {&p, const_cast<int64_t*>(&n16), &sink};
  const hipError_t e =
      ev_start == nullptr && ev_stop == nullptr
          ? hipLaunchKernel(reinterpret_cast<const void*>(&read_probe_kernel), dim3(unsigned(blocks)),
                            dim3(kProbeThreads), kargs, 0, static_cast<hipStream_t>(stream))
          : hipExtLaunchKernel(reinterpret_cast<const void*>(&read_probe_kernel), dim3(unsigned(blocks)),
                               dim3(kProbeThreads), kargs, 0, static_cast<hipStream_t>(stream),
                               static_cast<hipEvent_t>(ev_start), static_cast<hipEvent_t>(ev_stop), 0);
  return e == hipSuccess ? MEDUSA_OK : MEDUSA_EHIP;
}
