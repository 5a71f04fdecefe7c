// Device-side helpers shared by the HIP kernels of the round (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <cstdint>

#include "medusa.h"

namespace medusa {

using bf16 = __bf16;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }

// The sticky device status word: non-zero means an earlier step of the round
// failed and nothing more may be stored.  Earlier steps are earlier kernels of the stream
// (or the host before them), whose writes stream order makes visible to a plain load.  A
// system-scope atomic load would send every wavefront's read of this one word past the
// caches to memory, where they queue behind each other (several microseconds at the start
// of a kernel of a thousand workgroups).
__device__ __forceinline__ bool round_failed(const int32_t* status) { return *status != 0; }

// First error wins; later ones leave the code unchanged.
__device__ __forceinline__ void raise_status(int32_t* status, int32_t code) {
  atomicCAS(status, 0, code);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Launch one kernel whose single argument is a struct passed by value,
// optionally recording timing events from the dispatch itself.
template <typename Args>
inline medusa_status launch(const void* kernel, dim3 grid, dim3 block, size_t shmem,
                            hipStream_t stream, Args& args, void* ev_start, void* ev_stop) {
  void* kargs[] = {&args};
  // without timing events the plain launch (what stream capture records as a kernel node);
  // with them, the extended launch that records the events from the dispatch itself
  const hipError_t e =
      ev_start == nullptr && ev_stop == nullptr
          ? hipLaunchKernel(kernel, grid, block, kargs, shmem, stream)
          : hipExtLaunchKernel(kernel, grid, block, kargs, shmem, stream, static_cast<hipEvent_t>(ev_start),
                               static_cast<hipEvent_t>(ev_stop), 0);
  return e == hipSuccess ? MEDUSA_OK : MEDUSA_EHIP;
}

}  // namespace medusa
