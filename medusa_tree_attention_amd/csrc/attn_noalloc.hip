// medusa_tree_attn_noalloc: the tree attention of medusa_tree_attn with the split partials
// in a device array that the library holds, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that forbid it).
//
// The array is a file-scope __device__ variable: each GPU the library runs on holds its
// own copy until the process ends.  Its address on a device is taken once, on the first
// call made with that device current, with hipGetSymbolAddress; the host-side name of the
// array is only a stand-in and is never passed to a kernel.  Calls on one GPU share the
// array, so calls that overlap on one GPU (different streams) race; calls on one stream
// are ordered.  Nothing in it has to start at zero: every partial the merge reads is
// written by the same call first.

#include <mutex>

#include "attn_common.h"

namespace medusa {
namespace {

constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kAttnWorkspaceMax];

void* g_scratch[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

}  // namespace
}  // namespace medusa

using namespace medusa;

extern "C" medusa_status medusa_tree_attn_noalloc(void* stream, medusa_dtype dt, int32_t B, int32_t Hq,
                                                  int32_t Hkv, int32_t d_h, int32_t N,
                                                  const int32_t* d_depth, const uint64_t* d_tree_mask,
                                                  int32_t mask_words, const int32_t* d_prefix_len,
                                                  const void* q, const void* k_new, const void* v_new,
                                                  void* k_cache, void* v_cache, int32_t S_max,
                                                  double rope_base, void* out, int32_t* d_status,
                                                  void* ev_start, void* ev_stop) {
  const size_t need = medusa_tree_attn_workspace_size(dt, B, Hq, Hkv, d_h, N, S_max);
  if (need > kAttnWorkspaceMax) return MEDUSA_ECAPACITY;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MEDUSA_EHIP;
  std::call_once(g_scratch_once[dev], [dev] {
    g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch[dev], HIP_SYMBOL(scratch));
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch[dev] == nullptr) return MEDUSA_EHIP;
  return medusa_tree_attn(stream, dt, B, Hq, Hkv, d_h, N, d_depth, d_tree_mask, mask_words, d_prefix_len, q,
                          k_new, v_new, k_cache, v_cache, S_max, rope_base, out, g_scratch[dev],
                          kAttnWorkspaceMax, d_status, ev_start, ev_stop);
}
