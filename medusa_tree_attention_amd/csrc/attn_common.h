// Arguments and checks shared by the tree-attention device paths.
#pragma once

#include <cstdint>

#include "common.h"

namespace medusa {

struct AttnArgs {
  const int32_t* depth;        // [N]
  const uint64_t* mask;        // [N][mask_words]
  const int32_t* prefix_len;   // [B]
  const void* q;               // [B][N][Hq][D]
  const void* k_new;           // [B][N][Hkv][D]
  const void* v_new;           // [B][N][Hkv][D]
  void* k_cache;               // [B][Hkv][S_max][D]
  void* v_cache;               // [B][Hkv][S_max][D]
  void* out;                   // [B][N][Hq][D]
  int32_t* status;
  void* workspace;
  double rope_base;
  int32_t B, Hq, Hkv, N, mask_words, S_max;
};

// Every sequence's staged rows [P_b, P_b + N) must lie inside the cache.  All
// blocks evaluate the same condition, so they all store or none does.  Each lane
// checks one sequence per pass (a vector load, not a chain of scalar ones) and the
// wavefront votes; the result is wave-uniform.
__device__ __forceinline__ bool prefixes_fit(const AttnArgs& a) {
  const int lane = threadIdx.x & 63;
  bool bad = false;
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const int b = b0 + lane;
    if (b < a.B) {
      const int64_t P = a.prefix_len[b];
      bad |= (P < 0) | (P + a.N > a.S_max);
    }
  }
  return __ballot(bad) == 0;
}

// The largest workspace the attention call asks for.  Split partials exist only when the
// grid has at most 256 workgroups; each holds 128 query rows of (m, l, s, -) in fp32 and 128
// 16-bit values.
constexpr size_t kAttnWorkspaceMax = size_t(256) * 128 * (16 + 128 * 2);

// Host-side dispatch helpers implemented next to the MFMA kernel.
bool mfma_path_applies(medusa_dtype dt, int32_t Hq, int32_t Hkv, int32_t d_h, int32_t N);
size_t attn_workspace_bytes(medusa_dtype dt, int32_t B, int32_t Hq, int32_t Hkv, int32_t d_h,
                            int32_t N, int32_t S_max);
medusa_status run_mfma(AttnArgs& a, int32_t d_h, hipStream_t stream, void* ev_start, void* ev_stop);

}  // namespace medusa
