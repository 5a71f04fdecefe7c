// Winning-path K/V compaction on the device.
//
// [M7.2] = "M7.2 - Medusa: Multi-Head Candidates, Tree Attention, and Verification"
//   §0x06A: G = a + 1; u_j = retrieve[p*, j]; source P + u_j, destination P + j.
//   §0x06B: gather a snapshot of the source rows, then copy, because source
//           and destination rows can overlap; current length becomes P + G.
//   §0x06D: validate indices and capacity before mutating anything; rows past
//           the new length keep their stale bytes.
// "Medusa 完全拆解：多头树式候选如何用一次验证解码多个 Token", section
//   "一次完整解码迭代", step 5: the same path-indexed copy.
//
// One block per (kv head, sequence, layer) holds that unit's G source rows of
// K and V in LDS, waits on a barrier, then writes them.  Units are disjoint in
// memory, so no hazard crosses blocks.  A second one-block kernel advances
// the prefix lengths after every layer has been compacted.

#include "common.h"

namespace medusa {

constexpr int kLayersPerLaunch = 32;
constexpr int kMaxPathWidth = 32;

struct CompactArgs {
  void* k[kLayersPerLaunch];
  void* v[kLayersPerLaunch];
  const int32_t* retrieve;    // [n_paths][W]
  const int32_t* best_path;   // [B]
  const int32_t* accept_len;  // [B]
  int32_t* prefix_len;        // [B]
  int32_t* status;
  int32_t B, Hkv, S_max, n_nodes, n_paths, W, row_bytes;
};

// 0 when every sequence's plan is valid, else the status code to raise.
__device__ int32_t plan_error(const CompactArgs& a) {
  int32_t err = 0;
  for (int b = 0; b < a.B && err == 0; ++b) {
    const int best = a.best_path[b], alen = a.accept_len[b];
    const int64_t P = a.prefix_len[b];
    if (best < 0 || best >= a.n_paths || alen < 0 || alen >= a.W) {
      err = MEDUSA_EINVAL;
      break;
    }
    for (int j = 0; j <= alen; ++j) {
      const int u = a.retrieve[int64_t(best) * a.W + j];
      if (u < 0 || u >= a.n_nodes) err = MEDUSA_EINVAL;
    }
    if (err == 0 && (P < 0 || P + a.n_nodes > a.S_max)) err = MEDUSA_ECAPACITY;
  }
  return err;
}

__global__ __launch_bounds__(256) void compact_kernel(CompactArgs a) {
  if (round_failed(a.status)) return;
  const int32_t err = plan_error(a);
  if (err != 0) {
    if (threadIdx.x == 0 && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
      raise_status(a.status, err);
    return;
  }
  const int g = blockIdx.x, b = blockIdx.y, layer = blockIdx.z;
  const int64_t P = a.prefix_len[b];
  const int G = a.accept_len[b] + 1;
  const int32_t* rows = a.retrieve + int64_t(a.best_path[b]) * a.W;
  const int cpr = a.row_bytes / 16;  // 16-byte chunks per row
  const int64_t head = (int64_t(b) * a.Hkv + g) * a.S_max;
  uint4* kc = static_cast<uint4*>(a.k[layer]) + head * cpr;
  uint4* vc = static_cast<uint4*>(a.v[layer]) + head * cpr;
  extern __shared__ uint4 snap[];  // [2][G][cpr]
  const int per = G * cpr;
  for (int c = threadIdx.x; c < 2 * per; c += blockDim.x) {
    const int j = (c % per) / cpr, x = c % cpr;
    const uint4* base = c < per ? kc : vc;
    snap[c] = base[(P + rows[j]) * cpr + x];
  }
  __syncthreads();  // every source row is read before any destination is written
  for (int c = threadIdx.x; c < 2 * per; c += blockDim.x) {
    const int j = (c % per) / cpr, x = c % cpr;
    uint4* base = c < per ? kc : vc;
    base[(P + j) * cpr + x] = snap[c];
  }
}

__global__ __launch_bounds__(64) void advance_kernel(CompactArgs a) {
  if (round_failed(a.status)) return;
  const int32_t err = plan_error(a);
  if (err != 0) {
    if (threadIdx.x == 0) raise_status(a.status, err);
    return;
  }
  // a single wavefront: every lane has evaluated the plan before any length changes
  for (int b = threadIdx.x; b < a.B; b += blockDim.x) a.prefix_len[b] += a.accept_len[b] + 1;
}

}  // namespace medusa

using namespace medusa;

extern "C" medusa_status medusa_kv_compact(void* stream, medusa_dtype dt, int32_t n_layers,
                                           int32_t B, int32_t Hkv, int32_t d_h, int32_t S_max,
                                           int32_t n_nodes, void* const* k_cache,
                                           void* const* v_cache, const int32_t* d_retrieve,
                                           int32_t n_paths, int32_t path_width,
                                           const int32_t* best_path, const int32_t* accept_len,
                                           int32_t* d_prefix_len, int32_t* d_status,
                                           void* ev_start, void* ev_stop) {
  if (dt != MEDUSA_F32 && dt != MEDUSA_BF16) return MEDUSA_EINVAL;
  if (n_layers < 0 || B < 1 || Hkv < 1 || n_nodes < 1 || S_max < n_nodes || n_paths < 1 ||
      path_width < 1)
    return MEDUSA_EINVAL;
  if (d_h != 64 && d_h != 128) return MEDUSA_EUNSUPPORTED;
  if (path_width > kMaxPathWidth) return MEDUSA_EUNSUPPORTED;
  if (!d_retrieve || !best_path || !accept_len || !d_prefix_len || !d_status) return MEDUSA_EINVAL;
  if (n_layers > 0 && (!k_cache || !v_cache)) return MEDUSA_EINVAL;
  for (int32_t l = 0; l < n_layers; ++l)
    if (!k_cache[l] || !v_cache[l]) return MEDUSA_EINVAL;

  CompactArgs a{};
  a.retrieve = d_retrieve;
  a.best_path = best_path;
  a.accept_len = accept_len;
  a.prefix_len = d_prefix_len;
  a.status = d_status;
  a.B = B;
  a.Hkv = Hkv;
  a.S_max = S_max;
  a.n_nodes = n_nodes;
  a.n_paths = n_paths;
  a.W = path_width;
  a.row_bytes = d_h * (dt == MEDUSA_F32 ? 4 : 2);
  const size_t shmem = size_t(2) * path_width * a.row_bytes;
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int32_t l0 = 0; l0 < n_layers; l0 += kLayersPerLaunch) {
    const int32_t nl = n_layers - l0 < kLayersPerLaunch ? n_layers - l0 : kLayersPerLaunch;
    for (int32_t i = 0; i < nl; ++i) {
      a.k[i] = k_cache[l0 + i];
      a.v[i] = v_cache[l0 + i];
    }
    medusa_status st = launch(reinterpret_cast<const void*>(&compact_kernel),
                              dim3(Hkv, B, nl), dim3(256), shmem, s, a, ev_start, nullptr);
    if (st != MEDUSA_OK) return st;
    ev_start = nullptr;
  }
  return launch(reinterpret_cast<const void*>(&advance_kernel), dim3(1), dim3(64), 0, s, a,
                ev_start, ev_stop);
}
