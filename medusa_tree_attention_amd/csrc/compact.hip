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
// Rounds that fit one workgroup (the usual case: a few sequences, one layer per
// call) run as a single kernel: every sequence's plan is checked one lane per
// sequence, every winning row is read into registers, a barrier orders all
// reads before any write, the rows are written and the prefix lengths advanced.
// Larger rounds: one block per (kv head, sequence, layer) holds that unit's G
// source rows of K and V in LDS, waits on a barrier, then writes them; units are
// disjoint in memory, so no hazard crosses blocks, and a second one-block kernel
// advances the prefix lengths after every layer has been compacted.

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

// Status code of sequence b's plan (0 when valid): the path and its length must be in
// range, every row on the accepted prefix must be a tree row, and the staged block must
// lie inside the cache.  rows[j] receives the accepted path's rows when given.
__device__ __forceinline__ int32_t seq_plan_error(const CompactArgs& a, int b, int32_t* rows) {
  const int best = a.best_path[b], alen = a.accept_len[b];
  const int64_t P = a.prefix_len[b];
  if (best < 0 || best >= a.n_paths || alen < 0 || alen >= a.W) return MEDUSA_EINVAL;
  int32_t err = 0;
#pragma unroll
  for (int j = 0; j < kMaxPathWidth; ++j) {
    if (j <= alen) {
      const int u = a.retrieve[int64_t(best) * a.W + j];
      if (u < 0 || u >= a.n_nodes) err = MEDUSA_EINVAL;
      if (rows) rows[j] = u;
    }
  }
  if (err == 0 && (P < 0 || P + a.n_nodes > a.S_max)) err = MEDUSA_ECAPACITY;
  return err;
}

// 0 when every sequence's plan is valid, else the code of the first sequence that is not.
// Evaluated by a whole wavefront, one lane per sequence; the result is wave-uniform.
__device__ int32_t plan_error(const CompactArgs& a) {
  const int lane = threadIdx.x & 63;
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const int b = b0 + lane;
    const int32_t e = b < a.B ? seq_plan_error(a, b, nullptr) : 0;
    const uint64_t m = __ballot(e != 0);
    if (m) return __shfl(e, __ffsll(static_cast<long long>(m)) - 1);
  }
  return 0;
}

constexpr int kFusedThreads = 1024;
constexpr int kFusedChunks = 16;  // 16-byte chunks each thread carries across the barrier
constexpr int kFusedMaxB = 64;
constexpr int kFusedRetrieve = 4096;  // retrieve entries (n_paths * W) kept in LDS

// q = n / d for 0 <= n < 2^24, 1 <= d < 2^24: the fp32 quotient is within one of the
// exact one, which a single correction step fixes
__device__ __forceinline__ int small_div(int n, int d, float inv_d) {
  int q = int(float(n) * inv_d);
  if ((q + 1) * d <= n) ++q;
  if (q * d > n) --q;
  return q;
}

__global__ __launch_bounds__(kFusedThreads) void compact_fused_kernel(CompactArgs a, int32_t n_layers) {
  const bool failed = round_failed(a.status);  // gates the stores only
  __shared__ int32_t s_alen[kFusedMaxB];
  __shared__ int64_t s_P[kFusedMaxB];
  __shared__ int32_t s_ret[kFusedRetrieve];
  __shared__ int32_t s_rows[kFusedMaxB][kMaxPathWidth];
  __shared__ int32_t s_list[kFusedMaxB * kMaxPathWidth];  // accepted rows: (b << 8) | j
  __shared__ int32_t s_err, s_R;
  const int tid = threadIdx.x;
  // the retrieve table, and each sequence's path, accepted length and prefix length, all
  // loaded at once
  for (int i = tid; i < a.n_paths * a.W; i += kFusedThreads) s_ret[i] = a.retrieve[i];
  int best = 0;
  if (tid < 64 && tid < a.B) {
    best = a.best_path[tid];
    s_alen[tid] = a.accept_len[tid];
    s_P[tid] = a.prefix_len[tid];
  }
  __syncthreads();
  // one lane per sequence: the plan's checks, the accepted rows, the first failing
  // sequence's code and the flat list of rows
  if (tid < 64) {
    const int b = tid;
    int32_t e = 0;
    int G = 0;
    if (b < a.B) {
      const int alen = s_alen[b];
      const int64_t P = s_P[b];
      if (best < 0 || best >= a.n_paths || alen < 0 || alen >= a.W) {
        e = MEDUSA_EINVAL;
      } else {
        for (int j = 0; j <= alen; ++j) {
          const int u = s_ret[best * a.W + j];
          s_rows[b][j] = u;
          if (u < 0 || u >= a.n_nodes) e = MEDUSA_EINVAL;
        }
        if (e == 0 && (P < 0 || P + a.n_nodes > a.S_max)) e = MEDUSA_ECAPACITY;
        if (e == 0) G = alen + 1;
      }
    }
    const uint64_t m = __ballot(e != 0);
    const int32_t first = m ? __shfl(e, __ffsll(static_cast<long long>(m)) - 1) : 0;
    int incl = G;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off, 64);
      if (b >= off) incl += v;
    }
    for (int j = 0; j < G; ++j) s_list[incl - G + j] = (b << 8) | j;
    if (b == 0) s_err = first;
    if (b == 63) s_R = incl;
  }
  __syncthreads();
  if (s_err != 0) {
    if (tid == 0 && !failed) raise_status(a.status, s_err);
    return;
  }
  // chunk c = (accepted row e, column col); a column is (layer, head, K or V, 16-byte x)
  const int cpr = a.row_bytes / 16;  // 8, 16 or 32
  const int cpr_log2 = cpr == 8 ? 3 : cpr == 16 ? 4 : 5;
  const int C = n_layers * a.Hkv * 2 * cpr;
  const int total = s_R * C;
  const float inv_C = 1.0f / float(C > 0 ? C : 1), inv_H = 1.0f / float(a.Hkv);
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  auto locate = [&](int c, bool dst) __attribute__((always_inline)) -> u32x4* {
    const int e = small_div(c, C, inv_C);
    const int col = c - e * C;
    const int entry = s_list[e];
    const int b = entry >> 8, j = entry & 255;
    const int x = col & (cpr - 1);
    const int t = col >> cpr_log2;
    const int kv = t & 1, gl = t >> 1;
    const int layer = small_div(gl, a.Hkv, inv_H), g = gl - layer * a.Hkv;
    const int64_t row = s_P[b] + (dst ? j : s_rows[b][j]);
    u32x4* base = static_cast<u32x4*>(kv ? a.v[layer] : a.k[layer]);
    return base + (((int64_t(b) * a.Hkv + g) * a.S_max + row) << cpr_log2) + x;
  };
  u32x4 v[kFusedChunks];
#pragma unroll
  for (int k = 0; k < kFusedChunks; ++k) {
    const int c = tid + k * kFusedThreads;
    if (c < total) v[k] = *locate(c, false);
  }
  // every source row is read (the loads complete) before any destination is written
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (failed) return;
#pragma unroll
  for (int k = 0; k < kFusedChunks; ++k) {
    const int c = tid + k * kFusedThreads;
    if (c < total) *locate(c, true) = v[k];
  }
  if (tid < a.B) a.prefix_len[tid] = int32_t(s_P[tid] + s_alen[tid] + 1);
}

__global__ __launch_bounds__(256) void compact_kernel(CompactArgs a) {
  const bool failed = round_failed(a.status);  // gates the stores only
  const int32_t err = plan_error(a);
  if (err != 0) {
    if (threadIdx.x == 0 && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && !failed)
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
  if (failed) return;
  for (int c = threadIdx.x; c < 2 * per; c += blockDim.x) {
    const int j = (c % per) / cpr, x = c % cpr;
    uint4* base = c < per ? kc : vc;
    base[(P + j) * cpr + x] = snap[c];
  }
}

__global__ __launch_bounds__(64) void advance_kernel(CompactArgs a) {
  const bool failed = round_failed(a.status);  // gates the stores only
  const int32_t err = plan_error(a);
  if (failed) return;
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
  // one workgroup when the largest possible round fits its registers
  const int64_t max_chunks = int64_t(n_layers) * B * Hkv * 2 * path_width * (a.row_bytes / 16);
  if (n_layers <= kLayersPerLaunch && B <= kFusedMaxB && int64_t(n_paths) * path_width <= kFusedRetrieve &&
      max_chunks <= int64_t(kFusedThreads) * kFusedChunks) {
    for (int32_t i = 0; i < n_layers; ++i) {
      a.k[i] = k_cache[i];
      a.v[i] = v_cache[i];
    }
    void* kargs[] = {&a, &n_layers};
    const void* kern = reinterpret_cast<const void*>(&compact_fused_kernel);
    const hipError_t e =
        ev_start == nullptr && ev_stop == nullptr
            ? hipLaunchKernel(kern, dim3(1), dim3(kFusedThreads), kargs, 0, s)
            : hipExtLaunchKernel(kern, dim3(1), dim3(kFusedThreads), kargs, 0, s, static_cast<hipEvent_t>(ev_start),
                                 static_cast<hipEvent_t>(ev_stop), 0);
    return e == hipSuccess ? MEDUSA_OK : MEDUSA_EHIP;
  }
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
