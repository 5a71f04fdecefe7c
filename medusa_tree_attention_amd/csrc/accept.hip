// Greedy longest-prefix acceptance on the device.
//
// [M7.2] = "M7.2 - Medusa: Multi-Head Candidates, Tree Attention, and Verification"
//   §0x03D: the logits of path row u_j score the token of row u_{j+1}.
//   §0x04D: a_p = sum_j prod_{r<=j} 1[c_{p,r+1} = argmax p_{p,r}]; the first
//           path reaching max a_p wins (path 0 when nothing matches); the
//           round publishes G = a + 1 tokens including the target-chosen root.
//   §0x07B: the posterior can be evaluated once per unique packed row instead
//           of on a [paths, width, V] gather -- done here: one argmax per row.
// "Medusa Part II: Candidate Trees, Verification, and Acceptance", Part 7:
//   the same cumulative-product rule; padded slots are path ends, not tokens.
//
// Kernel 1 (argmax): one block per (sequence, row) streams the V logits once,
//                    eight 16-byte loads in flight per thread.
// Kernel 2 (select):  one block per sequence counts each path's matching
//                     prefix and picks the first longest.

#include <climits>

#include "common.h"

namespace medusa {

struct AcceptArgs {
  const float* logits;        // [B][N][V] or null
  const int32_t* target_ids;  // [B][N] or null
  const int32_t* candidates;  // [B][n_slots]
  const int32_t* tree_indices;  // [N]
  const int32_t* retrieve;    // [n_paths][W]
  int32_t* best_path;         // [B]
  int32_t* accept_len;        // [B]
  int32_t* accepted;          // [B][W]
  int32_t* frontier;          // [B]
  int32_t* target;            // workspace [B][N]
  int32_t* status;
  int32_t B, N, V, n_slots, n_paths, W;
};

__device__ __forceinline__ void keep_better(float& v, int& i, float ov, int oi) {
  if (ov > v || (ov == v && oi < i)) {
    v = ov;
    i = oi;
  }
}

constexpr int kArgmaxThreads = 512;
constexpr int kArgmaxUnroll = 8;  // 16-byte loads each thread has in flight

__global__ __launch_bounds__(kArgmaxThreads) void argmax_kernel(AcceptArgs a) {
  if (round_failed(a.status)) return;
  const int64_t r = blockIdx.x;
  const float* row = a.logits + r * a.V;
  float best = -INFINITY;
  int idx = INT_MAX;
  bool nan = false;
  auto take = [&](float e, int i) __attribute__((always_inline)) {
    nan = nan || (e != e);
    if (e == e) keep_better(best, idx, e, i);
  };
  const bool vec = (a.V % 4 == 0) && ((reinterpret_cast<uintptr_t>(row) & 15) == 0);
  if (vec) {
    // kArgmaxUnroll loads per thread are issued before any is compared, so that a row is
    // streamed with about 64 KiB in flight per workgroup; loads past the row end read
    // element 0 again (in bounds) and are not compared
    const float4* row4 = reinterpret_cast<const float4*>(row);
    const int n4 = a.V / 4;
    for (int c0 = threadIdx.x; c0 < n4; c0 += kArgmaxThreads * kArgmaxUnroll) {
      float4 x[kArgmaxUnroll];
#pragma unroll
      for (int k = 0; k < kArgmaxUnroll; ++k) {
        const int c = c0 + k * kArgmaxThreads;
        x[k] = row4[c < n4 ? c : 0];
      }
#pragma unroll
      for (int k = 0; k < kArgmaxUnroll; ++k) {
        const int c = c0 + k * kArgmaxThreads;
        if (c < n4) {
          take(x[k].x, 4 * c);
          take(x[k].y, 4 * c + 1);
          take(x[k].z, 4 * c + 2);
          take(x[k].w, 4 * c + 3);
        }
      }
    }
  } else {
    for (int i = threadIdx.x; i < a.V; i += kArgmaxThreads) take(row[i], i);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(best, off, 64);
    const int oi = __shfl_xor(idx, off, 64);
    keep_better(best, idx, ov, oi);
  }
  constexpr int kWaves = kArgmaxThreads / 64;
  __shared__ float wv[kWaves];
  __shared__ int wi[kWaves];
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  if (lane == 0) {
    wv[wave] = best;
    wi[wave] = idx;
  }
  const bool any_nan = __syncthreads_or(nan);
  if (threadIdx.x == 0) {
    if (any_nan) {
      raise_status(a.status, MEDUSA_EINVAL);
      return;
    }
    for (int w = 1; w < kWaves; ++w) keep_better(wv[0], wi[0], wv[w], wi[w]);
    a.target[r] = wi[0];
  }
}

// The tree buffers must name valid slots and rows, every retrieve row must
// start at the root and be padded only at its end.  All blocks see the same
// buffers and reach the same verdict.
__device__ bool tree_buffers_valid(const AcceptArgs& a) {
  bool ok = true;
  for (int u = threadIdx.x; u < a.N; u += blockDim.x) {
    const int s = a.tree_indices[u];
    ok = ok && s >= 0 && s < a.n_slots;
  }
  for (int i = threadIdx.x; i < a.n_paths; i += blockDim.x) {
    const int32_t* r = a.retrieve + int64_t(i) * a.W;
    ok = ok && r[0] == 0;
    bool ended = false;
    for (int j = 0; j < a.W; ++j) {
      const int v = r[j];
      ok = ok && v >= -1 && v < a.N && !(ended && v != -1);
      ended = ended || v == -1;
    }
  }
  return __syncthreads_and(ok);
}

__global__ __launch_bounds__(256) void select_kernel(AcceptArgs a) {
  if (round_failed(a.status)) return;
  if (!tree_buffers_valid(a)) {
    if (threadIdx.x == 0 && blockIdx.x == 0) raise_status(a.status, MEDUSA_EINVAL);
    return;
  }
  const int b = blockIdx.x;
  const int32_t* tgt = a.logits ? a.target + int64_t(b) * a.N : a.target_ids + int64_t(b) * a.N;
  const int32_t* cand = a.candidates + int64_t(b) * a.n_slots;

  int best_len = -1, best_i = INT_MAX;
  for (int i = threadIdx.x; i < a.n_paths; i += blockDim.x) {
    const int32_t* r = a.retrieve + int64_t(i) * a.W;
    int len = 0;
    for (int j = 0; j + 1 < a.W; ++j) {
      const int nxt = r[j + 1];
      if (nxt < 0 || cand[a.tree_indices[nxt]] != tgt[r[j]]) break;
      ++len;
    }
    if (len > best_len || (len == best_len && i < best_i)) {
      best_len = len;
      best_i = i;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const int ol = __shfl_xor(best_len, off, 64);
    const int oi = __shfl_xor(best_i, off, 64);
    if (ol > best_len || (ol == best_len && oi < best_i)) {
      best_len = ol;
      best_i = oi;
    }
  }
  __shared__ int sl[4], si[4];
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  if (lane == 0) {
    sl[wave] = best_len;
    si[wave] = best_i;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < int(blockDim.x / 64); ++w) {
      if (sl[w] > sl[0] || (sl[w] == sl[0] && si[w] < si[0])) {
        sl[0] = sl[w];
        si[0] = si[w];
      }
    }
  }
  __syncthreads();
  const int alen = sl[0], best = si[0];
  const int32_t* r = a.retrieve + int64_t(best) * a.W;
  for (int j = threadIdx.x; j < a.W; j += blockDim.x)
    a.accepted[int64_t(b) * a.W + j] = j <= alen ? cand[a.tree_indices[r[j]]] : -1;
  if (threadIdx.x == 0) {
    a.best_path[b] = best;
    a.accept_len[b] = alen;
    a.frontier[b] = r[alen];
  }
}

}  // namespace medusa

using namespace medusa;

extern "C" size_t medusa_accept_workspace_size(int32_t B, int32_t N) {
  if (B < 1 || N < 1) return 0;
  return (size_t(B) * size_t(N) * sizeof(int32_t) + 255) / 256 * 256;
}

extern "C" medusa_status medusa_accept(void* stream, int32_t B, int32_t N, int32_t V,
                                       const float* logits, const int32_t* target_ids,
                                       const int32_t* candidates, int32_t n_slots,
                                       const int32_t* d_tree_indices, const int32_t* d_retrieve,
                                       int32_t n_paths, int32_t path_width, int32_t* best_path,
                                       int32_t* accept_len, int32_t* accepted_tokens,
                                       int32_t* frontier_row, void* workspace,
                                       size_t workspace_bytes, int32_t* d_status, void* ev_start,
                                       void* ev_stop) {
  if (B < 1 || N < 1 || n_slots < 1 || n_paths < 1 || path_width < 1) return MEDUSA_EINVAL;
  if ((logits == nullptr) == (target_ids == nullptr)) return MEDUSA_EINVAL;
  if (logits != nullptr && V < 1) return MEDUSA_EINVAL;
  if (!candidates || !d_tree_indices || !d_retrieve || !best_path || !accept_len ||
      !accepted_tokens || !frontier_row || !d_status)
    return MEDUSA_EINVAL;
  if (logits != nullptr &&
      (workspace == nullptr || workspace_bytes < medusa_accept_workspace_size(B, N)))
    return MEDUSA_EBUFSIZE;

  AcceptArgs a{};
  a.logits = logits;
  a.target_ids = target_ids;
  a.candidates = candidates;
  a.tree_indices = d_tree_indices;
  a.retrieve = d_retrieve;
  a.best_path = best_path;
  a.accept_len = accept_len;
  a.accepted = accepted_tokens;
  a.frontier = frontier_row;
  a.target = static_cast<int32_t*>(workspace);
  a.status = d_status;
  a.B = B;
  a.N = N;
  a.V = V;
  a.n_slots = n_slots;
  a.n_paths = n_paths;
  a.W = path_width;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (logits != nullptr) {
    medusa_status st = launch(reinterpret_cast<const void*>(&argmax_kernel),
                              dim3(unsigned(int64_t(B) * N)), dim3(kArgmaxThreads), 0, s, a, ev_start, nullptr);
    if (st != MEDUSA_OK) return st;
    ev_start = nullptr;
  }
  return launch(reinterpret_cast<const void*>(&select_kernel), dim3(B), dim3(256), 0, s, a,
                ev_start, ev_stop);
}
