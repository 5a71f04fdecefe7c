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
// Kernel 1 (argmax): each (sequence, row) is cut into `parts` contiguous pieces, one
//                    block per piece, every thread issuing all of its 16-byte loads
//                    before comparing; each block leaves the (value, index) winner of
//                    its piece in the workspace.
// Kernel 2 (select):  one block per sequence combines the pieces' winners of its rows,
//                     counts each path's matching prefix and picks the first longest.

#include <algorithm>
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
  int2* part;                 // workspace [B][N][parts]: (value bits, index) of each piece
  int32_t* status;
  int32_t B, N, V, n_slots, n_paths, W;
  int32_t parts, chunk4;      // pieces per row; float4 columns per piece (vector path)
};

__device__ __forceinline__ void keep_better(float& v, int& i, float ov, int oi) {
  if (ov > v || (ov == v && oi < i)) {
    v = ov;
    i = oi;
  }
}

constexpr int kArgmaxThreads = 256;
constexpr int kArgmaxUnroll = 8;  // 16-byte loads each thread has in flight
constexpr int kMaxParts = 16;     // pieces per row at most
constexpr size_t kSelectLds = 65536;  // bytes of tree buffers, candidates and targets

__global__ __launch_bounds__(kArgmaxThreads) void argmax_kernel(AcceptArgs a) {
  // the status gates the stores only: its load overlaps the logits stream
  const bool failed = round_failed(a.status);
  const int64_t r = blockIdx.x / a.parts;
  const int piece = int(blockIdx.x % a.parts);
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
    // float4 columns [lo, hi) of the row; all kArgmaxUnroll loads of a pass are issued
    // before any is compared, and loads past hi read column lo again (in bounds) and are
    // not compared
    const float4* row4 = reinterpret_cast<const float4*>(row);
    const int n4 = a.V / 4;
    const int lo = min(n4, piece * a.chunk4), hi = min(n4, lo + a.chunk4);
    for (int c0 = lo + int(threadIdx.x); c0 < hi; c0 += kArgmaxThreads * kArgmaxUnroll) {
      float4 x[kArgmaxUnroll];
#pragma unroll
      for (int k = 0; k < kArgmaxUnroll; ++k) {
        const int c = c0 + k * kArgmaxThreads;
        x[k] = row4[c < hi ? c : lo];
      }
#pragma unroll
      for (int k = 0; k < kArgmaxUnroll; ++k) {
        const int c = c0 + k * kArgmaxThreads;
        if (c < hi) {
          take(x[k].x, 4 * c);
          take(x[k].y, 4 * c + 1);
          take(x[k].z, 4 * c + 2);
          take(x[k].w, 4 * c + 3);
        }
      }
    }
  } else {
    const int chunk = (a.V + a.parts - 1) / a.parts;
    const int lo = min(a.V, piece * chunk), hi = min(a.V, lo + chunk);
    for (int i = lo + int(threadIdx.x); i < hi; i += kArgmaxThreads) take(row[i], i);
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
  if (threadIdx.x == 0 && !failed) {
    if (any_nan) {
      raise_status(a.status, MEDUSA_EINVAL);
      return;
    }
    for (int w = 1; w < kWaves; ++w) keep_better(wv[0], wi[0], wv[w], wi[w]);
    a.part[blockIdx.x] = make_int2(__float_as_int(wv[0]), wi[0]);
  }
}

// target token of row u of sequence b: the winner over the row's pieces (the lowest index
// among equal values), or the given id
__device__ __forceinline__ int32_t row_target(const AcceptArgs& a, int b, int u) {
  const int64_t row = int64_t(b) * a.N + u;
  if (!a.logits) return a.target_ids[row];
  const int2* pr = a.part + row * a.parts;
  float v = __int_as_float(pr[0].x);
  int i = pr[0].y;
  for (int k = 1; k < a.parts; ++k) keep_better(v, i, __int_as_float(pr[k].x), pr[k].y);
  return i;
}

// One block per sequence.  With kStaged, the tree buffers, this sequence's candidates and
// the target token of every row are first copied to LDS (all loads issued together), so
// that the path walks below make no dependent global loads; trees too large for that read
// them from memory.  The tree buffers must name valid slots and rows, and every retrieve
// row must start at the root and be padded only at its end; all blocks see the same
// buffers and reach the same verdict.
template <bool kStaged>
__global__ __launch_bounds__(256) void select_kernel(AcceptArgs a) {
  const bool failed = round_failed(a.status);  // gates the stores only
  const int b = blockIdx.x;
  extern __shared__ int32_t sm[];  // tgt[N], tix[N], cand[n_slots], ret[n_paths][W]
  const int32_t* tix = a.tree_indices;
  const int32_t* cand = a.candidates + int64_t(b) * a.n_slots;
  const int32_t* ret = a.retrieve;
  if (kStaged) {
    int32_t* s_tgt = sm;
    int32_t* s_tix = s_tgt + a.N;
    int32_t* s_cand = s_tix + a.N;
    int32_t* s_ret = s_cand + a.n_slots;
    for (int u = threadIdx.x; u < a.N; u += blockDim.x) {
      s_tgt[u] = row_target(a, b, u);
      s_tix[u] = tix[u];
    }
    for (int i = threadIdx.x; i < a.n_slots; i += blockDim.x) s_cand[i] = cand[i];
    for (int i = threadIdx.x; i < a.n_paths * a.W; i += blockDim.x) s_ret[i] = ret[i];
    __syncthreads();
    tix = s_tix;
    cand = s_cand;
    ret = s_ret;
  }
  auto tgt = [&](int u) __attribute__((always_inline)) { return kStaged ? sm[u] : row_target(a, b, u); };

  bool ok = true;
  for (int u = threadIdx.x; u < a.N; u += blockDim.x) ok = ok && tix[u] >= 0 && tix[u] < a.n_slots;
  for (int i = threadIdx.x; i < a.n_paths; i += blockDim.x) {
    const int32_t* r = ret + int64_t(i) * a.W;
    ok = ok && r[0] == 0;
    bool ended = false;
    for (int j = 0; j < a.W; ++j) {
      const int v = r[j];
      ok = ok && v >= -1 && v < a.N && !(ended && v != -1);
      ended = ended || v == -1;
    }
  }
  if (!__syncthreads_and(ok)) {
    if (threadIdx.x == 0 && blockIdx.x == 0 && !failed) raise_status(a.status, MEDUSA_EINVAL);
    return;
  }

  int best_len = -1, best_i = INT_MAX;
  for (int i = threadIdx.x; i < a.n_paths; i += blockDim.x) {
    const int32_t* r = ret + int64_t(i) * a.W;
    int len = 0;
    for (int j = 0; j + 1 < a.W; ++j) {
      const int nxt = r[j + 1];
      if (nxt < 0 || cand[tix[nxt]] != tgt(r[j])) break;
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
  if (failed) return;
  const int alen = sl[0], best = si[0];
  const int32_t* r = ret + int64_t(best) * a.W;
  for (int j = threadIdx.x; j < a.W; j += blockDim.x)
    a.accepted[int64_t(b) * a.W + j] = j <= alen ? cand[tix[r[j]]] : -1;
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
  return (size_t(B) * size_t(N) * kMaxParts * sizeof(int2) + 255) / 256 * 256;
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
  a.part = static_cast<int2*>(workspace);
  a.status = d_status;
  a.B = B;
  a.N = N;
  a.V = V;
  a.n_slots = n_slots;
  a.n_paths = n_paths;
  a.W = path_width;
  // pieces per row: about 1024 blocks over the whole batch, no piece under two loads per
  // thread (512 float4 columns)
  const int64_t rows = int64_t(B) * N;
  const int64_t n4 = (int64_t(V) + 3) / 4;
  const int64_t min_piece = 2 * kArgmaxThreads;
  int64_t parts = std::min<int64_t>({int64_t(kMaxParts), std::max<int64_t>(1, 1024 / rows),
                                     std::max<int64_t>(1, n4 / min_piece)});
  a.parts = int32_t(std::max<int64_t>(1, parts));
  a.chunk4 = int32_t((n4 + a.parts - 1) / a.parts);
  // the select kernel keeps the tree buffers, the candidates and the row targets in LDS
  // when they fit
  const size_t lds = (2 * size_t(N) + size_t(n_slots) + size_t(n_paths) * path_width) * sizeof(int32_t);
  const bool staged = lds <= kSelectLds;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (logits != nullptr) {
    medusa_status st = launch(reinterpret_cast<const void*>(&argmax_kernel),
                              dim3(unsigned(rows * a.parts)), dim3(kArgmaxThreads), 0, s, a, ev_start, nullptr);
    if (st != MEDUSA_OK) return st;
    ev_start = nullptr;
  }
  const void* sel = staged ? reinterpret_cast<const void*>(&select_kernel<true>)
                           : reinterpret_cast<const void*>(&select_kernel<false>);
  return launch(sel, dim3(B), dim3(256), staged ? lds : 0, s, a, ev_start, ev_stop);
}
