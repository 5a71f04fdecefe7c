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
//
// Fast typical acceptance, [M7.2] §0x04E: p = softmax(logits / T) of the row that
// scores the next path token, H = -sum p log(p + 1e-5), tau = min(epsilon, alpha
// exp(-H)); an edge passes when p(c) > tau; a_p counts the leading passes; among the
// longest, the largest sum of log p(c) over the accepted edges wins, the first on exact
// ties.  [Chai] "接受机制" gives epsilon = 0.3 and alpha = 0.09.
// Kernel 1 (row statistics): one 1024-thread block per row keeps the row in registers
//                    (32 logits per thread) and takes max, sum of exponentials and the
//                    guarded entropy over them: the row is read from HBM once.
// Kernel 2 (select):  as above, with the typical edge test and the log-likelihood
//                     tie-break.
//
// Accept and commit in one pass (medusa_accept_commit): the greedy select kernel's block
// for sequence b goes on, once it has chosen the path, to compact that sequence's K/V rows
// ([M7.2] §0x06A-§0x06B: cache rows P + j <- P + retrieve[p*][j] for j < G, every layer,
// kv head and matrix) and to hand the next round its starting state ([M7.2] §0x06C: the
// target's token at the terminal row is the next root, and the hidden state of that row
// feeds the next head step).  A thread owns one 16-byte column of one (layer, head,
// matrix) and reads it from all G source rows before writing any destination row, which
// is the snapshot [M7.2] §0x06B asks for (columns are disjoint bytes); only this block
// touches sequence b's rows and length, so no ordering crosses blocks.

#include <algorithm>
#include <cmath>
#include <climits>

#include "common.h"

// the device library's wavefront maximum and sum of a float (declared by the HIP headers only
// under an opt-in macro)
extern "C" __device__ __attribute__((const)) float __ockl_wfred_max_f32(float);
extern "C" __device__ __attribute__((const)) float __ockl_wfred_add_f32(float);

namespace medusa {

constexpr int kCommitLayers = 32;  // layers one accept-and-commit call compacts
constexpr int kCommitWidth = 8;    // path width (K + 1) the commit handles in registers

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
  float4* stats;              // typical: workspace [B][N] (max z, sum 2^(z - max), H, -), base 2
  int32_t* status;
  int32_t B, N, V, n_slots, n_paths, W;
  int32_t parts, chunk4;      // pieces per row; float4 columns per piece (vector path)
  float inv_temperature, epsilon, alpha;  // typical: inv_temperature = log2(e) / T
  // accept and commit
  void* kc[kCommitLayers];    // per layer: cache [B][Hkv][S_max][row_bytes]
  void* vc[kCommitLayers];
  int32_t* prefix_len;        // [B], advanced by G
  const unsigned char* hidden;  // [B][N][hidden_bytes] or null
  unsigned char* h_next;      // [B][hidden_bytes] or null
  int32_t* next_root;         // [B] or null
  int32_t n_layers, Hkv, S_max, row_bytes, hidden_bytes;
  int32_t check_capacity;     // the argmax kernel checks P_b + N <= S_max for every b
};

// Every sequence's staged block [P_b, P_b + N) must lie inside the cache, checked before
// any block of the select kernel advances a length (a block that checked afterwards could
// see an advanced length): by the first block of the kernel that runs before it.
__device__ __forceinline__ void check_capacity(const AcceptArgs& a, bool failed) {
  if (threadIdx.x >= 64) return;
  bool bad = false;
  for (int i = threadIdx.x; i < a.B; i += 64) {
    const int64_t P = a.prefix_len[i];
    bad = bad || P < 0 || P + a.N > a.S_max;
  }
  if (__ballot(bad) && threadIdx.x == 0 && !failed) raise_status(a.status, MEDUSA_ECAPACITY);
}

// the capacity check alone, for target-id rounds (which have no argmax kernel)
__global__ __launch_bounds__(64) void capacity_kernel(AcceptArgs a) {
  check_capacity(a, round_failed(a.status));
}

__device__ __forceinline__ void keep_better(float& v, int& i, float ov, int oi) {
  if (ov > v || (ov == v && oi < i)) {
    v = ov;
    i = oi;
  }
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
// a 16-byte load whose completion the compiler does not track: the caller waits with an
// explicit s_waitcnt and keeps the uses below it.  The logits are read once per round, so
// the load is marked nontemporal (nt): the argmax of the batched round took 9.7 us without
// the hint and 9.0 us with it.
__device__ __forceinline__ f32x4 load_f32x4(const void* p) {
  f32x4 v;
  asm volatile("global_load_dwordx4 %0, %1, off nt" : "=v"(v) : "v"(p) : "memory");
  return v;
}
// maxima without the canonicalising moves fmaxf adds (IEEE: a quiet NaN operand is left out)
__device__ __forceinline__ float vmax(float x, float y) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(x), "v"(y));
  return r;
}
__device__ __forceinline__ float vmax3(float x, float y, float z) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(y), "v"(z));
  return r;
}
// wait until at most n (a constant once unrolled, below 8) of this thread's loads are in flight
__device__ __forceinline__ void wait_loads(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
  }
}

constexpr int kArgmaxThreads = 256;
constexpr int kArgmaxUnroll = 8;  // 16-byte loads each thread has in flight
constexpr int kMaxParts = 16;     // pieces per row at most
constexpr size_t kSelectLds = 65536;  // bytes of tree buffers, candidates and targets
constexpr int kHiddenRegs = 4;         // 16-byte hidden-state chunks per thread held in registers

__global__ __launch_bounds__(kArgmaxThreads) void argmax_kernel(AcceptArgs a) {
  // the status gates the stores only: its load overlaps the logits stream
  const bool failed = round_failed(a.status);
  if (a.check_capacity && blockIdx.x == 0) check_capacity(a, failed);
  const int64_t r = blockIdx.x / a.parts;
  const int piece = int(blockIdx.x % a.parts);
  const float* row = a.logits + r * a.V;
  float best = -INFINITY;
  int idx = INT_MAX;
  bool nan = false;
  const bool vec = (a.V % 4 == 0) && ((reinterpret_cast<uintptr_t>(row) & 15) == 0);
  if (vec) {
    // float4 columns [lo, hi) of the row.  The kArgmaxUnroll loads of a pass are issued
    // back to back as inline assembly (loads past hi read column lo again, in bounds, and
    // are not compared), and each is taken as soon as it has landed, so that the compares
    // overlap the rest of the stream.  Per load: its maximum (v_max_f32 leaves a quiet NaN
    // out; NaNs are flagged on the side and fail the round), kept with the load's four
    // values when it beats the pass's best so far (strictly: an equal value in a later load
    // has a larger index); at the end of the pass the lowest column of the kept load that
    // holds the maximum gives the index.
    const float4* row4 = reinterpret_cast<const float4*>(row);
    const int n4 = a.V / 4;
    const int lo = min(n4, piece * a.chunk4), hi = min(n4, lo + a.chunk4);
    for (int c0 = lo + int(threadIdx.x); c0 < hi; c0 += kArgmaxThreads * kArgmaxUnroll) {
      f32x4 x[kArgmaxUnroll];
#pragma unroll
      for (int k = 0; k < kArgmaxUnroll; ++k) {
        const int c = c0 + k * kArgmaxThreads;
        x[k] = load_f32x4(row4 + (c < hi ? c : lo));
      }
      float pm = -INFINITY;
      int pk = 0;
      f32x4 px = {0.f, 0.f, 0.f, 0.f};
      bool pnan = false;
#pragma unroll
      for (int k = 0; k < kArgmaxUnroll; ++k) {
        wait_loads(kArgmaxUnroll - 1 - k);
        asm volatile("" : "+v"(x[k]));
        const float m = vmax(vmax3(x[k][0], x[k][1], x[k][2]), x[k][3]);
        pnan = pnan || __builtin_isunordered(x[k][0], x[k][1]) || __builtin_isunordered(x[k][2], x[k][3]);
        if (k == 0) {  // column c0 < hi: always in range
          pm = m;
          px = x[0];
        } else {
          const bool take = c0 + k * kArgmaxThreads < hi && m > pm;
          pm = take ? m : pm;
          pk = take ? k : pk;
          px = take ? x[k] : px;
        }
      }
      const int j = px[0] == pm ? 0 : px[1] == pm ? 1 : px[2] == pm ? 2 : 3;
      nan = nan || pnan;
      keep_better(best, idx, pm, 4 * (c0 + pk * kArgmaxThreads) + j);
    }
  } else {
    const int chunk = (a.V + a.parts - 1) / a.parts;
    const int lo = min(a.V, piece * chunk), hi = min(a.V, lo + chunk);
    for (int i = lo + int(threadIdx.x); i < hi; i += kArgmaxThreads) {
      const float e = row[i];
      nan = nan || (e != e);
      if (e == e) keep_better(best, idx, e, i);
    }
  }
  // the wavefront's maximum, then the lowest index holding it (wavefront reductions on the
  // data-parallel primitives, not lane shuffles through LDS)
  const float wm = __ockl_wfred_max_f32(best);
  const uint32_t wi = __ockl_wfred_min_u32(best == wm ? uint32_t(idx) : 0xffffffffu);
  const uint32_t wn = __ockl_wfred_or_u32(nan ? 1u : 0u);
  constexpr int kWaves = kArgmaxThreads / 64;
  __shared__ float wv[kWaves];
  __shared__ int wix[kWaves];
  __shared__ uint32_t wnan[kWaves];
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  if (lane == 0) {
    wv[wave] = wm;
    wix[wave] = int(wi);
    wnan[wave] = wn;
  }
  __syncthreads();
  if (threadIdx.x == 0 && !failed) {
    uint32_t any_nan = wnan[0];
    float v = wv[0];
    int i = wix[0];
    for (int w = 1; w < kWaves; ++w) {
      any_nan |= wnan[w];
      keep_better(v, i, wv[w], wix[w]);
    }
    if (any_nan) {
      raise_status(a.status, MEDUSA_EINVAL);
      return;
    }
    a.part[blockIdx.x] = make_int2(__float_as_int(v), i);
  }
}

// ---------------------------------------------------------------- typical acceptance
constexpr int kStatThreads = 1024;
constexpr int kStatCache = 32;  // logits per thread held in registers: rows up to 32768
constexpr float kLogGuard = 1e-5f;
constexpr float kLn2 = 0.6931471805599453f;

// block-wide reduction of one value per thread (sum or max), the result in every thread:
// per wavefront with the data-parallel primitives, then over the wavefronts through LDS.
// Each reduction of a kernel passes its own scratch (one slot per wavefront), so that one
// barrier suffices.
template <bool kMax>
__device__ __forceinline__ float block_reduce(float v, float* scratch) {
  v = kMax ? __ockl_wfred_max_f32(v) : __ockl_wfred_add_f32(v);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  float r = scratch[0];
  for (int w = 1; w < int(blockDim.x >> 6); ++w) r = kMax ? fmaxf(r, scratch[w]) : r + scratch[w];
  return r;
}

// Row statistics for fast typical acceptance, in base-2 units so that the hardware exp2 and
// log2 serve: z = logits log2(e) / T, M = max z, S = sum 2^(z - M), and the entropy
// H = -ln 2 sum p log2(p + 1e-5) with p = 2^(z - M) / S (the natural-log entropy).  With
// kCached the row (V <= 32768) stays in registers across the three reductions; longer rows
// are streamed three times.
template <bool kCached>
__global__ __launch_bounds__(kStatThreads) void typical_stats_kernel(AcceptArgs a) {
  const bool failed = round_failed(a.status);  // gates the stores only
  __shared__ float scratch[3][kStatThreads / 64];
  const int64_t r = blockIdx.x;
  const float* row = a.logits + r * a.V;
  const int tid = threadIdx.x;
  bool nan = false;
  float M, S, H;
  if (kCached) {
    float z[kStatCache];
    const bool vec = (a.V % 4 == 0) && ((reinterpret_cast<uintptr_t>(row) & 15) == 0);
    if (vec) {  // thread t holds float4 columns t + 1024 k
      const float4* row4 = reinterpret_cast<const float4*>(row);
      const int n4 = a.V / 4;
      // every load of the row issued before any is used (each logit is read once: a
      // nontemporal load), each taken as soon as it has landed
      f32x4 x[kStatCache / 4];
#pragma unroll
      for (int k = 0; k < kStatCache / 4; ++k) {
        const int c = tid + k * kStatThreads;
        x[k] = load_f32x4(row4 + (c < n4 ? c : 0));
      }
#pragma unroll
      for (int k = 0; k < kStatCache / 4; ++k) {
        wait_loads(kStatCache / 4 - 1 - k);
        asm volatile("" : "+v"(x[k]));
        const bool in = tid + k * kStatThreads < n4;
#pragma unroll
        for (int j = 0; j < 4; ++j) z[4 * k + j] = in ? x[k][j] : -INFINITY;
      }
    } else {
#pragma unroll
      for (int k = 0; k < kStatCache; ++k) {
        const int c = tid + k * kStatThreads;
        z[k] = c < a.V ? row[c] : -INFINITY;
      }
    }
    // the maximum of the raw logits: 1/T > 0 keeps their order, so M = max(x) / T
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < kStatCache; k += 2) {
      nan = nan || __builtin_isunordered(z[k], z[k + 1]);
      m = vmax3(m, z[k], z[k + 1]);
    }
    M = block_reduce<true>(m, scratch[0]) * a.inv_temperature;
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < kStatCache; ++k) {
      z[k] = __builtin_amdgcn_exp2f(fmaf(z[k], a.inv_temperature, -M));  // e = 2^(z - M); padding: 0
      s += z[k];
    }
    S = block_reduce<false>(s, scratch[1]);
    // with p = e / S: sum p log2(p + g) = (1/S) sum e log2(e + g S) - log2 S, one product
    // and one logarithm per logit
    const float gs = kLogGuard * S;
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < kStatCache; ++k) t = fmaf(z[k], __builtin_amdgcn_logf(z[k] + gs), t);
    H = (__builtin_amdgcn_logf(S) - block_reduce<false>(t, scratch[2]) / S) * kLn2;
  } else {
    float m = -INFINITY;
    for (int c = tid; c < a.V; c += kStatThreads) {
      const float x = row[c];
      nan = nan || (x != x);
      m = fmaxf(m, x * a.inv_temperature);
    }
    M = block_reduce<true>(m, scratch[0]);
    float s = 0.f;
    for (int c = tid; c < a.V; c += kStatThreads) s += __builtin_amdgcn_exp2f(row[c] * a.inv_temperature - M);
    S = block_reduce<false>(s, scratch[1]);
    const float inv_s = 1.0f / S;
    float h = 0.f;
    for (int c = tid; c < a.V; c += kStatThreads) {
      const float pk = __builtin_amdgcn_exp2f(row[c] * a.inv_temperature - M) * inv_s;
      h -= pk * __builtin_amdgcn_logf(pk + kLogGuard);
    }
    H = block_reduce<false>(h, scratch[2]) * kLn2;
  }
  const bool any_nan = __syncthreads_or(nan);
  if (tid == 0 && !failed) {
    if (any_nan)
      raise_status(a.status, MEDUSA_EINVAL);
    else
      a.stats[r] = make_float4(M, S, H, 0.f);
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

// The edge test of one tree edge (the node at row `parent` scores the candidate token c of
// its child): greedy, c equals the target token of row `parent`; typical, p(c) of that row
// exceeds tau, with log p(c) returned in ll.  `parent` and c must be in range.
template <bool kTypical>
__device__ __forceinline__ bool edge_passes(const AcceptArgs& a, int b, int parent, int c, int32_t tgt_parent,
                                            float& ll) {
  if (kTypical) {
    const int64_t row = int64_t(b) * a.N + parent;
    const float4 st = a.stats[row];
    const float pc = __builtin_amdgcn_exp2f(a.logits[row * a.V + c] * a.inv_temperature - st.x) / st.y;
    const float tau = fminf(a.epsilon, a.alpha * expf(-st.z));
    ll = __builtin_amdgcn_logf(pc) * kLn2;
    return pc > tau;
  }
  return c == tgt_parent;
}

// One block per sequence.  The tree buffers must name valid slots and rows, and every
// retrieve row must start at the root and be padded only at its end; all blocks see the same
// buffers and reach the same verdict.  kTypical selects the typical edge test (candidate ids
// must then be tokens of the vocabulary: they index the logits) and ranks paths of equal
// length by their summed log p.
// With kStaged the tree buffers, this sequence's candidates and the target token of every
// row are first copied to LDS, all loads issued together, and each path's edges are then
// tested side by side rather than one after another along the path (for typical acceptance
// the logits reads of a path are one batch of loads).  Trees too large for LDS walk each
// path from memory.
template <bool kStaged, bool kTypical, bool kCommit = false>
__global__ __launch_bounds__(256) void select_kernel(AcceptArgs a) {
  const bool failed = round_failed(a.status);  // gates the stores only
  const int b = blockIdx.x;
  // the committed length is read with the first loads, not after the path walk: only this
  // block writes it, at the very end
  const int64_t P = kCommit ? a.prefix_len[b] : 0;
  extern __shared__ int32_t sm[];  // tgt[N], tix[N], cand[n_slots], ret[nret]
  const int32_t* tix = a.tree_indices;
  const int32_t* cand = a.candidates + int64_t(b) * a.n_slots;
  const int32_t* ret = a.retrieve;
  const int t = int(threadIdx.x), nret = a.n_paths * a.W;
  bool ok = true;
  // this thread's candidate path: (length, summed log p, index), compared lexicographically
  int best_len = -1, best_i = INT_MAX;
  float best_ll = -INFINITY;
  auto better = [](int l, float ll, int i, int bl, float bll, int bi) {
    return l > bl || (l == bl && (ll > bll || (ll == bll && i < bi)));
  };
  if (kTypical)  // every sequence's candidates, so that all blocks reach the same verdict
    for (int i = t; i < a.B * a.n_slots; i += blockDim.x)
      ok = ok && a.candidates[i] >= 0 && a.candidates[i] < a.V;
  if (kStaged) {
    int32_t* s_tgt = sm;
    int32_t* s_tix = s_tgt + a.N;
    int32_t* s_cand = s_tix + a.N;
    int32_t* s_ret = s_cand + a.n_slots;
    // The first blockDim.x entries of every array come in one batch: each thread loads its
    // entry of each (an index past the end is clamped, in bounds, and not stored) and all
    // the piece results of its row's target, and nothing is stored to LDS before all of
    // them are issued.  Each entry is range-checked as it arrives.  Larger arrays finish in
    // the loops after.
    const int tu = min(t, a.N - 1);
    const int32_t v_tix = tix[tu];
    const int32_t v_cand = cand[min(t, a.n_slots - 1)];
    const int32_t v_ret = ret[min(t, nret - 1)];
    int32_t v_tgt = 0;
    if (!kTypical) {
      const int64_t row = int64_t(b) * a.N + tu;
      if (a.logits) {
        const int2* pr = a.part + row * a.parts;
        int2 pv[kMaxParts];
#pragma unroll
        for (int k = 0; k < kMaxParts; ++k) pv[k] = pr[min(k, a.parts - 1)];
        float v = __int_as_float(pv[0].x);
        int i = pv[0].y;
#pragma unroll
        for (int k = 1; k < kMaxParts; ++k)
          if (k < a.parts) keep_better(v, i, __int_as_float(pv[k].x), pv[k].y);
        v_tgt = i;
      } else {
        v_tgt = a.target_ids[row];
      }
    }
    auto ret_ok = [&](int e, int32_t v) __attribute__((always_inline)) {
      return v >= -1 && v < a.N && (e % a.W != 0 || v == 0);  // in range; the root first
    };
    if (t < a.N) {
      if (!kTypical) s_tgt[t] = v_tgt;
      s_tix[t] = v_tix;
      ok = ok && v_tix >= 0 && v_tix < a.n_slots;
    }
    if (t < a.n_slots) s_cand[t] = v_cand;
    if (t < nret) {
      s_ret[t] = v_ret;
      ok = ok && ret_ok(t, v_ret);
    }
    for (int u = t + int(blockDim.x); u < a.N; u += blockDim.x) {
      if (!kTypical) s_tgt[u] = row_target(a, b, u);
      const int32_t v = tix[u];
      s_tix[u] = v;
      ok = ok && v >= 0 && v < a.n_slots;
    }
    for (int i = t + int(blockDim.x); i < a.n_slots; i += blockDim.x) s_cand[i] = cand[i];
    for (int e = t + int(blockDim.x); e < nret; e += blockDim.x) {
      const int32_t v = ret[e];
      s_ret[e] = v;
      ok = ok && ret_ok(e, v);
    }
    __syncthreads();
    // Every path's run of passing edges from the root, one thread per path: the path's
    // entries are taken eight at a time and the edge tests of all eight issued together
    // (for typical acceptance, one batch of logits loads).  A padded entry fails its edge,
    // and an entry after padding is invalid (padding only at a row's end).
    for (int i = t; i < a.n_paths; i += blockDim.x) {
      const int32_t* r = s_ret + i * a.W;
      int len = 0;
      float ll = 0.f;
      bool run = true;
      int32_t prev = r[0];
      for (int j0 = 1; j0 < a.W; j0 += 8) {
        int32_t v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = j0 + k < a.W ? r[j0 + k] : -1;
        bool pass[8];
        float el[8];
        // branch-free, so that the reads of all eight edges are in flight together: indices
        // are clamped into range and the edge fails where one was not (a slot out of range
        // also fails the round below)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int32_t parent = k == 0 ? prev : v[k - 1], child = v[k];
          ok = ok && !(parent < 0 && child >= 0);
          const int32_t slot = s_tix[max(child, 0)];
          const bool live = child >= 0 && parent >= 0 && slot >= 0 && slot < a.n_slots;
          const int32_t c = s_cand[min(max(slot, 0), a.n_slots - 1)];
          const bool e = edge_passes<kTypical>(a, b, max(parent, 0), kTypical ? min(max(c, 0), a.V - 1) : c,
                                               kTypical ? 0 : s_tgt[max(parent, 0)], el[k]);
          pass[k] = live && e;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          run = run && pass[k];
          if (run) {
            ++len;
            if (kTypical) ll += el[k];
          }
        }
        prev = v[7];
      }
      if (better(len, ll, i, best_len, best_ll, best_i)) {
        best_len = len;
        best_ll = ll;
        best_i = i;
      }
    }
    if (!__syncthreads_and(ok)) {
      if (t == 0 && b == 0 && !failed) raise_status(a.status, MEDUSA_EINVAL);
      return;
    }
    tix = s_tix;
    cand = s_cand;
    ret = s_ret;
  } else {
    for (int u = t; u < a.N; u += blockDim.x) ok = ok && tix[u] >= 0 && tix[u] < a.n_slots;
    for (int i = t; i < a.n_paths; i += blockDim.x) {
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
      if (t == 0 && b == 0 && !failed) raise_status(a.status, MEDUSA_EINVAL);
      return;
    }
    for (int i = t; i < a.n_paths; i += blockDim.x) {
      const int32_t* r = ret + int64_t(i) * a.W;
      int len = 0;
      float ll = 0.f;
      for (int j = 0; j + 1 < a.W; ++j) {
        const int nxt = r[j + 1];
        if (nxt < 0) break;
        float e_ll = 0.f;
        if (!edge_passes<kTypical>(a, b, r[j], cand[tix[nxt]], kTypical ? 0 : row_target(a, b, r[j]), e_ll)) break;
        ll += e_ll;
        ++len;
      }
      if (better(len, ll, i, best_len, best_ll, best_i)) {
        best_len = len;
        best_ll = ll;
        best_i = i;
      }
    }
  }

  // the block's best path: per wavefront the longest length, then the largest summed log p
  // among those, then the lowest index (wavefront reductions), then over the wavefronts
  const int wl = __ockl_wfred_max_i32(best_len);
  const float wll = kTypical ? __ockl_wfred_max_f32(best_len == wl ? best_ll : -INFINITY) : 0.f;
  const uint32_t wi =
      __ockl_wfred_min_u32(best_len == wl && (!kTypical || best_ll == wll) ? uint32_t(best_i) : 0xffffffffu);
  __shared__ int sl[4], si[4];
  __shared__ float sll[4];
  const int wave = t / 64, lane = t % 64;
  if (lane == 0) {
    sl[wave] = wl;
    sll[wave] = wll;
    si[wave] = int(wi);
  }
  __syncthreads();
  int alen = sl[0], best = si[0];
  {
    float bll = sll[0];
    for (int w = 1; w < int(blockDim.x / 64); ++w)
      if (better(sl[w], sll[w], si[w], alen, bll, best)) {
        alen = sl[w];
        bll = sll[w];
        best = si[w];
      }
  }
  if (failed) return;
  const int32_t* r = ret + int64_t(best) * a.W;
  for (int j = t; j < a.W; j += blockDim.x)
    a.accepted[int64_t(b) * a.W + j] = j <= alen ? cand[tix[r[j]]] : -1;
  if (t == 0) {
    a.best_path[b] = best;
    a.accept_len[b] = alen;
    a.frontier[b] = r[alen];
  }
  if (kCommit) {
    const int G = alen + 1;
    const int fr = r[alen];
    // the terminal row's hidden state is loaded together with the cache rows below (the
    // first kHiddenRegs 16-byte chunks per thread; longer states finish afterwards)
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const unsigned char* hs = a.hidden + (int64_t(b) * a.N + fr) * a.hidden_bytes;
    unsigned char* hd = a.h_next + int64_t(b) * a.hidden_bytes;
    const int hchunks = a.h_next ? int(a.hidden_bytes >> 4) : 0;
    u32x4 hv[kHiddenRegs];
#pragma unroll
    for (int k = 0; k < kHiddenRegs; ++k) {
      const int i = t + k * int(blockDim.x);
      if (i < hchunks) hv[k] = *reinterpret_cast<const u32x4*>(hs + 16 * i);
    }
    // staged row j of the winning path moves to row P + j from row P + r[j]; a row already in
    // place (r[j] = j, always so for the root) is left alone, so a round that accepts no
    // candidate moves nothing
    int32_t src[kCommitWidth];
    bool moves = false;
#pragma unroll
    for (int j = 0; j < kCommitWidth; ++j) {
      src[j] = j < G ? r[j] : j;
      moves = moves || src[j] != j;
    }
    if (moves) {
      const int cpr = a.row_bytes >> 4;  // 16-byte columns per row
      const int per_layer = a.Hkv * 2 * cpr;
      const int items = a.n_layers * per_layer;
      // column it of (layer, kv head, matrix): every source row is read before any
      // destination row is written
      for (int it = t; it < items; it += blockDim.x) {
        const int l = it / per_layer, rem = it - l * per_layer;
        const int g = rem / (2 * cpr), rem2 = rem - g * 2 * cpr;
        const int m = rem2 / cpr, c = rem2 - m * cpr;
        unsigned char* base = static_cast<unsigned char*>(m ? a.vc[l] : a.kc[l]) +
                              ((int64_t(b) * a.Hkv + g) * a.S_max + P) * a.row_bytes + 16 * c;
        u32x4 v[kCommitWidth];
#pragma unroll
        for (int j = 0; j < kCommitWidth; ++j)
          if (src[j] != j) v[j] = *reinterpret_cast<const u32x4*>(base + int64_t(src[j]) * a.row_bytes);
#pragma unroll
        for (int j = 0; j < kCommitWidth; ++j)
          if (src[j] != j) *reinterpret_cast<u32x4*>(base + int64_t(j) * a.row_bytes) = v[j];
      }
    }
#pragma unroll
    for (int k = 0; k < kHiddenRegs; ++k) {
      const int i = t + k * int(blockDim.x);
      if (i < hchunks) *reinterpret_cast<u32x4*>(hd + 16 * i) = hv[k];
    }
    for (int i = t + kHiddenRegs * int(blockDim.x); i < hchunks; i += blockDim.x)
      *reinterpret_cast<u32x4*>(hd + 16 * i) = *reinterpret_cast<const u32x4*>(hs + 16 * i);
    // every thread read P before the first barrier (which waits for its loads)
    if (t == 0) {
      if (a.next_root) a.next_root[b] = kStaged ? sm[fr] : row_target(a, b, fr);
      a.prefix_len[b] = int32_t(P + G);
    }
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
  const void* sel = staged ? reinterpret_cast<const void*>(&select_kernel<true, false>)
                           : reinterpret_cast<const void*>(&select_kernel<false, false>);
  return launch(sel, dim3(B), dim3(256), staged ? lds : 0, s, a, ev_start, ev_stop);
}

extern "C" medusa_status medusa_accept_commit(
    void* stream, int32_t B, int32_t N, int32_t V, const float* logits, const int32_t* target_ids,
    const int32_t* candidates, int32_t n_slots, const int32_t* d_tree_indices, const int32_t* d_retrieve,
    int32_t n_paths, int32_t path_width, int32_t* best_path, int32_t* accept_len, int32_t* accepted_tokens,
    int32_t* frontier_row, medusa_dtype dt, int32_t n_layers, int32_t Hkv, int32_t d_h, int32_t S_max,
    void* const* k_cache, void* const* v_cache, int32_t* d_prefix_len, int32_t hidden_dim,
    const void* hidden, void* h_next, int32_t* next_root, void* workspace, size_t workspace_bytes,
    int32_t* d_status, void* ev_start, void* ev_stop) {
  if (B < 1 || N < 1 || n_slots < 1 || n_paths < 1 || path_width < 1) return MEDUSA_EINVAL;
  if ((logits == nullptr) == (target_ids == nullptr)) return MEDUSA_EINVAL;
  if (logits != nullptr && V < 1) return MEDUSA_EINVAL;
  if (!candidates || !d_tree_indices || !d_retrieve || !best_path || !accept_len || !accepted_tokens ||
      !frontier_row || !d_status || !d_prefix_len)
    return MEDUSA_EINVAL;
  if (dt != MEDUSA_F32 && dt != MEDUSA_BF16) return MEDUSA_EINVAL;
  if (n_layers < 0 || Hkv < 1 || S_max < N || hidden_dim < 0) return MEDUSA_EINVAL;
  if (n_layers > 0 && (!k_cache || !v_cache)) return MEDUSA_EINVAL;
  for (int32_t l = 0; l < n_layers; ++l)
    if (!k_cache[l] || !v_cache[l]) return MEDUSA_EINVAL;
  if ((h_next == nullptr) != (hidden == nullptr) || (h_next != nullptr && hidden_dim < 1)) return MEDUSA_EINVAL;
  const int32_t esize = dt == MEDUSA_BF16 ? 2 : 4;
  const int64_t row_bytes = int64_t(d_h) * esize, hidden_bytes = int64_t(hidden_dim) * esize;
  if (d_h < 1 || row_bytes % 16 != 0 || (h_next != nullptr && hidden_bytes % 16 != 0)) return MEDUSA_EUNSUPPORTED;
  if (n_layers > kCommitLayers || path_width > kCommitWidth) return MEDUSA_EUNSUPPORTED;
  for (int32_t l = 0; l < n_layers; ++l)
    if (((reinterpret_cast<uintptr_t>(k_cache[l]) | reinterpret_cast<uintptr_t>(v_cache[l])) & 15) != 0)
      return MEDUSA_EINVAL;
  if (h_next != nullptr &&
      ((reinterpret_cast<uintptr_t>(hidden) | reinterpret_cast<uintptr_t>(h_next)) & 15) != 0)
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
  for (int32_t l = 0; l < n_layers; ++l) {
    a.kc[l] = k_cache[l];
    a.vc[l] = v_cache[l];
  }
  a.prefix_len = d_prefix_len;
  a.hidden = static_cast<const unsigned char*>(hidden);
  a.h_next = static_cast<unsigned char*>(h_next);
  a.next_root = next_root;
  a.n_layers = n_layers;
  a.Hkv = Hkv;
  a.S_max = S_max;
  a.row_bytes = int32_t(row_bytes);
  a.hidden_bytes = int32_t(hidden_bytes);
  a.check_capacity = 1;
  const int64_t rows = int64_t(B) * N;
  const int64_t n4 = (int64_t(V) + 3) / 4;
  const int64_t min_piece = 2 * kArgmaxThreads;
  int64_t parts = std::min<int64_t>({int64_t(kMaxParts), std::max<int64_t>(1, 1024 / rows),
                                     std::max<int64_t>(1, n4 / min_piece)});
  a.parts = int32_t(std::max<int64_t>(1, parts));
  a.chunk4 = int32_t((n4 + a.parts - 1) / a.parts);
  const size_t lds = (2 * size_t(N) + size_t(n_slots) + size_t(n_paths) * path_width) * sizeof(int32_t);
  const bool staged = lds <= kSelectLds;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the capacity of every sequence is checked by a kernel that completes before the select
  // kernel advances any length: the argmax kernel, or a one-wave kernel for target ids
  medusa_status st = logits != nullptr
                         ? launch(reinterpret_cast<const void*>(&argmax_kernel), dim3(unsigned(rows * a.parts)),
                                  dim3(kArgmaxThreads), 0, s, a, ev_start, nullptr)
                         : launch(reinterpret_cast<const void*>(&capacity_kernel), dim3(1), dim3(64), 0, s, a,
                                  ev_start, nullptr);
  if (st != MEDUSA_OK) return st;
  const void* sel = staged ? reinterpret_cast<const void*>(&select_kernel<true, false, true>)
                           : reinterpret_cast<const void*>(&select_kernel<false, false, true>);
  return launch(sel, dim3(B), dim3(256), staged ? lds : 0, s, a, nullptr, ev_stop);
}

extern "C" medusa_status medusa_accept_typical(void* stream, int32_t B, int32_t N, int32_t V,
                                               const float* logits, double temperature, double epsilon,
                                               double alpha, const int32_t* candidates, int32_t n_slots,
                                               const int32_t* d_tree_indices, const int32_t* d_retrieve,
                                               int32_t n_paths, int32_t path_width, int32_t* best_path,
                                               int32_t* accept_len, int32_t* accepted_tokens,
                                               int32_t* frontier_row, void* workspace, size_t workspace_bytes,
                                               int32_t* d_status, void* ev_start, void* ev_stop) {
  if (B < 1 || N < 1 || V < 1 || n_slots < 1 || n_paths < 1 || path_width < 1) return MEDUSA_EINVAL;
  if (!(temperature > 0.0) || !(epsilon >= 0.0) || !(alpha >= 0.0) || !std::isfinite(temperature) ||
      !std::isfinite(epsilon) || !std::isfinite(alpha))
    return MEDUSA_EINVAL;
  if (!logits || !candidates || !d_tree_indices || !d_retrieve || !best_path || !accept_len ||
      !accepted_tokens || !frontier_row || !d_status)
    return MEDUSA_EINVAL;
  if (workspace == nullptr || workspace_bytes < medusa_accept_workspace_size(B, N)) return MEDUSA_EBUFSIZE;

  AcceptArgs a{};
  a.logits = logits;
  a.candidates = candidates;
  a.tree_indices = d_tree_indices;
  a.retrieve = d_retrieve;
  a.best_path = best_path;
  a.accept_len = accept_len;
  a.accepted = accepted_tokens;
  a.frontier = frontier_row;
  a.stats = static_cast<float4*>(workspace);
  a.status = d_status;
  a.B = B;
  a.N = N;
  a.V = V;
  a.n_slots = n_slots;
  a.n_paths = n_paths;
  a.W = path_width;
  a.parts = 1;
  a.inv_temperature = float(1.4426950408889634 / temperature);
  a.epsilon = float(epsilon);
  a.alpha = float(alpha);
  const size_t lds = (2 * size_t(N) + size_t(n_slots) + size_t(n_paths) * path_width) * sizeof(int32_t);
  const bool staged = lds <= kSelectLds;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const void* stats = V <= kStatThreads * kStatCache ? reinterpret_cast<const void*>(&typical_stats_kernel<true>)
                                                     : reinterpret_cast<const void*>(&typical_stats_kernel<false>);
  medusa_status st = launch(stats, dim3(unsigned(int64_t(B) * N)), dim3(kStatThreads), 0, s, a, ev_start, nullptr);
  if (st != MEDUSA_OK) return st;
  const void* sel = staged ? reinterpret_cast<const void*>(&select_kernel<true, true>)
                           : reinterpret_cast<const void*>(&select_kernel<false, true>);
  return launch(sel, dim3(B), dim3(256), staged ? lds : 0, s, a, nullptr, ev_stop);
}
