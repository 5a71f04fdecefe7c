// The Medusa head step and the candidate pool on the device (bf16 weights, gfx950).
//
// [Chai] = "Medusa 完全拆解：多头树式候选如何用一次验证解码多个 Token"
//   section "Medusa 的核心思路与系统位置": head k gives softmax(W2_k (SiLU(W1_k h) + h)),
//   W1_k [d, d], W2_k [V, d], column-vector convention.
// [Math] = "Medusa — Multi-Head Speculative Decoding Math", section "The Medusa head: math
//   and shapes": the same residual block feeding an unembedding.
// "Medusa Part II: Candidate Trees, Verification, and Acceptance", Part 4: each head
//   contributes its TOPK ranked ids (top-k of the head logits; the softmax does not change
//   the order).
// [M7.2] = "M7.2 - Medusa: Multi-Head Candidates, Tree Attention, and Verification"
//   §0x01B: slot(j, r) = 1 + j TOPK + r; [Chai] "一次完整解码迭代": the LM head gives the
//   root token (slot 0), the heads the rest.
//
// Mapping to CDNA4: both products are matrix-vector products against B <= 4 columns per
// pass, so every bf16 weight feeds four fp32 FMAs: the step is HBM-bound on the weights
// (4 heads x (d^2 + V d) x 2 bytes = 1.18 GB for d = 4096, V = 32000) and runs on the
// vector ALUs, not the matrix cores.
//  * GEMV: a workgroup of eight wavefronts owns a contiguous range of output rows of one
//    head and keeps the (up to four) input columns in LDS as fp32, zero-padded to a
//    multiple of 512.  A wavefront takes eight rows at a time; lane l reads 16 bytes (8
//    weights) of each of them per step, so one instruction loads 1 KiB of a row, and
//    accumulates 8 rows x 4 columns in fp32.  The next step's eight loads are issued before
//    the current step's FMAs (two register buffers), and at most 128 VGPRs keep two
//    workgroups (16 wavefronts) on every compute unit.  A row group's 32 sums are reduced
//    across the wavefront by a transposed butterfly: each exchange halves the values a
//    lane holds, 32 shuffles in all.  When the rows are too few to give every compute unit
//    16 wavefronts (the d x d residual product), 2..8 wavefronts split each row group's
//    columns and add their sums through LDS.
//  * The residual kernel writes u = SiLU(W1 h) + h in fp32; the unembedding kernel writes
//    the logits in fp32.
//  * Top-k in two passes: every unembedding workgroup ranks the best topk of its (at most
//    512) rows per column right after computing them -- the logits go to LDS, one wavefront
//    per column takes rounds over ranking keys held in registers, without barriers -- and
//    one workgroup per (head, sequence) then merges the workgroups' lists.  An entry is
//    ranked by one 64-bit key (value order in the high word, inverted index in the low
//    word, so among equal logits the lower token id ranks first); round r takes the
//    largest key below round r-1's winner (DPP maxima within a wavefront).  The logits
//    themselves are written only when the caller asks for them.

#include <algorithm>
#include <climits>
#include <cmath>

#include "common.h"

namespace medusa {
namespace {

constexpr int kGemvThreads = 512;
constexpr int kGemvWaves = kGemvThreads / 64;
constexpr int kGemvRows = 8;      // rows per wavefront group
constexpr int kBlockRows = 512;   // output rows per workgroup at most (staged in LDS; ranked in registers)
constexpr int kCols = 4;          // input columns per launch
constexpr int kPad = 512;         // LDS columns are zero-padded to a multiple of this
constexpr int kMergeThreads = 256;
constexpr int kMergeCache = 8;    // list keys per merge thread held in registers
constexpr int kMaxTopk = 64;
constexpr int kMaxD = 8192;
constexpr int kSplitBelow = 256 * 8;    // row groups are shared only below 8 per compute unit
// cache policy of the weight loads: nontemporal (nt).  Every weight is read once per call;
// marking the stream nontemporal took the unembedding product of the batched full round from
// 191.5 to 175.2 us
constexpr int kStreamLoad = 2;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// The ranking as one unsigned 64-bit key: the high word maps the float order onto the
// unsigned order (negative values bit-inverted, non-negative ones with the sign bit set;
// -0 is taken as +0 first), the low word is the inverted index, so the largest key is the
// largest value and, among equal values, the lowest index.  Key 0 lies below every real
// entry (it stands for "none"); a NaN never gets a key (it is reported instead).
__device__ __forceinline__ uint64_t rank_key(float v, int i) {
  unsigned b = __float_as_uint(v == 0.f ? 0.f : v);
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return (uint64_t(b) << 32) | uint64_t(~unsigned(i));
}
__device__ __forceinline__ int key_index(uint64_t key) { return int(~unsigned(key)); }
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <int kCtrl>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x) {
  const unsigned lo = __builtin_amdgcn_update_dpp(0u, unsigned(x), kCtrl, 0xf, 0xf, false);
  const unsigned hi = __builtin_amdgcn_update_dpp(0u, unsigned(x >> 32), kCtrl, 0xf, 0xf, false);
  return (uint64_t(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t x, int lane) {
  const unsigned lo = __builtin_amdgcn_readlane(unsigned(x), lane);
  const unsigned hi = __builtin_amdgcn_readlane(unsigned(x >> 32), lane);
  return (uint64_t(hi) << 32) | lo;
}
// maximum over the wavefront (all lanes active), uniform: the quad swaps, the half-row and
// row mirrors leave every row of 16 lanes with its maximum, then the four rows are read out
__device__ __forceinline__ uint64_t wave_max_key(uint64_t x) {
  x = max_u64(x, dpp_u64<0xB1>(x));   // quad_perm [1, 0, 3, 2]
  x = max_u64(x, dpp_u64<0x4E>(x));   // quad_perm [2, 3, 0, 1]
  x = max_u64(x, dpp_u64<0x141>(x));  // row_half_mirror
  x = max_u64(x, dpp_u64<0x140>(x));  // row_mirror
  return max_u64(max_u64(readlane_u64(x, 0), readlane_u64(x, 16)),
                 max_u64(readlane_u64(x, 32), readlane_u64(x, 48)));
}
// maximum over the workgroup; slot[2][waves] alternates by round so that one barrier per
// round suffices (a slot is rewritten two rounds later, after the next barrier)
template <int kThreads>
__device__ __forceinline__ uint64_t block_max_key(uint64_t x, uint64_t (*slot)[kThreads / 64], int round) {
  const int wave = threadIdx.x >> 6;
  x = wave_max_key(x);
  if ((threadIdx.x & 63) == 0) slot[round & 1][wave] = x;
  __syncthreads();
  x = slot[round & 1][0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) x = max_u64(x, slot[round & 1][w]);
  return x;
}

constexpr uint64_t kNanList = ~uint64_t(0);  // marks a ranked list whose rows hold a NaN

struct GemvArgs {
  const bf16* W;        // [K][R][d]
  const bf16* x_bf16;   // residual kernel: h [B][d]
  const float* x_f32;   // unembedding kernel: u [K][B][d]
  float* out;           // [K][B][R]; the unembedding kernel's logits, or null
  int32_t* status;
  uint64_t* keys;       // unembedding kernel: [K][B][nblk][topk] ranked keys per row block
  int32_t B, d, dpad, R, col0, ncols, rows_per_block, split, topk, nblk;
};

struct TopkArgs {
  const int32_t* root;  // [B]
  int32_t* candidates;  // [B][1 + K topk]
  int32_t* status;
  uint64_t* seg_keys;   // [K][B][S][topk] ranked keys of the unembedding row blocks
  int32_t B, K, V, topk, S;
};

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

template <bool kResidual>
__global__ __launch_bounds__(kGemvThreads) __attribute__((amdgpu_waves_per_eu(4)))
void head_gemv_kernel(GemvArgs g) {
  __shared__ float part[kGemvWaves][32];       // split row groups: partial sums
  extern __shared__ float xs[];                // [kCols][dpad], zero past d
  const int k = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar loop state

  // The input columns, widened to fp32, in 16-byte pieces: a batch is up to kFill pieces
  // per thread whose loads (clamped to valid addresses) are all issued before any is
  // converted and stored.  Pieces past the inputs store zeros.
  constexpr int kFill = 8;
  const int per = kResidual ? 8 : 4;  // elements per 16-byte piece
  const int np = g.dpad / per;        // pieces per column
  u32x4 raw[kFill];
  int dst[kFill];
  bool ok[kFill];
  // buffer loads, like the weights', so that every load of the kernel is counted in order
  const int esz = kResidual ? 2 : 4;
  const void* xbase = kResidual ? static_cast<const void*>(g.x_bf16)
                                : static_cast<const void*>(g.x_f32 + int64_t(k) * g.B * g.d);
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(xbase), short(0), int(unsigned(g.B) * unsigned(g.d) * unsigned(esz)), 0x00020000);
  auto fill_issue = [&](int p0) __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < kFill; ++f) {
      const int p = p0 + f * kGemvThreads;
      const int c = p / np, e = (p - c * np) * per;
      dst[f] = p < kCols * np ? c * g.dpad + e : -1;
      ok[f] = p < kCols * np && c < g.ncols && e < g.d;
      const int cc = ok[f] ? c : 0, ee = ok[f] ? e : 0;
      const unsigned off = (unsigned(g.col0 + cc) * unsigned(g.d) + unsigned(ee)) * unsigned(esz);
      raw[f] = __builtin_amdgcn_raw_buffer_load_b128(xres, off, 0u, 0);
    }
  };
  auto fill_store = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < kFill; ++f) {
      if (dst[f] < 0) continue;
      const u32x4 q = ok[f] ? raw[f] : u32x4{0u, 0u, 0u, 0u};
      if (kResidual) {
        *reinterpret_cast<float4*>(xs + dst[f]) =
            make_float4(bf16_lo(q[0]), bf16_hi(q[0]), bf16_lo(q[1]), bf16_hi(q[1]));
        *reinterpret_cast<float4*>(xs + dst[f] + 4) =
            make_float4(bf16_lo(q[2]), bf16_hi(q[2]), bf16_lo(q[3]), bf16_hi(q[3]));
      } else {
        *reinterpret_cast<float4*>(xs + dst[f]) = make_float4(
            __uint_as_float(q[0]), __uint_as_float(q[1]), __uint_as_float(q[2]), __uint_as_float(q[3]));
      }
    }
  };

  // wavefront -> (row slot, column part); parts of one slot are adjacent wavefronts
  const int slot = wave / g.split, pid = wave - slot * g.split;
  const int stride = (kGemvWaves / g.split) * kGemvRows;
  const int r0 = blockIdx.x * g.rows_per_block;
  const int r1 = min(g.R, r0 + g.rows_per_block);
  const int chunks = g.d >> 3;                 // 16-byte pieces of a row
  const int nch = g.dpad / kPad;               // 64-piece columns of a row
  const int my_nch = (nch - pid + g.split - 1) / g.split;
  const int first = r0 + slot * kGemvRows;
  const int ngroups = first < r1 && my_nch > 0 ? (r1 - first + stride - 1) / stride : 0;
  const int steps = ngroups * my_nch;
  const bf16* Wk = g.W + int64_t(k) * g.R * g.d;

  // The weights of head k through one buffer resource (byte offsets below 2^32, checked
  // on the host): a lane's offset in a VGPR, the row step in an SGPR.  Step j of a group
  // covers piece lane + 64 (pid + split j) of each row; pieces past the row re-read its last
  // piece and meet zeros in xs; rows past the range re-read the range's last row.
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16*>(Wk), short(0), int(unsigned(g.R) * unsigned(g.d) * 2u), 0x00020000);
  auto load = [&](int base, int j, u32x4 (&w)[kGemvRows]) __attribute__((always_inline)) {
    const int ch = min(lane + 64 * (pid + g.split * j), chunks - 1);
    const unsigned voff = (unsigned(base) * unsigned(g.d) + 8u * unsigned(ch)) * 2u;
    const int last = r1 - 1 - base;  // >= 0: a group starts inside the range
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) {
      const int rr = r < last ? r : last;
      w[r] = __builtin_amdgcn_raw_buffer_load_b128(wres, voff, unsigned(rr) * unsigned(g.d) * 2u, kStreamLoad);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the FMAs that follow
  };
  auto fma_step = [&](int j, const u32x4 (&w)[kGemvRows], float (&acc)[kGemvRows][kCols])
      __attribute__((always_inline)) {
    const int xo = 8 * (lane + 64 * (pid + g.split * j));
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      float xv[kCols][4];
#pragma unroll
      for (int c = 0; c < kCols; ++c) {
        const float4 t = *reinterpret_cast<const float4*>(xs + c * g.dpad + xo + 4 * hf);
        xv[c][0] = t.x; xv[c][1] = t.y; xv[c][2] = t.z; xv[c][3] = t.w;
      }
#pragma unroll
      for (int r = 0; r < kGemvRows; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const unsigned word = w[r][2 * hf + (e >> 1)];
          const float wf = (e & 1) ? bf16_hi(word) : bf16_lo(word);
#pragma unroll
          for (int c = 0; c < kCols; ++c) acc[r][c] = fmaf(wf, xv[c][e], acc[r][c]);
        }
    }
  };
  // the 32 sums of a row group over the wavefront; lanes 2i and 2i+1 end with sum i
  // (row i / 4, column i % 4)
  auto reduce = [&](float (&acc)[kGemvRows][kCols]) __attribute__((always_inline)) -> float {
    float v[kGemvRows * kCols];
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r)
#pragma unroll
      for (int c = 0; c < kCols; ++c) {
        v[r * kCols + c] = acc[r][c];
        acc[r][c] = 0.f;
      }
#pragma unroll
    for (int st = 0; st < 5; ++st) {
      const int half = 16 >> st, mask = 32 >> st;
      // all ones in the upper lane of each pair; the selects are bit operations so that
      // they stay selects between two registers
      const unsigned up = (lane & mask) ? ~0u : 0u;
#pragma unroll
      for (int i = 0; i < half; ++i) {
        const unsigned a = __float_as_uint(v[i]), b = __float_as_uint(v[i + half]);
        const float keep = __uint_as_float((a & ~up) | (b & up));
        const float send = __uint_as_float((b & ~up) | (a & up));
        v[i] = keep + __shfl_xor(send, mask, 64);
      }
    }
    return v[0] + __shfl_xor(v[0], 1, 64);
  };
  // this block's outputs [kCols][rows], written out at the end (so that the status word is
  // needed only there)
  float* blk = xs + kCols * g.dpad;
  auto store = [&](int base, float total) __attribute__((always_inline)) {
    const int idx = lane >> 1, r = idx >> 2, c = idx & 3;
    const int row = base + r;
    if ((lane & 1) == 0 && row < r1 && c < g.ncols) {
      float v = total;
      if (kResidual) {
        const float x = xs[c * g.dpad + row];  // the residual input h (R = d)
        v = v / (1.0f + expf(-v)) + x;         // SiLU(W1 h) + h
      }
      blk[c * g.rows_per_block + (row - r0)] = v;
    }
  };

  float acc[kGemvRows][kCols];
#pragma unroll
  for (int r = 0; r < kGemvRows; ++r)
#pragma unroll
    for (int c = 0; c < kCols; ++c) acc[r][c] = 0.f;
  float held = 0.f;  // split row groups: this wavefront's partial sum
  u32x4 wa[kGemvRows], wb[kGemvRows];
  int lbase = first, lj = 0;  // the next step to load
  int cbase = first, cj = 0;  // the step being computed
  auto advance = [&](int& base, int& j) __attribute__((always_inline)) {
    if (++j == my_nch) {
      j = 0;
      base += stride;
    }
  };
  auto finish_step = [&]() __attribute__((always_inline)) {
    if (cj + 1 == my_nch) {
      const float total = reduce(acc);
      if (g.split == 1) store(cbase, total);
      else held = total;
    }
    advance(cbase, cj);
  };
  // The loads of the next step are issued before the current step's FMAs.  Every path
  // into the loop head has exactly one step's loads in flight (into wa): the loop runs
  // whole pairs of steps, the odd last step follows it, and a prefetch with no next step
  // re-reads the current step's pieces (still in L2), so the waits before the FMAs always
  // leave the prefetched loads outstanding.
  // the first batch of input pieces, then the first step's weights: the waits for the
  // (older) input loads leave the weight loads in flight while the columns are staged
  // (a wavefront without rows loads the block's first row and never uses it, so that the
  // count of loads in flight is the same on every path)
  fill_issue(tid);
  __builtin_amdgcn_sched_barrier(0);
  load(steps > 0 ? lbase : r0, 0, wa);
  if (steps > 0) advance(lbase, lj);
  fill_store();
  for (int p0 = tid + kFill * kGemvThreads; p0 < kCols * np; p0 += kFill * kGemvThreads) {
    fill_issue(p0);  // inputs wider than one batch (fp32 columns above 4096)
    fill_store();
  }
  __syncthreads();
  for (int t = 0; t + 1 < steps; t += 2) {
    load(lbase, lj, wb);  // step t + 1 exists
    advance(lbase, lj);
    fma_step(cj, wa, acc);
    finish_step();
    const bool more = t + 2 < steps;
    load(more ? lbase : cbase, more ? lj : cj, wa);
    if (more) advance(lbase, lj);
    fma_step(cj, wb, acc);
    finish_step();
  }
  if (steps & 1) {
    fma_step(cj, wa, acc);
    finish_step();
  }
  if (g.split > 1) {  // one row group per wavefront: add the parts of each slot
    if ((lane & 1) == 0) part[wave][lane >> 1] = held;
    __syncthreads();
    if (pid == 0 && ngroups > 0) {
      float total = part[wave][lane >> 1];
      for (int p = 1; p < g.split; ++p) total += part[wave + p][lane >> 1];
      store(first, total);
    }
  }
  __syncthreads();  // every output of the block is in blk
  const bool failed = round_failed(g.status);  // gates the output stores only
  if (!failed && g.out) {  // coalesced: consecutive threads write consecutive rows
    const int n = r1 - r0;
    for (int i = tid; i < g.ncols * g.rows_per_block; i += kGemvThreads) {
      const int c = i / g.rows_per_block, r = i - c * g.rows_per_block;
      if (r < n) g.out[(int64_t(k) * g.B + g.col0 + c) * g.R + r0 + r] = blk[i];
    }
  }
  if (!kResidual) {
    // The block's best topk rows of every column, best first, as ranking keys (key 0 past
    // the block's rows): one wavefront per column, the keys in registers (at most
    // kBlockRows / 64 per lane), rounds without barriers.
    if (wave < g.ncols) {
      const int c = wave, n = r1 - r0;
      uint64_t key[kBlockRows / 64];
      bool nan = false;
#pragma unroll
      for (int q = 0; q < kBlockRows / 64; ++q) {
        const int i = lane + 64 * q;
        const float v = blk[c * g.rows_per_block + (i < n ? i : 0)];
        nan = nan || (i < n && v != v);
        key[q] = i < n && v == v ? rank_key(v, r0 + i) : 0;
      }
      uint64_t* out = g.keys + ((int64_t(k) * g.B + g.col0 + c) * g.nblk + blockIdx.x) * g.topk;
      if (__ballot(nan)) {
        if (lane == 0) raise_status(g.status, MEDUSA_EINVAL);
        for (int r = lane; r < g.topk; r += 64) out[r] = kNanList;
      } else {
        uint64_t prev = ~uint64_t(0);  // keys below prev remain
        for (int r = 0; r < g.topk; ++r) {
          uint64_t best = 0;
#pragma unroll
          for (int q = 0; q < kBlockRows / 64; ++q)
            if (key[q] < prev) best = max_u64(best, key[q]);
          best = wave_max_key(best);
          if (lane == 0) out[r] = best;
          prev = best;
        }
      }
    }
  }
}


// One workgroup per (head, sequence) merges the row blocks' lists into candidate
// slots 1 + head topk + r, and head 0's workgroups write the root token into slot 0.  Up to
// kMergeCache keys per thread are held in registers; longer lists are re-read each round.
template <bool kCached>
__global__ __launch_bounds__(kMergeThreads) void head_topk_merge_kernel(TopkArgs a) {
  __shared__ uint64_t slot[2][kMergeThreads / 64];
  const bool failed = round_failed(a.status);  // gates the stores only
  const int kb = blockIdx.x, k = kb / a.B, b = kb - k * a.B;
  const int tid = threadIdx.x;
  const int n = a.S * a.topk;
  const uint64_t* keys = a.seg_keys + int64_t(kb) * n;
  uint64_t kc[kCached ? kMergeCache : 1];
  bool nan = false;
  if (kCached) {
#pragma unroll
    for (int q = 0; q < kMergeCache; ++q) kc[q] = keys[min(tid + q * kMergeThreads, n - 1)];
#pragma unroll
    for (int q = 0; q < kMergeCache; ++q) {
      if (tid + q * kMergeThreads >= n) kc[q] = 0;
      nan = nan || (kc[q] == kNanList);
    }
  } else {
    for (int i = tid; i < n; i += kMergeThreads) nan = nan || (keys[i] == kNanList);
  }
  if (__syncthreads_or(nan)) {
    if (tid == 0) raise_status(a.status, MEDUSA_EINVAL);
    return;
  }
  int32_t* cand = a.candidates + int64_t(b) * (1 + a.K * a.topk);
  uint64_t prev = ~uint64_t(0);
  for (int r = 0; r < a.topk; ++r) {
    uint64_t best = 0;
    if (kCached) {
#pragma unroll
      for (int q = 0; q < kMergeCache; ++q)
        if (kc[q] < prev) best = max_u64(best, kc[q]);
    } else {
      for (int i = tid; i < n; i += kMergeThreads) {
        const uint64_t key = keys[i];
        if (key < prev) best = max_u64(best, key);
      }
    }
    best = block_max_key<kMergeThreads>(best, slot, r);
    if (tid == 0 && !failed) cand[1 + k * a.topk + r] = key_index(best);
    prev = best;
  }
  if (tid == 0 && k == 0 && !failed) cand[0] = a.root[b];
}

// Launch shape of one GEMV over R rows: row groups of 8; with fewer groups than half the
// wavefront slots of the chip, 2..8 wavefronts share a group (each taking every split-th
// column of pieces), one group per wavefront; otherwise about per_cu workgroups per compute
// unit and head, each over a contiguous row range (at most max_rows rows, a multiple of 64).
// Long streams per wavefront beat full occupancy here: the residual product at hidden 4096
// (2048 groups) runs 30 us with one wavefront of 8 steps per group against 36 us with two
// wavefronts of 4 steps each.
struct GemvShape {
  int32_t split, rows_per_block, blocks;
};

GemvShape gemv_shape(int32_t R, int32_t K, int32_t dpad, int32_t per_cu, int32_t max_rows) {
  GemvShape sh{};
  const int64_t groups = int64_t(K) * ((R + kGemvRows - 1) / kGemvRows);
  const int32_t nch = dpad / kPad;
  sh.split = 1;
  while (sh.split < kGemvWaves && sh.split * 2 <= nch && groups * sh.split < kSplitBelow) sh.split *= 2;
  if (sh.split > 1) {
    sh.rows_per_block = (kGemvWaves / sh.split) * kGemvRows;
  } else {
    const int64_t blocks = (int64_t(256) * per_cu + K - 1) / K;  // per head
    const int64_t rows = (R + blocks - 1) / blocks;
    const int64_t unit = int64_t(kGemvWaves) * kGemvRows;
    sh.rows_per_block = int32_t(std::min<int64_t>((rows + unit - 1) / unit * unit, max_rows));
  }
  sh.blocks = (R + sh.rows_per_block - 1) / sh.rows_per_block;
  return sh;
}

int32_t dpad_of(int32_t d) { return (d + kPad - 1) / kPad * kPad; }

// dynamic LDS of the two GEMV kernels: the input columns and the block's staged outputs
size_t lds_residual(int32_t dpad) { return size_t(kCols) * (dpad + kBlockRows) * sizeof(float); }
size_t lds_unembed(int32_t dpad) { return size_t(kCols) * (dpad + kBlockRows) * sizeof(float); }
int32_t resident(size_t lds) { return (160 * 1024) / (lds + 1024) >= 2 ? 2 : 1; }

GemvShape unembed_shape(int32_t K, int32_t d, int32_t V) {
  const int32_t dpad = dpad_of(d);
  return gemv_shape(V, K, dpad, resident(lds_unembed(dpad)), kBlockRows);
}

struct HeadPlan {
  size_t u_offset, keys_offset, bytes;
  int32_t nblk;
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// the ranked lists are sized for the largest topk, so the size depends on the shapes only
HeadPlan head_plan(int32_t B, int32_t K, int32_t d, int32_t V) {
  HeadPlan p{};
  p.nblk = unembed_shape(K, d, V).blocks;
  const size_t lists = size_t(K) * B * p.nblk * kMaxTopk;
  p.u_offset = 0;
  p.keys_offset = align256(size_t(K) * B * d * sizeof(float));
  p.bytes = p.keys_offset + align256(lists * sizeof(uint64_t));
  return p;
}

}  // namespace
}  // namespace medusa

using namespace medusa;

extern "C" size_t medusa_head_workspace_size(int32_t B, int32_t K, int32_t d, int32_t V) {
  if (B < 1 || K < 1 || d < 1 || V < 1) return 0;
  return head_plan(B, K, d, V).bytes;
}

extern "C" medusa_status medusa_head_candidates(void* stream, int32_t B, int32_t K, int32_t d, int32_t V,
                                                int32_t topk, const void* h, const void* W1, const void* W2,
                                                const int32_t* d_root_tokens, int32_t* candidates,
                                                float* head_logits, void* workspace, size_t workspace_bytes,
                                                int32_t* d_status, void* ev_start, void* ev_stop) {
  if (B < 1 || K < 1 || d < 8 || V < 1 || topk < 1) return MEDUSA_EINVAL;
  if (!h || !W1 || !W2 || !d_root_tokens || !candidates || !d_status) return MEDUSA_EINVAL;
  if (d % 8 != 0 || d > kMaxD || topk > kMaxTopk || topk > V) return MEDUSA_EUNSUPPORTED;
  // every buffer the kernels address through a buffer resource spans less than 4 GiB
  constexpr int64_t kMaxBytes = int64_t(0xFFFFFFF0);
  if (int64_t(V) * d * 2 > kMaxBytes || int64_t(B) * d * 4 > kMaxBytes) return MEDUSA_EUNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(h) | reinterpret_cast<uintptr_t>(W1) | reinterpret_cast<uintptr_t>(W2)) & 15)
    return MEDUSA_EINVAL;
  const HeadPlan plan = head_plan(B, K, d, V);
  if (workspace == nullptr || workspace_bytes < plan.bytes) return MEDUSA_EBUFSIZE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  float* u = reinterpret_cast<float*>(ws + plan.u_offset);
  uint64_t* keys = reinterpret_cast<uint64_t*>(ws + plan.keys_offset);
  const int32_t dpad = dpad_of(d);
  const size_t lds_r = lds_residual(dpad), lds_u = lds_unembed(dpad);
  // beyond the default dynamic LDS of a launch
  if (lds_r > 60 * 1024 &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(&head_gemv_kernel<true>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, int(lds_r)) != hipSuccess)
    return MEDUSA_EHIP;
  if (lds_u > 60 * 1024 &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(&head_gemv_kernel<false>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, int(lds_u)) != hipSuccess)
    return MEDUSA_EHIP;
  const GemvShape sh_r = gemv_shape(d, K, dpad, resident(lds_r), kBlockRows);
  const GemvShape sh_u = unembed_shape(K, d, V);
  auto gemv = [&](bool residual, int32_t col0, void* e0, void* e1) -> medusa_status {
    const GemvShape& sh = residual ? sh_r : sh_u;
    GemvArgs g{};
    g.W = static_cast<const bf16*>(residual ? W1 : W2);
    g.x_bf16 = static_cast<const bf16*>(h);
    g.x_f32 = u;
    g.out = residual ? u : head_logits;
    g.status = d_status;
    g.keys = keys;
    g.B = B;
    g.d = d;
    g.dpad = dpad;
    g.R = residual ? d : V;
    g.col0 = col0;
    g.ncols = B - col0 < kCols ? B - col0 : kCols;
    g.rows_per_block = sh.rows_per_block;
    g.split = sh.split;
    g.topk = topk;
    g.nblk = sh.blocks;
    const void* kern = residual ? reinterpret_cast<const void*>(&head_gemv_kernel<true>)
                                : reinterpret_cast<const void*>(&head_gemv_kernel<false>);
    return launch(kern, dim3(unsigned(sh.blocks), unsigned(K)), dim3(kGemvThreads), residual ? lds_r : lds_u, s,
                  g, e0, e1);
  };
  for (int32_t c0 = 0; c0 < B; c0 += kCols) {
    medusa_status st = gemv(true, c0, c0 == 0 ? ev_start : nullptr, nullptr);
    if (st != MEDUSA_OK) return st;
  }
  for (int32_t c0 = 0; c0 < B; c0 += kCols) {
    medusa_status st = gemv(false, c0, nullptr, nullptr);
    if (st != MEDUSA_OK) return st;
  }
  TopkArgs t{};
  t.root = d_root_tokens;
  t.candidates = candidates;
  t.status = d_status;
  t.seg_keys = keys;
  t.B = B;
  t.K = K;
  t.V = V;
  t.topk = topk;
  t.S = plan.nblk;
  const void* merge = int64_t(plan.nblk) * topk <= int64_t(kMergeThreads) * kMergeCache
                          ? reinterpret_cast<const void*>(&head_topk_merge_kernel<true>)
                          : reinterpret_cast<const void*>(&head_topk_merge_kernel<false>);
  return launch(merge, dim3(unsigned(int64_t(K) * B)), dim3(kMergeThreads), 0, s, t, nullptr, ev_stop);
}
