// Tree attention for one layer: RoPE at P + depth, staged K/V rows, and the
// attention of every tree row over the committed cache plus its ancestors.
//
// [M7.2] = "M7.2 - Medusa: Multi-Head Candidates, Tree Attention, and Verification"
//   §0x03A: position(u) = P + depth(u); siblings share a RoPE phase.
//   §0x03C: N query rows against P + N key rows; every prefix row visible,
//           staged row u stored at cache row P + u, visible to w iff the tree
//           mask says u is an ancestor of w or w itself.
// [Chai] = "Medusa 完全拆解：多头树式候选如何用一次验证解码多个 Token", section
//   "Tree Attention：把一棵树压进一次并行前向": softmax(QK^T/sqrt(d_h) + M)V with
//   M = 0 / -inf; each node sees the context, its ancestors and itself.
//
// Two device paths:
//  * stage + rowwise (this file): one wavefront per query row, fp32 math.
//    Handles every supported shape and is the fp32 path.
//  * the MFMA path (attn_mfma.hip) for bf16, d_h = 128 and 64 (the latter padded
//    to the 128-wide layout): GQA query blocks against the streamed cache on
//    matrix cores.

#include <cmath>

#include "attn_common.h"
#include "common.h"

namespace medusa {

// Stage the N new K/V rows of every sequence and kv head: K rotated to
// P + depth(u) (angles and rotation in binary64, stored in the cache dtype),
// V copied.  Grid (N, B); every block checks every prefix length first so that
// either all blocks store or none does.
template <typename T, int D>
__global__ __launch_bounds__(256) void stage_kv_kernel(AttnArgs a) {
  if (round_failed(a.status)) return;
  if (!prefixes_fit(a)) {
    if (threadIdx.x == 0 && blockIdx.x == 0 && blockIdx.y == 0) raise_status(a.status, MEDUSA_ECAPACITY);
    return;
  }
  const int u = blockIdx.x, b = blockIdx.y;
  const int P = a.prefix_len[b];
  const double pos = double(P + a.depth[u]);
  __shared__ double cs[D / 2], sn[D / 2];
  for (int i = threadIdx.x; i < D / 2; i += blockDim.x) {
    const double ang = pos * pow(a.rope_base, -2.0 * i / D);
    sincos(ang, &sn[i], &cs[i]);
  }
  __syncthreads();
  const T* kn = static_cast<const T*>(a.k_new) + (int64_t(b) * a.N + u) * a.Hkv * D;
  const T* vn = static_cast<const T*>(a.v_new) + (int64_t(b) * a.N + u) * a.Hkv * D;
  for (int idx = threadIdx.x; idx < a.Hkv * (D / 2); idx += blockDim.x) {
    const int g = idx / (D / 2), i = idx % (D / 2);
    const int64_t row = ((int64_t(b) * a.Hkv + g) * a.S_max + P + u) * D;
    const double x1 = to_f32(kn[g * D + i]), x2 = to_f32(kn[g * D + i + D / 2]);
    T* kr = static_cast<T*>(a.k_cache) + row;
    kr[i] = from_f32<T>(float(x1 * cs[i] - x2 * sn[i]));
    kr[i + D / 2] = from_f32<T>(float(x2 * cs[i] + x1 * sn[i]));
    T* vr = static_cast<T*>(a.v_cache) + row;
    vr[i] = vn[g * D + i];
    vr[i + D / 2] = vn[g * D + i + D / 2];
  }
}

template <typename T, int D>
__device__ __forceinline__ float dot_row(const float* q, const T* k) {
  constexpr int E = 16 / sizeof(T);
  float s = 0.f;
#pragma unroll 4
  for (int i = 0; i < D; i += E) {
    const uint4 raw = *reinterpret_cast<const uint4*>(k + i);
    const T* e = reinterpret_cast<const T*>(&raw);
#pragma unroll
    for (int j = 0; j < E; ++j) s += q[i + j] * to_f32(e[j]);
  }
  return s;
}

// One wavefront per query row (b, u, h): lanes take 64 keys at a time for the
// scores and the output dimensions for P.V, with an online softmax.  Reads the
// staged rows the stage kernel wrote.  Four rows per block.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_rowwise_kernel(AttnArgs a) {
  if (round_failed(a.status)) return;
  if (!prefixes_fit(a)) return;  // the stage kernel already raised the status
  constexpr int DL = D / 64;     // output dims per lane
  __shared__ float qs[4][D];
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int64_t rows = int64_t(a.B) * a.N * a.Hq;
  const int64_t row = int64_t(blockIdx.x) * 4 + wave;
  const bool live = row < rows;
  const int h = live ? int(row % a.Hq) : 0;
  const int u = live ? int((row / a.Hq) % a.N) : 0;
  const int b = live ? int(row / (int64_t(a.Hq) * a.N)) : 0;
  const int g = h / (a.Hq / a.Hkv);
  const int P = a.prefix_len[b];
  const double pos = double(P + a.depth[u]);
  const float scale = 1.0f / sqrtf(float(D));

  const T* qrow = static_cast<const T*>(a.q) + ((int64_t(b) * a.N + u) * a.Hq + h) * D;
#pragma unroll
  for (int t = 0; t < DL; ++t) {
    const int i = lane + 64 * t;
    const int j = i % (D / 2);
    const int partner = i < D / 2 ? i + D / 2 : i - D / 2;
    double sn, cs;
    sincos(pos * pow(a.rope_base, -2.0 * j / D), &sn, &cs);
    const double x = to_f32(qrow[i]), y = to_f32(qrow[partner]);
    const double r = i < D / 2 ? x * cs - y * sn : x * cs + y * sn;
    qs[wave][i] = float(r) * scale;
  }
  __syncthreads();

  const int64_t head = (int64_t(b) * a.Hkv + g) * a.S_max;
  const T* kc = static_cast<const T*>(a.k_cache) + head * D;
  const T* vc = static_cast<const T*>(a.v_cache) + head * D;
  const uint64_t* mrow = a.mask + int64_t(u) * a.mask_words;
  float m = -INFINITY, l = 0.f, acc[DL];
#pragma unroll
  for (int t = 0; t < DL; ++t) acc[t] = 0.f;

  // keys [0, P) are the committed prefix; [P, P + N) the staged rows under the mask
  const int total = P + a.N;
  for (int k0 = 0; k0 < total; k0 += 64) {
    const int k = k0 + lane;
    float s = -INFINITY;
    bool visible = k < P;
    if (!visible && k < total) {
      const int v = k - P;
      visible = (mrow[v / 64] >> (v % 64)) & 1u;
    }
    if (visible) s = dot_row<T, D>(qs[wave], kc + int64_t(k) * D);
    const float cmax = wave_max(s);
    if (cmax == -INFINITY) continue;
    const float m_new = fmaxf(m, cmax);
    const float corr = __expf(m - m_new);
    const float p = visible ? __expf(s - m_new) : 0.f;
    l = l * corr + wave_sum(p);
#pragma unroll
    for (int t = 0; t < DL; ++t) acc[t] *= corr;
    const int nk = min(64, total - k0);
    for (int j = 0; j < nk; ++j) {
      const float pj = __shfl(p, j, 64);
      if (pj == 0.f) continue;
      const T* vr = vc + int64_t(k0 + j) * D;
#pragma unroll
      for (int t = 0; t < DL; ++t) acc[t] += pj * to_f32(vr[lane + 64 * t]);
    }
    m = m_new;
  }
  if (!live) return;
  T* orow = static_cast<T*>(a.out) + ((int64_t(b) * a.N + u) * a.Hq + h) * D;
  const float inv = 1.0f / l;
#pragma unroll
  for (int t = 0; t < DL; ++t) orow[lane + 64 * t] = from_f32<T>(acc[t] * inv);
}

template <typename T, int D>
medusa_status run_rowwise(AttnArgs& a, hipStream_t stream, void* ev_start, void* ev_stop) {
  medusa_status st = launch(reinterpret_cast<const void*>(&stage_kv_kernel<T, D>),
                            dim3(a.N, a.B), dim3(256), 0, stream, a, ev_start, nullptr);
  if (st != MEDUSA_OK) return st;
  const int64_t rows = int64_t(a.B) * a.N * a.Hq;
  return launch(reinterpret_cast<const void*>(&attn_rowwise_kernel<T, D>),
                dim3(unsigned((rows + 3) / 4)), dim3(256), 0, stream, a, nullptr, ev_stop);
}

}  // namespace medusa

using namespace medusa;

extern "C" size_t medusa_tree_attn_workspace_size(medusa_dtype dt, int32_t B, int32_t Hq,
                                                  int32_t Hkv, int32_t d_h, int32_t N,
                                                  int32_t S_max) {
  return attn_workspace_bytes(dt, B, Hq, Hkv, d_h, N, S_max);
}

extern "C" medusa_status medusa_tree_attn(void* stream, medusa_dtype dt, int32_t B, int32_t Hq,
                                          int32_t Hkv, int32_t d_h, int32_t N,
                                          const int32_t* d_depth, const uint64_t* d_tree_mask,
                                          int32_t mask_words, const int32_t* d_prefix_len,
                                          const void* q, const void* k_new, const void* v_new,
                                          void* k_cache, void* v_cache, int32_t S_max,
                                          double rope_base, void* out, void* workspace,
                                          size_t workspace_bytes, int32_t* d_status,
                                          void* ev_start, void* ev_stop) {
  if (dt != MEDUSA_F32 && dt != MEDUSA_BF16) return MEDUSA_EINVAL;
  if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || S_max < N || mask_words < 1) return MEDUSA_EINVAL;
  if (Hq % Hkv != 0) return MEDUSA_EINVAL;
  if (int64_t(N) > int64_t(64) * mask_words) return MEDUSA_EINVAL;
  if (!(rope_base > 0.0) || !std::isfinite(rope_base)) return MEDUSA_EINVAL;
  if (d_h != 64 && d_h != 128) return MEDUSA_EUNSUPPORTED;
  if (!d_depth || !d_tree_mask || !d_prefix_len || !q || !k_new || !v_new || !k_cache ||
      !v_cache || !out || !d_status)
    return MEDUSA_EINVAL;
  const size_t need = attn_workspace_bytes(dt, B, Hq, Hkv, d_h, N, S_max);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return MEDUSA_EBUFSIZE;

  AttnArgs a{};
  a.depth = d_depth;
  a.mask = d_tree_mask;
  a.prefix_len = d_prefix_len;
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.out = out;
  a.status = d_status;
  a.workspace = workspace;
  a.rope_base = rope_base;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.N = N;
  a.mask_words = mask_words;
  a.S_max = S_max;
  hipStream_t s = static_cast<hipStream_t>(stream);

  if (mfma_path_applies(dt, Hq, Hkv, d_h, N)) return run_mfma(a, d_h, s, ev_start, ev_stop);
  if (dt == MEDUSA_F32)
    return d_h == 64 ? run_rowwise<float, 64>(a, s, ev_start, ev_stop)
                     : run_rowwise<float, 128>(a, s, ev_start, ev_stop);
  return d_h == 64 ? run_rowwise<bf16, 64>(a, s, ev_start, ev_stop)
                   : run_rowwise<bf16, 128>(a, s, ev_start, ev_stop);
}
