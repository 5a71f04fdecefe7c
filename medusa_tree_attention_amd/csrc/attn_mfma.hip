// Matrix-core tree attention for bf16, d_h = 128 (gfx950).
//
// What is computed is the tree attention of [M7.2] = "M7.2 - Medusa: Multi-Head
// Candidates, Tree Attention, and Verification", §0x03A/§0x03C (position
// P + depth; N query rows against the P committed rows and the N staged rows,
// staged row u stored at cache row P + u and visible to w iff u is an ancestor
// of w or w itself) -- the same contract as the wavefront-per-row path.
//
// Mapping to CDNA4:
//  * One (sequence b, kv head g) pair owns a query block of N * (Hq/Hkv) rows:
//    every tree node times every query head of the GQA group.  That block
//    against a key tile is a dense contraction, so both products run on
//    v_mfma_f32_32x32x16_bf16.
//  * A workgroup takes 64 query rows (a q-tile) and one contiguous split of
//    the committed prefix.  Its four wavefronts hold the same 64 rotated,
//    pre-scaled query rows in registers and take interleaved 32-key tiles of
//    the split; the last split also takes the staged rows.  The q-tiles of
//    one split are launched onto one XCD (block id modulo 8) so that their
//    identical KV stream is served once from that XCD's L2.
//  * Scores are formed transposed, S^T = K Q^T (K rows are the A operand, read
//    from LDS with 16-byte reads), so the probability tile comes out of the
//    accumulator already in the B-operand layout of O^T = V^T P^T; V^T is read
//    from LDS with the transposing ds_read_b64_tr_b16.  No shuffle of P.
//  * Online softmax in log2 units; the running maximum only moves when a tile
//    exceeds it by more than 2^8, so the O rescale is almost never paid.
//  * Staged keys are rotated to P + depth(u) in registers (binary64 phase
//    angles kept as fp32 cos/sin in LDS), written to cache rows P + u, and
//    masked per lane with the packed ancestor bitmask.
//  * The four wavefronts' (m, l, O) are merged through LDS; splits are merged
//    by the last workgroup to finish (atomic arrival counter in the workspace,
//    reset by that workgroup), so one launch does the whole call.

#include <cmath>

#include "attn_common.h"

namespace medusa {
namespace {

constexpr int kD = 128;          // head dimension
constexpr int kRowsWG = 64;      // query rows per workgroup
constexpr int kTile = 32;        // keys per tile
constexpr int kWaves = 4;
constexpr int kTableDepth = 32;  // RoPE phases kept in LDS; deeper trees are rejected
constexpr int kTargetWGs = 256;  // one workgroup per compute unit
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;  // log2 units

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

struct MfmaArgs {
  AttnArgs a;
  int32_t group;           // Hq / Hkv
  int32_t rows;            // N * group query rows per (sequence, kv head)
  int32_t qtiles;          // ceil(rows / 64)
  int32_t splits;          // workgroups sharing one q-tile's keys
  int32_t xcd_map;         // keep the q-tiles of one (unit, split) on one XCD
  int32_t partial_offset;  // byte offset of the split partials in the workspace
  double theta[kD / 2];    // RoPE inverse frequencies base^(-2i/d)
};

struct Partial {
  float m[kRowsWG];
  float l[kRowsWG];
  float o[kRowsWG][kD];
};

struct Plan {
  int32_t units, group, rows, qtiles, splits;
  bool xcd_map;
  size_t partial_offset, bytes;
};

Plan make_plan(int32_t B, int32_t Hq, int32_t Hkv, int32_t N, int32_t S_max) {
  Plan p{};
  p.units = B * Hkv;
  p.group = Hq / Hkv;
  p.rows = N * p.group;
  p.qtiles = (p.rows + kRowsWG - 1) / kRowsWG;
  const int32_t wgs = p.units * p.qtiles;
  int32_t splits = (kTargetWGs + wgs / 2) / wgs;
  const int32_t max_splits = (S_max - N) / 256;  // at least ~256 prefix keys per split
  splits = splits < max_splits ? splits : max_splits;
  p.splits = splits < 1 ? 1 : splits;
  p.xcd_map = (int64_t(p.units) * p.splits) % 8 == 0;
  p.partial_offset = (size_t(p.units) * p.qtiles * sizeof(int32_t) + 255) / 256 * 256;
  p.bytes = p.partial_offset +
            (p.splits > 1 ? size_t(p.units) * p.qtiles * p.splits * sizeof(Partial) : 0);
  return p;
}

// byte offset of (row, 16-byte chunk) in a 32 x 256-byte tile; chunks are
// XOR-swizzled by row so that column reads spread over the LDS banks
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 256 + ((chunk ^ (row & 15)) << 4);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// 32-bit LDS address of a __shared__ pointer, made wave-uniform
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      uint32_t(size_t((__attribute__((address_space(3))) const void*)(p))));
}

// Direct global -> LDS load of 16 bytes per lane: lane l's bytes land at lds + 16 l.
// Issued as inline assembly so that the compiler does not pair it with a full
// vmcnt(0) drain before every LDS read; the tile pipeline waits with explicit,
// in-order vmcnt counts instead (an extra load issued later only lengthens a wait).
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds), "v"(g)
               : "memory", "m0");
}
__device__ __forceinline__ void wait_vm16() { asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); }
__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__global__ __launch_bounds__(256, 1) void tree_attn_mfma_kernel(MfmaArgs p) {
  const AttnArgs& a = p.a;
  if (round_failed(a.status)) return;
  if (!prefixes_fit(a)) {
    if (blockIdx.x == 0 && threadIdx.x == 0) raise_status(a.status, MEDUSA_ECAPACITY);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int half = lane >> 5, l32 = lane & 31;

  // ---- this workgroup's (sequence, kv head, split, q-tile)
  int grp, qt;
  if (p.xcd_map) {
    const int slot = blockIdx.x >> 3;
    grp = int(blockIdx.x & 7) + 8 * (slot / p.qtiles);
    qt = slot % p.qtiles;
  } else {
    grp = blockIdx.x / p.qtiles;
    qt = blockIdx.x % p.qtiles;
  }
  const int unit = grp / p.splits, split = grp % p.splits;
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int P = a.prefix_len[b];
  const int N = a.N;

  __shared__ float2 s_cs[kTableDepth][kD / 2];
  // two tile buffers per wave (K 8 KiB + V 8 KiB each); the final merge reuses them
  __shared__ __attribute__((aligned(16))) unsigned char s_tile0[kWaves][16384];
  __shared__ __attribute__((aligned(16))) unsigned char s_tile1[kWaves][16384];
  __shared__ int s_int;

  // ---- RoPE phases (cos, sin) of positions P + d for every depth d of the tree
  if (tid == 0) s_int = 0;
  __syncthreads();
  int dmax = 0;
  for (int i = tid; i < N; i += 256) dmax = max(dmax, a.depth[i]);
  atomicMax(&s_int, dmax);
  __syncthreads();
  dmax = s_int;
  if (dmax >= kTableDepth) {  // uniform: every block sees the same tree
    if (blockIdx.x == 0 && tid == 0) raise_status(a.status, MEDUSA_EUNSUPPORTED);
    return;
  }
  for (int i = tid; i < (dmax + 1) * (kD / 2); i += 256) {
    const int d = i / (kD / 2), j = i % (kD / 2);
    double sn, cs;
    sincos(double(P + d) * p.theta[j], &sn, &cs);
    s_cs[d][j] = make_float2(float(cs), float(sn));
  }
  __syncthreads();

  // ---- query rows of this q-tile: rotated, scaled to log2 units, bf16 B operands
  // lane holds query column l32 of column block c, dims 16 s + 8 half + e (e < 8)
  const float qscale = kLog2e / sqrtf(float(kD));
  bf16x8 qop[2][8];
  int qnode[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int r = qt * kRowsWG + c * 32 + l32;
    const bool live = r < p.rows;
    const int u = live ? r / p.group : 0;
    const int h = kvh * p.group + (live ? r % p.group : 0);
    qnode[c] = min(r / p.group, N - 1);
    const bf16* qr = static_cast<const bf16*>(a.q) + ((int64_t(b) * N + u) * a.Hq + h) * kD;
    float x[8][8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint4 raw = live ? *reinterpret_cast<const uint4*>(qr + 16 * s + 8 * half)
                             : make_uint4(0, 0, 0, 0);
      const bf16x8 v = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[s][e] = float(v[e]);
    }
    const int dep = a.depth[u];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 cs = s_cs[dep][16 * s + 8 * half + e];
        const float x1 = x[s][e], x2 = x[s + 4][e];
        x[s][e] = x1 * cs.x - x2 * cs.y;
        x[s + 4][e] = x2 * cs.x + x1 * cs.y;
      }
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) qop[c][s][e] = static_cast<bf16>(x[s][e] * qscale);
    }
  }

  // ---- key range: split `split` of the committed prefix, plus the staged rows in the last split
  const int per = ((P + p.splits - 1) / p.splits + kTile - 1) / kTile * kTile;
  const int k_lo = min(P, split * per), k_hi = min(P, k_lo + per);
  const int n_pre = (k_hi - k_lo + kTile - 1) / kTile;
  const int n_stg = (split == p.splits - 1) ? (N + kTile - 1) / kTile : 0;
  const int n_tiles = n_pre + n_stg;
  const int steps = (n_tiles + kWaves - 1) / kWaves;

  const int64_t head = (int64_t(b) * a.Hkv + kvh) * a.S_max * kD;
  const bf16* kc = static_cast<const bf16*>(a.k_cache) + head;
  const bf16* vc = static_cast<const bf16*>(a.v_cache) + head;
  bf16* kc_w = static_cast<bf16*>(a.k_cache) + head;
  bf16* vc_w = static_cast<bf16*>(a.v_cache) + head;
  const bf16* kn = static_cast<const bf16*>(a.k_new);
  const bf16* vn = static_cast<const bf16*>(a.v_new);

  // Tile t lands in one of this wave's LDS buffers by direct global->LDS loads: instruction
  // i moves rows 4 i .. 4 i + 3 (1 KiB, lane l -> bytes 16 l); lane l fetches logical chunk
  // (l % 16) ^ (row % 16) so that the buffer holds the swizzled layout swz() reads.
  auto issue_tile = [&](int t, unsigned char* buf) -> bool {
    if (t >= n_tiles) return false;
    const uint32_t base = lds_addr(buf);
    const bool staged = t >= n_pre;
    const int k0 = staged ? (t - n_pre) * kTile : k_lo + t * kTile;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rt = 4 * i + (lane >> 4);
      const int c = (lane & 15) ^ (rt & 15);
      const bf16 *ks, *vs;
      if (staged) {
        const int u = k0 + rt < N ? k0 + rt : 0;
        const int64_t src = ((int64_t(b) * N + u) * a.Hkv + kvh) * kD;
        ks = kn + src;
        vs = vn + src;
      } else {
        const int row = k0 + rt < k_hi ? k0 + rt : k0;
        ks = kc + int64_t(row) * kD;
        vs = vc + int64_t(row) * kD;
      }
      dma16(ks + 8 * c, base + 1024 * i);
      dma16(vs + 8 * c, base + 8192 + 1024 * i);
    }
    return true;
  };
  // Staged rows: rotate K in place to P + depth(u); q-tile 0 also stores K~ and V to cache
  // rows P + u.  In each row every lane reads its chunk and the partner chunk (dims -+ 64)
  // before any lane of the wave writes.
  auto rotate_staged = [&](int t, unsigned char* buf) {
    const int v0 = (t - n_pre) * kTile;
    const int c = lane & 15;
    for (int i = 0; i < 8; ++i) {
      const int rt = 4 * i + (lane >> 4);
      const int uu = v0 + rt;
      const int u = uu < N ? uu : 0;
      uint4* kx = reinterpret_cast<uint4*>(buf + swz(rt, c));
      const uint4 xr = *kx;
      const uint4 yr = *reinterpret_cast<const uint4*>(buf + swz(rt, c ^ 8));
      const bf16x8 xv = __builtin_bit_cast(bf16x8, xr), yv = __builtin_bit_cast(bf16x8, yr);
      const int dep = a.depth[u];
      bf16x8 rot;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 cs = s_cs[dep][8 * (c & 7) + e];
        const float x = float(xv[e]), y = float(yv[e]);
        rot[e] = static_cast<bf16>(c < 8 ? x * cs.x - y * cs.y : x * cs.x + y * cs.y);
      }
      const uint4 rr = __builtin_bit_cast(uint4, rot);
      __builtin_amdgcn_wave_barrier();
      *kx = rr;
      if (qt == 0 && uu < N) {
        const int64_t dst = (int64_t(P) + uu) * kD + c * 8;
        *reinterpret_cast<uint4*>(kc_w + dst) = rr;
        *reinterpret_cast<uint4*>(vc_w + dst) = *reinterpret_cast<const uint4*>(buf + 8192 + swz(rt, c));
      }
      __builtin_amdgcn_wave_barrier();
    }
  };

  f32x16 oacc[4][2];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[db][c][e] = 0.f;
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

  // One pipeline step: start the wave's next tile into `nxt`, then compute on `cur`.
  auto step = [&](int st, unsigned char* cur, unsigned char* nxt) {
    const int t = st * kWaves + wave;
    const bool ahead = issue_tile(t + kWaves, nxt);
    if (t >= n_tiles) return;
    if (ahead) wait_vm16();  // this tile's 16 loads are done; the next tile's 16 stay in flight
    else wait_vm0();
    if (t >= n_pre) rotate_staged(t, cur);
    const unsigned char* kb = cur;
    const unsigned char* vb = cur + 8192;

    // S^T = K Q^T: keys of the tile (rows) x 64 query columns, in two 32-column blocks
    f32x16 sacc[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[c][e] = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 kop = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kb + swz(l32, 2 * s + half)));
      sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[0][s], sacc[0], 0, 0, 0);
      sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[1][s], sacc[1], 0, 0, 0);
    }

    // visibility of the 16 keys this lane holds: key 8 (e / 4) + 4 half + e % 4
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      uint32_t bits;
      if (t < n_pre) {
        const int nvalid = k_hi - (k_lo + t * kTile);
        bits = nvalid >= 32 ? 0xffffffffu : ((1u << nvalid) - 1u);
      } else {
        const int v0 = (t - n_pre) * kTile;
        const uint64_t word = a.mask[int64_t(qnode[c]) * a.mask_words + (v0 >> 6)];
        bits = uint32_t(word >> (v0 & 63));
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = 8 * (e >> 2) + 4 * half + (e & 3);
        if (!((bits >> m) & 1u)) sacc[c][e] = -INFINITY;
      }
    }

    // online softmax (log2 units) per query column
    bf16x8 pop[2][2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float tmax = sacc[c][0];
#pragma unroll
      for (int e = 1; e < 16; ++e) tmax = fmaxf(tmax, sacc[c][e]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const bool grow = tmax > m_run[c] + kRescaleSlack;
      if (__ballot(grow)) {
        const float m_new = grow ? tmax : m_run[c];
        const float corr = grow ? exp2_fast(m_run[c] - m_new) : 1.0f;
        l_run[c] *= corr;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[db][c][e] *= corr;
        m_run[c] = m_new;
      }
      const float msafe = m_run[c] == -INFINITY ? 0.f : m_run[c];
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pe = exp2_fast(sacc[c][e] - msafe);
        sacc[c][e] = pe;
        psum += pe;
      }
      l_run[c] += psum;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int e = 0; e < 8; ++e) pop[c][t2][e] = static_cast<bf16>(sacc[c][8 * t2 + e]);
    }

    // O^T += V^T P^T: V^T operand for (32-dim block db, 16-key step t2) via transposing reads;
    // k index 8 h + e of the step pairs with key 16 t2 + 8 (e / 4) + 4 h + e % 4, which is
    // exactly the order in which the score accumulator holds P
    const int gq = lane >> 4, gi = lane & 15;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int dim = db * 32 + 16 * (gq & 1) + 4 * (gi & 3);
      const int doff = (dim & 4) << 1;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const int key0 = 16 * t2 + 4 * (gq >> 1) + (gi >> 2);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(vb + swz(key0, dim >> 3) + doff));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(vb + swz(key0 + 8, dim >> 3) + doff));
        const bf16x8 vop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[db][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[0][t2], oacc[db][0], 0, 0, 0);
        oacc[db][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[1][t2], oacc[db][1], 0, 0, 0);
      }
    }
  };

  // double-buffered stream over this wave's tiles; the two buffers are distinct LDS objects
  unsigned char* buf0 = s_tile0[wave];
  unsigned char* buf1 = s_tile1[wave];
  issue_tile(wave, buf0);
  for (int st = 0; st < steps; st += 2) {
    step(st, buf0, buf1);
    if (st + 1 < steps) step(st + 1, buf1, buf0);
  }

  // ---- merge the four wavefronts through LDS (two passes of 64 dims)
  float lsum[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) lsum[c] = l_run[c] + __shfl_xor(l_run[c], 32, 64);
  __syncthreads();
  float* obuf = reinterpret_cast<float*>(&s_tile0[0][0]);    // [wave][64 q][64 dims]
  float2* mlb = reinterpret_cast<float2*>(&s_tile1[0][0]);   // [wave][64 q]
  if (half == 0) {
#pragma unroll
    for (int c = 0; c < 2; ++c) mlb[wave * 64 + c * 32 + l32] = make_float2(m_run[c], lsum[c]);
  }
  Partial* part = nullptr;
  if (p.splits > 1)
    part = reinterpret_cast<Partial*>(static_cast<unsigned char*>(a.workspace) + p.partial_offset) +
           (int64_t(unit) * p.qtiles + qt) * p.splits + split;
  auto store_out = [&](int q, int dim0, float4 v) {
    const int r = qt * kRowsWG + q;
    if (r >= p.rows) return;
    const int u = r / p.group, h = kvh * p.group + r % p.group;
    bf16* o = static_cast<bf16*>(a.out) + ((int64_t(b) * N + u) * a.Hq + h) * kD + dim0;
    const bf16x4 ov = {static_cast<bf16>(v.x), static_cast<bf16>(v.y), static_cast<bf16>(v.z),
                       static_cast<bf16>(v.w)};
    *reinterpret_cast<bf16x4*>(o) = ov;
  };
#pragma unroll
  for (int dh = 0; dh < 2; ++dh) {
#pragma unroll
    for (int d2 = 0; d2 < 2; ++d2) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x16& o = oacc[2 * dh + d2][c];
          const float4 v = make_float4(o[4 * g4], o[4 * g4 + 1], o[4 * g4 + 2], o[4 * g4 + 3]);
          const int q = c * 32 + l32, dl = 32 * d2 + 8 * g4 + 4 * half;
          *reinterpret_cast<float4*>(obuf + (wave * 64 + q) * 64 + dl) = v;
        }
      }
    }
    __syncthreads();
    for (int it = tid; it < 64 * 16; it += 256) {
      const int q = it >> 4, d4 = it & 15;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mlb[w * 64 + q].x);
      float L = 0.f;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float2 ml = mlb[w * 64 + q];
        const float wt = M == -INFINITY ? 0.f : exp2_fast(ml.x - M);
        L += wt * ml.y;
        const float4 v = *reinterpret_cast<const float4*>(obuf + (w * 64 + q) * 64 + 4 * d4);
        acc.x += wt * v.x;
        acc.y += wt * v.y;
        acc.z += wt * v.z;
        acc.w += wt * v.w;
      }
      const int dim0 = 64 * dh + 4 * d4;
      if (p.splits == 1) {
        const float inv = 1.0f / L;
        store_out(q, dim0, make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv));
      } else {
        *reinterpret_cast<float4*>(&part->o[q][dim0]) = acc;
        if (dh == 0 && d4 == 0) {
          part->m[q] = M;
          part->l[q] = L;
        }
      }
    }
    __syncthreads();
  }
  if (p.splits == 1) return;

  // ---- the last split to arrive merges all splits of this q-tile
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    int* counter = static_cast<int*>(a.workspace) + (unit * p.qtiles + qt);
    const int prev = atomicAdd(counter, 1);
    s_int = prev == p.splits - 1;
    if (s_int) atomicExch(counter, 0);  // ready for the next call
  }
  __syncthreads();
  if (!s_int) return;
  __threadfence();
  const Partial* base = part - split;
  for (int it = tid; it < 64 * 32; it += 256) {
    const int q = it >> 5, d4 = it & 31;
    if (qt * kRowsWG + q >= p.rows) continue;
    float M = -INFINITY;
    for (int s = 0; s < p.splits; ++s) M = fmaxf(M, base[s].m[q]);
    float L = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < p.splits; ++s) {
      const float ms = base[s].m[q];
      const float wt = ms == -INFINITY ? 0.f : exp2_fast(ms - M);
      L += wt * base[s].l[q];
      const float4 v = *reinterpret_cast<const float4*>(&base[s].o[q][4 * d4]);
      acc.x += wt * v.x;
      acc.y += wt * v.y;
      acc.z += wt * v.z;
      acc.w += wt * v.w;
    }
    const float inv = 1.0f / L;
    store_out(q, 4 * d4, make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv));
  }
}

}  // namespace

bool mfma_path_applies(medusa_dtype dt, int32_t, int32_t, int32_t d_h, int32_t) {
  return dt == MEDUSA_BF16 && d_h == kD;
}

size_t attn_workspace_bytes(medusa_dtype dt, int32_t B, int32_t Hq, int32_t Hkv, int32_t d_h,
                            int32_t N, int32_t S_max) {
  if (B < 1 || Hkv < 1 || Hq < 1 || N < 1 || S_max < N) return 0;
  if (!mfma_path_applies(dt, Hq, Hkv, d_h, N)) return 256;
  return make_plan(B, Hq, Hkv, N, S_max).bytes;
}

medusa_status run_mfma(AttnArgs& a, hipStream_t stream, void* ev_start, void* ev_stop) {
  const Plan plan = make_plan(a.B, a.Hq, a.Hkv, a.N, a.S_max);
  MfmaArgs p{};
  p.a = a;
  p.group = plan.group;
  p.rows = plan.rows;
  p.qtiles = plan.qtiles;
  p.splits = plan.splits;
  p.xcd_map = plan.xcd_map ? 1 : 0;
  p.partial_offset = int32_t(plan.partial_offset);
  for (int j = 0; j < kD / 2; ++j) p.theta[j] = std::pow(a.rope_base, -2.0 * j / kD);
  const unsigned grid = unsigned(int64_t(plan.units) * plan.splits * plan.qtiles);
  return launch(reinterpret_cast<const void*>(&tree_attn_mfma_kernel), dim3(grid), dim3(256), 0,
                stream, p, ev_start, ev_stop);
}

}  // namespace medusa
