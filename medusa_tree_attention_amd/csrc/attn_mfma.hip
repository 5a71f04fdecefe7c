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
//    the committed prefix; the last split also takes the staged rows.  Its
//    four wavefronts hold the same 64 rotated, pre-scaled query rows in
//    registers and each streams its own interleaved 32-key tiles, so the main
//    loop has no workgroup barrier.  The q-tiles of one split are launched
//    onto one XCD (block id modulo 8) so that their common KV stream is
//    fetched from HBM once and served from that XCD's L2.
//  * Tiles move by direct global->LDS loads (no staging registers), K two
//    tiles ahead and V one tile ahead, with explicit in-order vmcnt waits.
//  * Scores are formed transposed, S^T = K Q^T (K rows are the A operand,
//    16-byte LDS reads), so the probability tile comes out of the accumulator
//    already in the B-operand order of O^T = V^T P^T; V^T comes from LDS with
//    the transposing ds_read_b64_tr_b16.  P is never shuffled.
//  * Software pipeline per wave: the scores of tile j+1 run on the matrix
//    core while the VALU does the softmax of tile j.
//  * Online softmax in log2 units; the running maximum only moves when a tile
//    exceeds it by more than 2^8, so the O rescale is almost never paid.
//  * Staged keys are rotated to P + depth(u) in LDS (binary64 phase angles
//    kept as fp32 cos/sin), written to cache rows P + u by q-tile 0, and
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

// the values of lanes i and i ^ 32, in some order, for a cross-half max or sum
__device__ __forceinline__ void halves(float v, float& x, float& y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}

// 32-bit LDS address of a __shared__ pointer, made wave-uniform
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      uint32_t(size_t((__attribute__((address_space(3))) const void*)(p))));
}

// Direct global -> LDS load of 16 bytes per lane from base + voff (base wave-uniform):
// lane l's bytes land at lds + 16 l.  Issued as inline assembly so that the compiler
// does not pair it with a full vmcnt(0) drain before every LDS read; the tile pipeline
// waits with explicit, in-order vmcnt counts instead (a load issued later only
// lengthens a wait).
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(voff), "s"(base)
               : "memory", "m0");
}
__device__ __forceinline__ void wait_vm(int outstanding) {
  if (outstanding >= 16)
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else if (outstanding >= 8)
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

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
  // per wave: K and V double buffers of one 32 x 128 tile each; the final merge reuses them
  __shared__ __attribute__((aligned(16))) unsigned char s_k[2][kWaves][8192];
  __shared__ __attribute__((aligned(16))) unsigned char s_v[2][kWaves][8192];
  __shared__ int s_int;

  // ---- key range: split `split` of the committed prefix, plus the staged rows in the last split
  const int per = ((P + p.splits - 1) / p.splits + kTile - 1) / kTile * kTile;
  const int k_lo = min(P, split * per), k_hi = min(P, k_lo + per);
  const int n_pre = (k_hi - k_lo + kTile - 1) / kTile;
  const int n_stg = (split == p.splits - 1) ? (N + kTile - 1) / kTile : 0;
  const int n_tiles = n_pre + n_stg;
  // this wave's tiles are wave, wave + 4, wave + 8, ...
  const int J = wave < n_tiles ? (n_tiles - wave + kWaves - 1) / kWaves : 0;
  auto tile_of = [&](int j) __attribute__((always_inline)) { return wave + kWaves * j; };

  const int64_t head = (int64_t(b) * a.Hkv + kvh) * a.S_max * kD;
  const bf16* kc = static_cast<const bf16*>(a.k_cache) + head;
  const bf16* vc = static_cast<const bf16*>(a.v_cache) + head;
  bf16* kc_w = static_cast<bf16*>(a.k_cache) + head;
  bf16* vc_w = static_cast<bf16*>(a.v_cache) + head;
  const bf16* kn = static_cast<const bf16*>(a.k_new);
  const bf16* vn = static_cast<const bf16*>(a.v_new);
  auto kbuf = [&](int j) __attribute__((always_inline)) -> unsigned char* { return s_k[j & 1][wave]; };
  auto vbuf = [&](int j) __attribute__((always_inline)) -> unsigned char* { return s_v[j & 1][wave]; };

  // One tile's K or V rows into a buffer by direct global->LDS loads: instruction i moves
  // rows 4 i .. 4 i + 3 (1 KiB, lane l -> bytes 16 l); lane l fetches logical chunk
  // (l % 16) ^ (row % 16) so that the buffer holds the layout swz() reads back.  For a
  // full prefix tile the byte offsets of rows 0..15 are fixed per lane (rows 16..31 use
  // the same offsets from a base 16 rows further on).
  const int n_full = (k_hi - k_lo) / kTile;
  uint32_t poff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rt = 4 * i + (lane >> 4);
    poff[i] = uint32_t(rt * 256 + (((lane & 15) ^ rt) << 4));
  }
  auto issue = [&](int t, bool is_v, unsigned char* buf) __attribute__((always_inline)) {
    const uint32_t lds = lds_addr(buf);
    if (t < n_full) {
      const bf16* base = (is_v ? vc : kc) + int64_t(k_lo + t * kTile) * kD;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dma16(base, poff[i], lds + 1024 * i);
        dma16(base + 16 * kD, poff[i], lds + 1024 * (i + 4));
      }
    } else if (t < n_pre) {  // the partial prefix tile: rows past the split repeat row 0
      const int k0 = k_lo + t * kTile;
      const bf16* base = (is_v ? vc : kc) + int64_t(k0) * kD;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int rt = 4 * i + (lane >> 4);
        const int r = k0 + rt < k_hi ? rt : 0;
        dma16(base, uint32_t(r * 256 + (((lane & 15) ^ (rt & 15)) << 4)), lds + 1024 * i);
      }
    } else {  // staged rows come from k_new / v_new; rows past the tree repeat row 0
      const int v0 = (t - n_pre) * kTile;
      const bf16* base = (is_v ? vn : kn) + (int64_t(b) * N * a.Hkv + kvh) * kD;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int rt = 4 * i + (lane >> 4);
        const int u = v0 + rt < N ? v0 + rt : 0;
        dma16(base, uint32_t((u * a.Hkv * kD + 8 * ((lane & 15) ^ (rt & 15))) * 2), lds + 1024 * i);
      }
    }
  };

  // start the first tiles before the latency-bound set-up below
  if (J > 0) issue(tile_of(0), false, kbuf(0));
  if (J > 1) issue(tile_of(1), false, kbuf(1));
  if (J > 0) issue(tile_of(0), true, vbuf(0));

  // ---- RoPE phases (cos, sin) of positions P + d for every depth d of the tree
  if (tid == 0) s_int = 0;
  __syncthreads();
  int dmax = 0;
  for (int i = tid; i < N; i += 256) dmax = max(dmax, a.depth[i]);
  atomicMax(&s_int, dmax);
  __syncthreads();
  dmax = s_int;
  if (dmax >= kTableDepth) {  // uniform: every block sees the same tree
    wait_vm(0);               // no load may still target LDS when the block exits
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
    uint4 raw[8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
      raw[s] = live ? *reinterpret_cast<const uint4*>(qr + 16 * s + 8 * half) : make_uint4(0, 0, 0, 0);
    const int dep = a.depth[u];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 lo = __builtin_bit_cast(bf16x8, raw[s]);
      const bf16x8 hi = __builtin_bit_cast(bf16x8, raw[s + 4]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 cs = s_cs[dep][16 * s + 8 * half + e];
        const float x1 = float(lo[e]), x2 = float(hi[e]);
        qop[c][s][e] = static_cast<bf16>((x1 * cs.x - x2 * cs.y) * qscale);
        qop[c][s + 4][e] = static_cast<bf16>((x2 * cs.x + x1 * cs.y) * qscale);
      }
    }
  }

  // Staged rows: rotate K in place to P + depth(u); q-tile 0 also stores K~ to cache rows
  // P + u.  In each row every lane reads its chunk and the partner chunk (dims -+ 64)
  // before any lane of the wave writes.
  auto rotate_staged = [&](int t, unsigned char* buf) __attribute__((always_inline)) {
    const int v0 = (t - n_pre) * kTile;
    const int c = lane & 15;
    for (int i = 0; i < 8; ++i) {
      const int rt = 4 * i + (lane >> 4);
      const int uu = v0 + rt;
      const int u = uu < N ? uu : 0;
      uint4* kx = reinterpret_cast<uint4*>(buf + swz(rt, c));
      const bf16x8 xv = __builtin_bit_cast(bf16x8, *kx);
      const bf16x8 yv = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(buf + swz(rt, c ^ 8)));
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
      if (qt == 0 && uu < N)
        *reinterpret_cast<uint4*>(kc_w + (int64_t(P) + uu) * kD + c * 8) = rr;
      __builtin_amdgcn_wave_barrier();
    }
  };
  // Staged rows: q-tile 0 copies V to cache rows P + u
  auto store_staged_v = [&](int t, const unsigned char* buf) __attribute__((always_inline)) {
    const int v0 = (t - n_pre) * kTile;
    const int c = lane & 15;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rt = 4 * i + (lane >> 4);
      if (v0 + rt < N)
        *reinterpret_cast<uint4*>(vc_w + (int64_t(P) + v0 + rt) * kD + c * 8) =
            *reinterpret_cast<const uint4*>(buf + swz(rt, c));
    }
  };
  // S^T = K Q^T for one tile: 32 keys x 64 query columns
  auto qk = [&](const unsigned char* kb, f32x16 (&s)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[c][e] = 0.f;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const bf16x8 kop = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kb + swz(l32, 2 * st + half)));
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[0][st], s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[1][st], s[1], 0, 0, 0);
    }
  };
  // visibility bits of a tile's 32 keys for query column block c (bit m = key m of the tile)
  auto tile_bits = [&](int t, int c) __attribute__((always_inline)) -> uint32_t {
    if (t < n_pre) {
      const int nvalid = k_hi - (k_lo + t * kTile);
      return nvalid >= 32 ? 0xffffffffu : ((1u << nvalid) - 1u);
    }
    const int v0 = (t - n_pre) * kTile;
    const uint64_t word = a.mask[int64_t(qnode[c]) * a.mask_words + (v0 >> 6)];
    return uint32_t(word >> (v0 & 63));
  };

  f32x16 oacc[4][2];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[db][c][e] = 0.f;
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

  // per-lane LDS offsets of the V^T operand reads: 32-dim block db, key group h of the
  // 16-key step; the step t2 adds 16 rows (4096 bytes) to both
  const int gq = lane >> 4, gi = lane & 15;
  int voff[4][2];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int dim = db * 32 + 16 * (gq & 1) + 4 * (gi & 3);
    const int key0 = 4 * (gq >> 1) + (gi >> 2);
    voff[db][0] = swz(key0, dim >> 3) + ((dim & 4) << 1);
    voff[db][1] = swz(key0 + 8, dim >> 3) + ((dim & 4) << 1);
  }

  // The wave's tiles in order: full prefix tiles first (the pipelined main loop), then at
  // most one partial prefix tile and the staged tiles (the tail, which masks and rotates).
  const int Jf = wave < n_full ? (n_full - wave + kWaves - 1) / kWaves : 0;

  // start tile j+2's K and tile j+1's V; returns how many loads were issued
  auto prefetch = [&](int j) __attribute__((always_inline)) -> int {
    int n = 0;
    if (j + 2 < J) {
      issue(tile_of(j + 2), false, kbuf(j + 2));
      n += 8;
    }
    if (j + 1 < J) {
      issue(tile_of(j + 1), true, vbuf(j + 1));
      n += 8;
    }
    return n;
  };
  // running-max update of one tile's scores; rescales O and l in the rare case it moves
  auto update_max = [&](f32x16 (&sc)[2], float (&m_use)[2]) __attribute__((always_inline)) {
    bool grow_any = false;
    bool grow[2];
    float tmax[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float x = fmaxf(fmaxf(sc[c][0], sc[c][1]), fmaxf(sc[c][2], sc[c][3]));
#pragma unroll
      for (int e = 4; e < 16; e += 2) x = fmaxf(x, fmaxf(sc[c][e], sc[c][e + 1]));
      float y0, y1;
      halves(x, y0, y1);
      tmax[c] = fmaxf(y0, y1);
      grow[c] = tmax[c] > m_run[c] + kRescaleSlack;
      grow_any = grow_any || grow[c];
    }
    if (__ballot(grow_any)) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const float m_new = grow[c] ? tmax[c] : m_run[c];
        const float corr = grow[c] ? exp2_fast(m_run[c] - m_new) : 1.0f;
        l_run[c] *= corr;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[db][c][e] *= corr;
        m_run[c] = m_new;
      }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) m_use[c] = m_run[c] == -INFINITY ? 0.f : m_run[c];
  };
  // probabilities of one tile (in place), their row sums, and the bf16 B operands of P^T
  auto softmax = [&](f32x16 (&sc)[2], const float (&m_use)[2], bf16x8 (&pop)[2][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pe = exp2_fast(sc[c][e] - m_use[c]);
        sc[c][e] = pe;
        psum += pe;
      }
      l_run[c] += psum;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int e = 0; e < 8; ++e) pop[c][t2][e] = static_cast<bf16>(sc[c][8 * t2 + e]);
    }
  };
  // O^T += V^T P^T: k index 8 h + e of a 16-key step pairs with key 16 t2 + 8 (e / 4) +
  // 4 h + e % 4, exactly the order in which the score accumulator holds P
  auto pv = [&](const unsigned char* vb, const bf16x8 (&pop)[2][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + voff[db][0] + 4096 * t2));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + voff[db][1] + 4096 * t2));
        const bf16x8 vop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[db][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[0][t2], oacc[db][0], 0, 0, 0);
        oacc[db][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[1][t2], oacc[db][1], 0, 0, 0);
      }
    }
  };

  f32x16 s_a[2], s_b[2];
  if (J > 0) wait_vm(0);
  if (Jf > 0) qk(kbuf(0), s_a);

  // main loop over full prefix tiles: the scores of tile j+1 run on the matrix core while
  // the VALU turns tile j into probabilities
  auto iter = [&](int j, f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2]) __attribute__((always_inline)) {
    wait_vm(prefetch(j));  // K of tile j+1 and V of tile j have landed
    float m_use[2];
    update_max(s_cur, m_use);
    if (j + 1 < Jf) qk(kbuf(j + 1), s_nxt);
    bf16x8 pop[2][2];
    softmax(s_cur, m_use, pop);
    pv(vbuf(j), pop);
  };
  for (int j = 0; j < Jf; j += 2) {
    iter(j, s_a, s_b);
    if (j + 1 < Jf) iter(j + 1, s_b, s_a);
  }

  // tail: partial prefix tile and staged tiles, one at a time.  Tile j's scores are formed
  // here, so K of tile j+2 (same buffer as tile j) is only started once they are.
  for (int j = Jf; j < J; ++j) {
    const int t = tile_of(j);
    wait_vm(0);  // K and V of tile j have landed
    if (j + 1 < J) issue(tile_of(j + 1), true, vbuf(j + 1));
    if (t >= n_pre) {
      if (qt == 0) store_staged_v(t, vbuf(j));
      rotate_staged(t, kbuf(j));
    }
    qk(kbuf(j), s_a);
    if (j + 2 < J) issue(tile_of(j + 2), false, kbuf(j + 2));
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint32_t bits = tile_bits(t, c);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = 8 * (e >> 2) + 4 * half + (e & 3);
        if (!((bits >> m) & 1u)) s_a[c][e] = -INFINITY;
      }
    }
    float m_use[2];
    update_max(s_a, m_use);
    bf16x8 pop[2][2];
    softmax(s_a, m_use, pop);
    pv(vbuf(j), pop);
  }

  // ---- merge the four wavefronts through LDS (two passes of 64 dims)
  float lsum[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    float y0, y1;
    halves(l_run[c], y0, y1);
    lsum[c] = y0 + y1;
  }
  __syncthreads();
  float* obuf = reinterpret_cast<float*>(&s_k[0][0][0]);    // [wave][64 q][64 dims]
  float2* mlb = reinterpret_cast<float2*>(&s_v[0][0][0]);   // [wave][64 q]
  if (half == 0) {
#pragma unroll
    for (int c = 0; c < 2; ++c) mlb[wave * 64 + c * 32 + l32] = make_float2(m_run[c], lsum[c]);
  }
  Partial* part = nullptr;
  if (p.splits > 1)
    part = reinterpret_cast<Partial*>(static_cast<unsigned char*>(a.workspace) + p.partial_offset) +
           (int64_t(unit) * p.qtiles + qt) * p.splits + split;
  auto store_out = [&](int q, int dim0, float4 v) __attribute__((always_inline)) {
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
