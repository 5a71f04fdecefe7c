// Matrix-core tree attention for bf16, d_h = 128 (gfx950).
//
// What is computed is the tree attention of [M7.2] = "M7.2 - Medusa: Multi-Head
// Candidates, Tree Attention, and Verification", §0x03A/§0x03C (position
// P + depth; N query rows against the P committed rows and the N staged rows,
// staged row u stored at cache row P + u and visible to w iff u is an ancestor
// of w or w itself) -- the same contract as the wavefront-per-row path.
//
// Mapping to CDNA4:
//  * One (sequence b, kv head g) pair -- a unit -- owns a query block of
//    N * (Hq/Hkv) rows: every tree node times every query head of the GQA group.
//    That block against a key tile is a dense contraction, so both products run
//    on v_mfma_f32_32x32x16_bf16.  With 256 rows per unit each key byte feeds
//    about as many flops as the matrix cores retire per HBM byte, so the kernel
//    is balanced between HBM and MFMA and must overlap the two.
//  * A workgroup takes up to 256 query rows of one unit (four wavefronts of 64
//    rows) and one contiguous split of the unit's key tiles: the committed prefix
//    followed by the staged rows.  Every key tile is fetched from HBM once, into
//    LDS, and read there by all four wavefronts.  Query blocks of 128 rows or
//    fewer use two key phases instead: wavefront pairs take alternate tiles.
//  * The LDS holds a ring of eight 32-key tiles (K and V, 128 KiB) filled by
//    direct global->LDS loads up to seven tiles ahead, so that about 100 KiB per
//    CU is in flight, which is what HBM latency times bandwidth asks for.  Each
//    wavefront loads its eight rows of every tile; one workgroup barrier per
//    tile publishes the tile and frees the slot of the tile before.
//  * Scores are formed transposed, S^T = K Q^T (K rows are the A operand,
//    16-byte LDS reads), so the probability tile comes out of the accumulator
//    already in the B-operand order of O^T = V^T P^T; V^T comes from LDS with
//    the transposing ds_read_b64_tr_b16.  P is never shuffled.
//  * Software pipeline per wavefront: the scores of tile j+1 run on the matrix
//    core while the VALU does the softmax of tile j.
//  * Online softmax in log2 units; the running maximum only moves when a tile
//    exceeds it by more than 2^8, so the O rescale is almost never paid.
//  * Staged keys are rotated to P + depth(u) in LDS by the wavefront that
//    loaded them (binary64 phase angles kept as fp32 cos/sin), written to cache
//    rows P + u by query block 0, and masked per lane with the ancestor bitmask.
//  * Splits of one query block are merged by a second, small kernel from
//    (m, l, O) partials in the workspace; with a single split the first kernel
//    writes the output itself.

#include <cmath>

#include "attn_common.h"

namespace medusa {
namespace {

constexpr int kD = 128;          // head dimension
constexpr int kTile = 32;        // keys per tile
constexpr int kWaves = 4;
constexpr int kRowsWave = 64;    // query rows per wavefront
constexpr int kRing = 8;         // tile buffers in LDS
constexpr int kTileBytes = 2 * kTile * kD * 2;  // K then V of one tile
constexpr int kTableDepth = 32;  // RoPE phases kept in LDS; deeper trees are rejected
constexpr int kDepthLds = 8192;  // node depths cached in LDS (bytes); later nodes read HBM
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
  int32_t group;     // Hq / Hkv
  int32_t rows;      // N * group query rows per unit
  int32_t n_kp;      // key phases: 1 (four wavefronts share every tile) or 2
  int32_t qrows;     // query rows per workgroup: 64 * 4 / n_kp
  int32_t qblocks;   // ceil(rows / qrows)
  int32_t splits;    // workgroups sharing one query block's keys
  int32_t xcd_map;   // keep the query blocks of one (unit, split) on one XCD
  int64_t o_offset;  // byte offset of the partial O in the workspace
  double theta[kD / 2];  // RoPE inverse frequencies base^(-2i/d)
};

struct MergeArgs {
  const float2* ml;  // [units][qblocks][splits][qrows] (m, l)
  const float* o;    // [units][qblocks][splits][qrows][D]
  void* out;
  const int32_t* status;
  int32_t Hq, Hkv, N, group, rows, qrows, qblocks, splits;
};

struct Plan {
  int32_t units, group, rows, n_kp, qrows, qblocks, splits;
  bool xcd_map;
  size_t o_offset, bytes;
};

Plan make_plan(int32_t B, int32_t Hq, int32_t Hkv, int32_t N, int32_t S_max) {
  Plan p{};
  p.units = B * Hkv;
  p.group = Hq / Hkv;
  p.rows = N * p.group;
  p.n_kp = p.rows > 2 * kRowsWave ? 1 : 2;
  p.qrows = kRowsWave * kWaves / p.n_kp;
  p.qblocks = (p.rows + p.qrows - 1) / p.qrows;
  const int32_t wgs = p.units * p.qblocks;
  int32_t splits = (kTargetWGs + wgs / 2) / wgs;
  // at least four stages of tiles per split
  const int64_t tiles = (int64_t(S_max) - N + kTile - 1) / kTile + (N + kTile - 1) / kTile;
  const int64_t max_splits = tiles / (4 * p.n_kp);
  splits = splits < max_splits ? splits : int32_t(max_splits);
  p.splits = splits < 1 ? 1 : splits;
  p.xcd_map = p.qblocks > 1 && (int64_t(p.units) * p.splits) % 8 == 0;
  const size_t slots = size_t(p.units) * p.qblocks * p.splits * p.qrows;
  p.o_offset = (slots * sizeof(float2) + 255) / 256 * 256;
  p.bytes = p.splits > 1 ? p.o_offset + slots * kD * sizeof(float) : 256;
  return p;
}

// byte offset of (row, 16-byte chunk) in a 32 x 256-byte matrix; chunks are
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
// does not pair it with a full vmcnt(0) drain before every LDS read; the tile ring
// waits with explicit, in-order vmcnt counts instead (a load issued later only
// lengthens a wait).
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  const uint64_t addr = uint64_t(base);
  // readfirstlane yields a signed int: widen through uint32_t so the low word is not sign-extended
  const uint32_t lo = uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(addr)));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(addr >> 32)));
  const uint64_t sbase = uint64_t(lo) | (uint64_t(hi) << 32);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

// wait until at most n of this wavefront's vector memory operations are outstanding
// (n rounded down to a multiple of 4, which only makes the wait stricter)
__device__ __forceinline__ void wait_vm(int n) {
  switch (n >= 24 ? 6 : n >> 2) {
    case 6: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(20)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
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
  const int n_kp = p.n_kp;
  const int kp = wave % n_kp, rb = wave / n_kp;  // key phase, 64-row block

  // ---- this workgroup's (sequence, kv head, split, query block)
  int grp, qb;
  if (p.xcd_map) {
    const int slot = blockIdx.x >> 3;
    grp = int(blockIdx.x & 7) + 8 * (slot / p.qblocks);
    qb = slot % p.qblocks;
  } else {
    grp = blockIdx.x / p.qblocks;
    qb = blockIdx.x % p.qblocks;
  }
  const int unit = grp / p.splits, split = grp % p.splits;
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int P = a.prefix_len[b];
  const int N = a.N;

  __shared__ __attribute__((aligned(16))) unsigned char s_ring[kRing][kTileBytes];
  __shared__ float2 s_cs[kTableDepth][kD / 2];
  __shared__ unsigned char s_dep[kDepthLds];
  __shared__ int s_int;

  // ---- key tiles of the unit: n_pre prefix tiles (the last one may be partial), then the
  // staged tiles.  Stage i of this split holds tiles (s_lo + i) * n_kp + k, k < n_kp, in
  // ring slot i % S.
  const int n_pre = (P + kTile - 1) / kTile;
  const int T = n_pre + (N + kTile - 1) / kTile;
  const int n_stages = (T + n_kp - 1) / n_kp;
  const int s_lo = int(int64_t(split) * n_stages / p.splits);
  const int n_st = int(int64_t(split + 1) * n_stages / p.splits) - s_lo;
  const int S = kRing / n_kp;  // 8 or 4 stages in the ring
  auto tile_start = [&](int i) __attribute__((always_inline)) { return (s_lo + i) * n_kp; };
  auto tile_end = [&](int i) __attribute__((always_inline)) { return min(T, (s_lo + i + 1) * n_kp); };

  const int64_t head = (int64_t(b) * a.Hkv + kvh) * a.S_max * kD;
  const bf16* kc = static_cast<const bf16*>(a.k_cache) + head;
  const bf16* vc = static_cast<const bf16*>(a.v_cache) + head;
  bf16* kc_w = static_cast<bf16*>(a.k_cache) + head;
  bf16* vc_w = static_cast<bf16*>(a.v_cache) + head;
  const bf16* kn = static_cast<const bf16*>(a.k_new) + (int64_t(b) * N * a.Hkv + kvh) * kD;
  const bf16* vn = static_cast<const bf16*>(a.v_new) + (int64_t(b) * N * a.Hkv + kvh) * kD;
  // LDS buffer of stage i's k-th tile: K at +0, V at +8192
  auto tbuf = [&](int i, int k) __attribute__((always_inline)) -> unsigned char* {
    return s_ring[(i & (S - 1)) * n_kp + k];
  };

  // Rows 8 w .. 8 w + 7 of one tile's K and V by direct global->LDS loads (wavefront w,
  // two instructions of four rows per matrix): lane l lands at byte 1024 i + 16 l of the
  // matrix, i.e. row 4 i + l / 16, stored chunk l % 16, and fetches logical chunk
  // (l % 16) ^ (row % 16), so that the buffer holds the layout swz() reads back.
  uint32_t poff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int rt = 4 * (2 * wave + h) + (lane >> 4);
    poff[h] = uint32_t(rt * 256 + (((lane & 15) ^ (rt & 15)) << 4));
  }
  auto issue_tile = [&](int t, unsigned char* buf) __attribute__((always_inline)) {
    const uint32_t lds = lds_addr(buf) + 2048 * wave;
    if ((t + 1) * kTile <= P) {  // full prefix tile
      const int64_t off = int64_t(t) * kTile * kD;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        dma16(kc + off, poff[h], lds + 1024 * h);
        dma16(vc + off, poff[h], lds + 8192 + 1024 * h);
      }
    } else if (t < n_pre) {  // the partial prefix tile: rows past P repeat row 0
      const int64_t off = int64_t(t) * kTile * kD;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int rt = 4 * (2 * wave + h) + (lane >> 4);
        const int r = t * kTile + rt < P ? rt : 0;
        const uint32_t o = uint32_t(r * 256 + (((lane & 15) ^ (rt & 15)) << 4));
        dma16(kc + off, o, lds + 1024 * h);
        dma16(vc + off, o, lds + 8192 + 1024 * h);
      }
    } else {  // staged rows from k_new / v_new; rows past the tree repeat node 0
      const int v0 = (t - n_pre) * kTile;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int rt = 4 * (2 * wave + h) + (lane >> 4);
        const int u = v0 + rt < N ? v0 + rt : 0;
        const uint32_t o = uint32_t((u * a.Hkv * kD + 8 * ((lane & 15) ^ (rt & 15))) * 2);
        dma16(kn, o, lds + 1024 * h);
        dma16(vn, o, lds + 8192 + 1024 * h);
      }
    }
  };
  auto issue_stage = [&](int i) __attribute__((always_inline)) {
    for (int k = 0; k < n_kp; ++k) {
      const int t = tile_start(i) + k;
      if (t < T) issue_tile(t, tbuf(i, k));
    }
  };
  // wait until this wavefront's loads of stage i have landed, stages up to `last` having
  // been issued (four loads per tile)
  auto wait_stage = [&](int i, int last) __attribute__((always_inline)) {
    wait_vm(last > i ? 4 * (tile_end(last) - tile_end(i)) : 0);
  };

  // fill the ring, all but one slot, before the latency-bound set-up below
  const int first = min(S - 1, n_st);
  for (int i = 0; i < first; ++i) issue_stage(i);

  // ---- node depths (LDS copy) and the RoPE phases (cos, sin) of positions P + d for
  // every depth d of the tree
  if (tid == 0) s_int = 0;
  __syncthreads();
  int dmax = 0;
  for (int i = tid; i < N; i += 256) {
    const int d = a.depth[i];
    dmax = max(dmax, d);
    if (i < kDepthLds) s_dep[i] = static_cast<unsigned char>(d);
  }
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
  auto depth_of = [&](int u) __attribute__((always_inline)) -> int {
    return u < kDepthLds ? int(s_dep[u]) : a.depth[u];
  };

  // ---- this wavefront's 64 query rows: rotated, scaled to log2 units, bf16 B operands;
  // lane holds query column l32 of column block c, dims 16 s + 8 half + e (e < 8)
  const int row0 = qb * p.qrows + rb * kRowsWave;
  const float qscale = kLog2e / sqrtf(float(kD));
  bf16x8 qop[2][8];
  int qnode[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int r = row0 + c * 32 + l32;
    const bool live = r < p.rows;
    const int u = live ? r / p.group : 0;
    const int h = kvh * p.group + (live ? r % p.group : 0);
    qnode[c] = u;
    const bf16* qr = static_cast<const bf16*>(a.q) + ((int64_t(b) * N + u) * a.Hq + h) * kD;
    uint4 raw[8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
      raw[s] = live ? *reinterpret_cast<const uint4*>(qr + 16 * s + 8 * half) : make_uint4(0, 0, 0, 0);
    const int dep = depth_of(u);
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

  // Staged rows of one tile that this wavefront loaded (rows 8 w .. 8 w + 7): rotate K in
  // place to P + depth(u); query block 0 also stores K~ and V to cache rows P + u.  Lane l
  // takes row 8 w + l / 8 and the chunk pair (l % 8, l % 8 + 8), i.e. dims j and j + 64.
  auto fix_staged = [&](int t, unsigned char* buf) __attribute__((always_inline)) {
    const int rt = 8 * wave + (lane >> 3), c = lane & 7;
    const int uu = (t - n_pre) * kTile + rt;
    const int dep = depth_of(uu < N ? uu : 0);
    uint4* px = reinterpret_cast<uint4*>(buf + swz(rt, c));
    uint4* py = reinterpret_cast<uint4*>(buf + swz(rt, c + 8));
    const bf16x8 xv = __builtin_bit_cast(bf16x8, *px);
    const bf16x8 yv = __builtin_bit_cast(bf16x8, *py);
    bf16x8 rx, ry;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float2 cs = s_cs[dep][8 * c + e];
      const float x = float(xv[e]), y = float(yv[e]);
      rx[e] = static_cast<bf16>(x * cs.x - y * cs.y);
      ry[e] = static_cast<bf16>(y * cs.x + x * cs.y);
    }
    *px = __builtin_bit_cast(uint4, rx);
    *py = __builtin_bit_cast(uint4, ry);
    if (qb == 0 && uu < N) {
      bf16* kd = kc_w + (int64_t(P) + uu) * kD;
      bf16* vd = vc_w + (int64_t(P) + uu) * kD;
      *reinterpret_cast<uint4*>(kd + 8 * c) = __builtin_bit_cast(uint4, rx);
      *reinterpret_cast<uint4*>(kd + 8 * c + 64) = __builtin_bit_cast(uint4, ry);
      *reinterpret_cast<uint4*>(vd + 8 * c) = *reinterpret_cast<const uint4*>(buf + 8192 + swz(rt, c));
      *reinterpret_cast<uint4*>(vd + 8 * c + 64) = *reinterpret_cast<const uint4*>(buf + 8192 + swz(rt, c + 8));
    }
  };
  // once stage i has landed: the staged tiles of the stage get their rows fixed
  auto fix_stage = [&](int i) __attribute__((always_inline)) {
    for (int k = 0; k < n_kp; ++k) {
      const int t = tile_start(i) + k;
      if (t >= n_pre && t < T) fix_staged(t, tbuf(i, k));
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
  // visibility bits of a tile's 32 keys for query column block c (bit m = key m of the
  // tile); all ones for a full prefix tile
  auto tile_bits = [&](int t, uint32_t (&bits)[2]) __attribute__((always_inline)) {
    if (t < n_pre) {
      const int nvalid = P - t * kTile;
      bits[0] = bits[1] = nvalid >= 32 ? 0xffffffffu : ((1u << nvalid) - 1u);
    } else {
      const int v0 = (t - n_pre) * kTile;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint64_t word = a.mask[int64_t(qnode[c]) * a.mask_words + (v0 >> 6)];
        bits[c] = uint32_t(word >> (v0 & 63));
      }
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

  // per-lane LDS offsets of the V^T operand reads: 32-dim block db, key group h of the
  // 16-key step; the step t2 adds 16 rows (4096 bytes) to both
  const int gq = lane >> 4, gi = lane & 15;
  int voff[4][2];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int dim = db * 32 + 16 * (gq & 1) + 4 * (gi & 3);
    const int key0 = 4 * (gq >> 1) + (gi >> 2);
    voff[db][0] = 8192 + swz(key0, dim >> 3) + ((dim & 4) << 1);
    voff[db][1] = 8192 + swz(key0 + 8, dim >> 3) + ((dim & 4) << 1);
  }

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
  auto pv = [&](const unsigned char* tb, const bf16x8 (&pop)[2][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tb + voff[db][0] + 4096 * t2));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tb + voff[db][1] + 4096 * t2));
        const bf16x8 vop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[db][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[0][t2], oacc[db][0], 0, 0, 0);
        oacc[db][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[1][t2], oacc[db][1], 0, 0, 0);
      }
    }
  };

  // this wavefront's tile of stage i: visibility bits and scores
  auto prep = [&](int i, f32x16 (&s)[2], uint32_t (&bits)[2]) __attribute__((always_inline)) {
    const int t = tile_start(i) + kp;
    if (t < T) {
      tile_bits(t, bits);
      qk(tbuf(i, kp), s);
    }
  };
  // masking, softmax and PV of this wavefront's tile of stage i
  auto consume = [&](int i, f32x16 (&s)[2], const uint32_t (&bits)[2]) __attribute__((always_inline)) {
    const int t = tile_start(i) + kp;
    if (t >= T) return;
    if (t >= n_pre - 1) {  // the last prefix tile or a staged tile
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = 8 * (e >> 2) + 4 * half + (e & 3);
          if (!((bits[c] >> m) & 1u)) s[c][e] = -INFINITY;
        }
    }
    float m_use[2];
    update_max(s, m_use);
    bf16x8 pop[2][2];
    softmax(s, m_use, pop);
    pv(tbuf(i, kp), pop);
  };
  // one step: publish stage i+1 and refill the slot of stage i-1, form the scores of
  // stage i+1 on the matrix core, then finish stage i
  auto step = [&](int i, f32x16 (&s_cur)[2], uint32_t (&b_cur)[2], f32x16 (&s_nxt)[2],
                  uint32_t (&b_nxt)[2]) __attribute__((always_inline)) {
    if (i + 1 < n_st) {
      wait_stage(i + 1, min(i + S - 2, n_st - 1));
      fix_stage(i + 1);
      __syncthreads();  // stage i+1 visible; every wavefront is done with stage i-1
      if (i + S - 1 < n_st) issue_stage(i + S - 1);
      prep(i + 1, s_nxt, b_nxt);
    }
    consume(i, s_cur, b_cur);
  };

  f32x16 s_a[2], s_b[2];
  uint32_t b_a[2] = {0u, 0u}, b_b[2] = {0u, 0u};
  if (n_st > 0) {
    wait_stage(0, first - 1);
    fix_stage(0);
    __syncthreads();
    prep(0, s_a, b_a);
  }
  for (int i = 0; i < n_st; i += 2) {
    step(i, s_a, b_a, s_b, b_b);
    if (i + 1 < n_st) step(i + 1, s_b, b_b, s_a, b_a);
  }

  // ---- combine the key phases (n_kp = 2: wavefront (rb, 1) hands its state to (rb, 0))
  float lsum[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    float y0, y1;
    halves(l_run[c], y0, y1);
    lsum[c] = y0 + y1;
  }
  if (n_kp == 2) {
    __syncthreads();  // every wavefront is done with the ring
    float* xo = reinterpret_cast<float*>(&s_ring[0][0]) + rb * (128 * 64 + 4 * 64);
    if (kp == 1) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int e = 0; e < 16; ++e) xo[((db * 2 + c) * 16 + e) * 64 + lane] = oacc[db][c][e];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        xo[128 * 64 + c * 64 + lane] = m_run[c];
        xo[128 * 64 + (2 + c) * 64 + lane] = lsum[c];
      }
    }
    __syncthreads();
    if (kp == 1) return;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const float m1 = xo[128 * 64 + c * 64 + lane], l1 = xo[128 * 64 + (2 + c) * 64 + lane];
      const float M = fmaxf(m_run[c], m1);
      const float w0 = m_run[c] == -INFINITY ? 0.f : exp2_fast(m_run[c] - M);
      const float w1 = m1 == -INFINITY ? 0.f : exp2_fast(m1 - M);
      lsum[c] = w0 * lsum[c] + w1 * l1;
      m_run[c] = M;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          oacc[db][c][e] = w0 * oacc[db][c][e] + w1 * xo[((db * 2 + c) * 16 + e) * 64 + lane];
    }
  }

  // ---- results: lane (half, l32) holds, for query row c * 32 + l32 of its 64-row block,
  // dims 32 db + 8 g + 4 half + 0..3 in oacc[db][c][4 g .. 4 g + 3]
  if (p.splits == 1) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int r = row0 + c * 32 + l32;
      if (r >= p.rows) continue;
      const int u = r / p.group, h = kvh * p.group + r % p.group;
      bf16* o = static_cast<bf16*>(a.out) + ((int64_t(b) * N + u) * a.Hq + h) * kD + 4 * half;
      const float inv = 1.0f / lsum[c];
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16& v = oacc[db][c];
          const bf16x4 ov = {static_cast<bf16>(v[4 * g] * inv), static_cast<bf16>(v[4 * g + 1] * inv),
                             static_cast<bf16>(v[4 * g + 2] * inv), static_cast<bf16>(v[4 * g + 3] * inv)};
          *reinterpret_cast<bf16x4*>(o + 32 * db + 8 * g) = ov;
        }
    }
    return;
  }
  const int64_t slot0 = ((int64_t(unit) * p.qblocks + qb) * p.splits + split) * p.qrows + rb * kRowsWave;
  float2* ml = static_cast<float2*>(a.workspace) + slot0;
  float* po = reinterpret_cast<float*>(static_cast<unsigned char*>(a.workspace) + p.o_offset) + slot0 * kD;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int q = c * 32 + l32;
    if (half == 0) ml[q] = make_float2(m_run[c], lsum[c]);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& v = oacc[db][c];
        *reinterpret_cast<float4*>(po + q * kD + 32 * db + 8 * g + 4 * half) =
            make_float4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
      }
  }
}

// Merge of the splits: thread (row, 4 dims) combines the splits' (m, l, O) partials.
__global__ __launch_bounds__(256) void tree_attn_merge_kernel(MergeArgs p) {
  if (round_failed(p.status)) return;
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int d4 = int(idx & 31);
  const int64_t g = idx >> 5;  // (unit, query block, row of the block)
  const int r = int(g % p.qrows);
  const int64_t uq = g / p.qrows;
  const int qb = int(uq % p.qblocks);
  const int unit = int(uq / p.qblocks);
  const int row = qb * p.qrows + r;
  if (row >= p.rows) return;
  const int64_t base = uq * p.splits * p.qrows + r;  // slot of split 0
  float M = -INFINITY;
  for (int s = 0; s < p.splits; ++s) M = fmaxf(M, p.ml[base + int64_t(s) * p.qrows].x);
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < p.splits; ++s) {
    const int64_t slot = base + int64_t(s) * p.qrows;
    const float2 ml = p.ml[slot];
    const float wt = ml.x == -INFINITY ? 0.f : exp2_fast(ml.x - M);
    L += wt * ml.y;
    const float4 v = *reinterpret_cast<const float4*>(p.o + slot * kD + 4 * d4);
    acc.x += wt * v.x;
    acc.y += wt * v.y;
    acc.z += wt * v.z;
    acc.w += wt * v.w;
  }
  const float inv = 1.0f / L;
  const int b = unit / p.Hkv, kvh = unit % p.Hkv;
  const int u = row / p.group, h = kvh * p.group + row % p.group;
  bf16* o = static_cast<bf16*>(p.out) + ((int64_t(b) * p.N + u) * p.Hq + h) * kD + 4 * d4;
  const bf16x4 ov = {static_cast<bf16>(acc.x * inv), static_cast<bf16>(acc.y * inv),
                     static_cast<bf16>(acc.z * inv), static_cast<bf16>(acc.w * inv)};
  *reinterpret_cast<bf16x4*>(o) = ov;
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
  p.n_kp = plan.n_kp;
  p.qrows = plan.qrows;
  p.qblocks = plan.qblocks;
  p.splits = plan.splits;
  p.xcd_map = plan.xcd_map ? 1 : 0;
  p.o_offset = int64_t(plan.o_offset);
  for (int j = 0; j < kD / 2; ++j) p.theta[j] = std::pow(a.rope_base, -2.0 * j / kD);
  const unsigned grid = unsigned(int64_t(plan.units) * plan.splits * plan.qblocks);
  const void* attn = reinterpret_cast<const void*>(&tree_attn_mfma_kernel);
  if (plan.splits == 1) return launch(attn, dim3(grid), dim3(256), 0, stream, p, ev_start, ev_stop);
  const medusa_status st = launch(attn, dim3(grid), dim3(256), 0, stream, p, ev_start, nullptr);
  if (st != MEDUSA_OK) return st;
  MergeArgs m{};
  m.ml = static_cast<const float2*>(a.workspace);
  m.o = reinterpret_cast<const float*>(static_cast<const unsigned char*>(a.workspace) + plan.o_offset);
  m.out = a.out;
  m.status = a.status;
  m.Hq = a.Hq;
  m.Hkv = a.Hkv;
  m.N = a.N;
  m.group = plan.group;
  m.rows = plan.rows;
  m.qrows = plan.qrows;
  m.qblocks = plan.qblocks;
  m.splits = plan.splits;
  const int64_t threads = int64_t(plan.units) * plan.qblocks * plan.qrows * 32;
  return launch(reinterpret_cast<const void*>(&tree_attn_merge_kernel),
                dim3(unsigned((threads + 255) / 256)), dim3(256), 0, stream, m, nullptr, ev_stop);
}

}  // namespace medusa
