// Matrix-core tree attention for bf16, d_h = 128 and 64 (gfx950).
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
//    is balanced between HBM and MFMA and has to overlap the two.
//  * A workgroup of eight wavefronts (two per SIMD, so that one wavefront's
//    softmax overlaps the other's matrix work) takes 128 query rows of one unit,
//    32 per wavefront, and one contiguous split of the unit's key tiles: the
//    committed prefix followed by the staged rows.  The workgroup's two halves
//    take alternate tiles (two key phases) and are combined through LDS at the
//    end.  A unit of 256 rows has two query blocks; their workgroups run on one
//    XCD, so each key tile comes from HBM once and from that XCD's L2 the second
//    time, while the split partials that the merge kernel reads stay half the
//    size they would be with one 256-row block and twice the splits.
//  * The LDS holds a ring of eight 32-key tiles (K and V, 128 KiB): four stages
//    of two tiles, filled by direct global->LDS loads up to three stages ahead.
//    Each wavefront loads four rows of every tile of a stage; one workgroup
//    barrier per stage publishes the stage and frees the slot of the stage before.
//  * LDS tiles are XOR-swizzled so that both the 16-byte K-operand reads and the
//    transposing V^T reads are free of bank conflicts on the 64-bank LDS.
//  * Scores are formed transposed, S^T = K Q^T (K rows are the A operand,
//    16-byte LDS reads), so the probability tile comes out of the accumulator
//    already in the B-operand order of O^T = V^T P^T; V^T comes from LDS with
//    the transposing ds_read_b64_tr_b16.  P is never shuffled.
//  * The rotated, scaled query q~ is carried as two bf16 operands, hi = bf16(q~)
//    and lo = bf16(q~ - hi), and each score is K hi + K lo.  One bf16 rounding of
//    q~ alone moves a score by about 2^-9 |q~||k|, which a peaked softmax hands on
//    to the output almost undamped; the pair is exact to about 2^-17.
//  * Software pipeline per wavefront: the scores of tile j+1 are formed on the
//    matrix core before the softmax of tile j.
//  * Online softmax in log2 units; the running maximum only moves when a tile
//    exceeds it by more than 2^8, so the O rescale is almost never paid.  Row
//    sums are taken over the bf16-rounded probabilities (the values P V uses)
//    with packed bf16 dot products.
//  * Everything the set-up reads from memory (status, prefix lengths, query
//    inputs, node depths, staged visibility words) is loaded at once, together
//    with the tiles of the first two stages, and consumed before the rest of the
//    ring is filled, so that no compiler-inserted wait drains the tile ring.
//  * Staged keys are rotated to P + depth(u) in LDS by the wavefront that
//    loaded them, written to cache rows P + u by query block 0, and masked per
//    lane with the ancestor bitmask.  RoPE phases are reduced modulo 2 pi in
//    binary64 and evaluated in fp32.
//  * Splits of one query block are merged by a second, small kernel from (m, l)
//    and O / l partials in the workspace, O / l as 16-bit fixed point scaled by the
//    row's largest |O / l| (within 2^-16 of it: a bf16 partial would add a second
//    rounding of the output's size); with a single split the first kernel writes
//    the output itself.

#include <algorithm>
#include <cmath>
#include <type_traits>

#include "attn_common.h"

namespace medusa {
namespace {

constexpr int kD = 128;          // head dimension of the LDS and operand layout (d_h = 64 is padded to it)
constexpr int kTile = 32;        // keys per tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kKeyPhases = kWaves / 4;   // wavefronts per SIMD: each takes every kKeyPhases-th tile
constexpr int kDmaRows = 32 / kWaves;     // rows of every tile each wavefront loads
constexpr int kDmaOps = kDmaRows / 4;     // direct-to-LDS instructions per matrix and tile
constexpr int kRowsWave = 32;    // query rows per wavefront
constexpr int kRing = 8;         // tile buffers in LDS
constexpr int kTileBytes = 2 * kTile * kD * 2;  // K then V of one tile
constexpr int kTableDepth = 32;  // RoPE phases kept in LDS; deeper trees are rejected
constexpr int kEarlyDepth = 8;   // phases formed before the node depths are known
constexpr int kDepthLds = 4096;  // node depths cached in LDS (bytes); later nodes read memory
constexpr int kMaskLds = 8;      // staged tiles whose visibility words are kept in LDS
constexpr int kTargetWGs = 256;  // one workgroup per compute unit
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;  // log2 units
constexpr double kTwoPiHi = 6.283185307179586;         // 2 pi = hi + lo
constexpr double kTwoPiLo = 2.4492935982947064e-16;
constexpr double kInvTwoPi = 0.15915494309189535;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Indices are divided by run-time divisors without the integer division sequence (about 25
// instructions, several of them quarter rate; the set-up of a workgroup needs a dozen).
//
// Per-lane indices use an fp32 reciprocal.  With r = 1/d rounded up to fp32,
// trunc(fl(n r)) = floor(n / d) for 0 <= n < kFastDivMax and d <= kFastDivMax: the product
// is at least n / d, so an exact quotient stays whole, and it exceeds n / d by less than
// (n + d) 2^-23 / d, which stays below the distance 1 / d to the next integer.
constexpr int32_t kFastDivMax = 1 << 21;
float rcp_up(int32_t d) {
  float r = 1.0f / float(d);
  if (double(r) * d < 1.0) r = std::nextafter(r, 2.0f);
  return r;
}
__device__ __forceinline__ int idiv(int n, float r) { return int(float(n) * r); }

// Wave-uniform indices use a multiply-high on the scalar unit (Granlund and Montgomery,
// "Division by invariant integers using multiplication", 1994, the round-up multiplier of
// N + 1 bits): with l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1,
// floor(n / d) = (mulhi(n, m) + n) >> l for 0 <= n < 2^31 (the sum cannot wrap there).
struct UDiv {
  uint32_t m, l;
};
UDiv make_udiv(uint32_t d) {
  uint32_t l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  return UDiv{uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1), l};
}
__device__ __forceinline__ int udiv(int n, UDiv v) {
  return int((__umulhi(uint32_t(n), v.m) + uint32_t(n)) >> v.l);
}

struct MfmaArgs {
  AttnArgs a;
  int32_t group;     // Hq / Hkv
  int32_t rows;      // N * group query rows per unit
  int32_t n_kp;      // key phases: 1 (all eight wavefronts share every tile) or 2
  int32_t qrows;     // query rows per workgroup: 32 * 8 / n_kp
  int32_t qblocks;   // ceil(rows / qrows)
  int32_t splits;    // workgroups sharing one query block's keys
  int32_t xcd_map;   // keep the query blocks of one (unit, split) on one XCD
  int64_t o_offset;  // byte offset of the partial O in the workspace
  double log2_base;  // log2 of the RoPE base: frequency i is 2^(-(2i/d) log2 base)
  float rcp_group;               // rcp_up(group)
  UDiv div_qblocks, div_splits, div_hkv;  // make_udiv() of the divisors
};

struct MergeArgs {
  const float4* ml;  // [units][qblocks][splits][qrows] (m, l, s0, s1): largest |O / l| per half
  const unsigned char* o;  // O / (l s) as 16-bit fixed point, in the attention wavefronts' lane order
  void* out;
  const int32_t* status;
  int32_t Hq, Hkv, N, group, rows, qrows, qblocks, splits;
  float rcp_group;  // rcp_up(group)
  UDiv div_hkv;     // make_udiv(Hkv)
};


struct Plan {
  int32_t units, group, rows, n_kp, qrows, qblocks, splits;
  bool xcd_map;
  size_t o_offset, bytes;
};

static_assert(size_t(kTargetWGs) * (kRowsWave * kWaves / kKeyPhases) * (sizeof(float4) + kD * sizeof(int16_t)) <=
                  kAttnWorkspaceMax,
              "the split partials of the largest plan fit the stated workspace bound");

Plan make_plan(int32_t B, int32_t Hq, int32_t Hkv, int32_t d_h, int32_t N, int32_t S_max) {
  Plan p{};
  p.units = B * Hkv;
  p.group = Hq / Hkv;
  p.rows = N * p.group;
  p.n_kp = kKeyPhases;
  p.qrows = kRowsWave * kWaves / p.n_kp;
  p.qblocks = (p.rows + p.qrows - 1) / p.qrows;
  const int32_t wgs = p.units * p.qblocks;
  // one workgroup per compute unit at most: a second wave of workgroups would double the time
  int32_t splits = kTargetWGs / wgs;
  // at least four stages of tiles per split
  const int64_t tiles = (int64_t(S_max) - N + kTile - 1) / kTile + (N + kTile - 1) / kTile;
  const int64_t max_splits = tiles / (4 * p.n_kp);
  splits = splits < max_splits ? splits : int32_t(max_splits);
  p.splits = splits < 1 ? 1 : splits;
  p.xcd_map = p.qblocks > 1 && (int64_t(p.units) * p.splits) % 8 == 0;
  const size_t slots = size_t(p.units) * p.qblocks * p.splits * p.qrows;
  p.o_offset = (slots * sizeof(float4) + 255) / 256 * 256;
  p.bytes = p.splits > 1 ? p.o_offset + slots * size_t(d_h) * sizeof(int16_t) : 256;
  return p;
}

// Byte offset of (row, 16-byte chunk) in a 32 x 256-byte matrix.  Chunks are XOR-swizzled
// by a key that is a bijection over any 16 aligned rows (so the 16-byte K-operand reads
// of 16 rows hit 16 distinct bank groups of the 64-bank LDS) and whose high two bits differ
// within every aligned group of 4 rows (so the transposing V^T reads, 4 rows x 4 chunks per
// 32 lanes, do as well): both read patterns are free of bank conflicts.
__device__ __forceinline__ int swz_key(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 256 + ((chunk ^ swz_key(row)) << 4);
}

// Head dimension d_h = 64 runs on the same layout, padded to kD = 128: dims 0..31 of a row
// sit in the 16-byte chunks 0..3 and dims 32..63 in chunks 8..11, so that the RoPE pairs
// (i, i + d_h / 2) of the row are the layout's pairs (j, j + 64) and frequency j of the
// layout is that of pair i = j.  The other chunks are padding: the query rows hold zeros
// there (their products with any finite key add nothing), keys and values hold copies of
// real chunks, and the padded output dims are dropped.  src_chunk gives the chunk of the
// global row that a layout chunk is fetched from.
template <int kDH>
__device__ __forceinline__ int src_chunk(int c) {
  if constexpr (kDH == kD) return c;
  else return (c & 8) ? 4 + (c & 3) : (c & 3);
}
template <int kDH>
__device__ __forceinline__ bool real_chunk(int c) { return kDH == kD || (c & 4) == 0; }
// output dims of accumulator block db (32 layout dims), or -1 for a padded block
template <int kDH>
__device__ __forceinline__ int out_block(int db) { return kDH == kD ? 32 * db : ((db & 1) ? -1 : 16 * db); }

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
  const uint32_t m0v = uint32_t(__builtin_amdgcn_readfirstlane(lds));
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(m0v), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

// wait until at most n of this wavefront's vector memory operations are outstanding
// (n rounded down to an even count and capped at 30, which only makes the wait stricter)
__device__ __forceinline__ void wait_vm(int n) {
  switch (n >= 30 ? 15 : n >> 1) {
    case 15: asm volatile("s_waitcnt vmcnt(30)" ::: "memory"); break;
    case 14: asm volatile("s_waitcnt vmcnt(28)" ::: "memory"); break;
    case 13: asm volatile("s_waitcnt vmcnt(26)" ::: "memory"); break;
    case 12: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
    case 11: asm volatile("s_waitcnt vmcnt(22)" ::: "memory"); break;
    case 10: asm volatile("s_waitcnt vmcnt(20)" ::: "memory"); break;
    case 9: asm volatile("s_waitcnt vmcnt(18)" ::: "memory"); break;
    case 8: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
    case 7: asm volatile("s_waitcnt vmcnt(14)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}

// maxima without the canonicalising moves IEEE-mode fmaxf adds in front of MFMA results
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max2f(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Set-up loads issued as inline assembly: the compiler tracks no completion for them, so
// none of its own waits -- which would also wait for the tile loads issued after them --
// stands in front of their uses.  A value may be used only after a wait_vm that covers
// its load, and after pin(), which keeps the uses from moving above that wait.
__device__ __forceinline__ u32x4 load_b128(const void* p) {
  u32x4 v;
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(v) : "v"(p) : "memory");
  return v;
}
// the same, marked nontemporal (data read once)
__device__ __forceinline__ u32x4 load_b128_nt(const void* p) {
  u32x4 v;
  asm volatile("global_load_dwordx4 %0, %1, off nt" : "=v"(v) : "v"(p) : "memory");
  return v;
}
__device__ __forceinline__ u32x2 load_b64(const void* p) {
  u32x2 v;
  asm volatile("global_load_dwordx2 %0, %1, off" : "=v"(v) : "v"(p) : "memory");
  return v;
}
__device__ __forceinline__ uint32_t load_b32(const void* p) {
  uint32_t v;
  asm volatile("global_load_dword %0, %1, off" : "=v"(v) : "v"(p) : "memory");
  return v;
}
template <typename T>
__device__ __forceinline__ void pin(T& v) { asm volatile("" : "+v"(v)); }

template <int kDH>
__global__ __launch_bounds__(kThreads, 1) void tree_attn_mfma_kernel(MfmaArgs p) {
  const AttnArgs& a = p.a;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int half = lane >> 5, l32 = lane & 31;
  constexpr int n_kp = kKeyPhases;
  const int kp = wave % n_kp, rb = wave / n_kp;  // key phase, 32-row block

  // ---- this workgroup's (sequence, kv head, split, query block)
  // (selected, not branched on, so that the kernel arguments arrive in one round trip)
  const int bx = blockIdx.x, bq = p.xcd_map ? bx >> 3 : bx;
  const int sq = udiv(bq, p.div_qblocks);
  const int grp = p.xcd_map ? (bx & 7) + 8 * sq : sq;
  const int qb = bq - sq * p.qblocks;
  const int unit = udiv(grp, p.div_splits), split = grp - unit * p.splits;
  const int b = udiv(unit, p.div_hkv), kvh = unit - b * a.Hkv;
  const int N = a.N;
  const int n_stg = (N + kTile - 1) / kTile;

  __shared__ __attribute__((aligned(16))) unsigned char s_ring[kRing][kTileBytes];
  __shared__ float2 s_cs[kTableDepth][kD / 2 + 2];  // rows padded: lanes at other depths hit other banks
  __shared__ unsigned char s_dep[kDepthLds];
  __shared__ uint32_t s_mw[kWaves][kMaskLds][kRowsWave];
  __shared__ int s_bad[kWaves];

  // ---- set-up loads, independent of each other and issued together (as inline assembly,
  // see load_b128): every address is clamped into range instead of branching.  This
  // lane's query row is row0 + l32 of the unit: node u_q, head h_q.
  const int P = a.prefix_len[b];  // scalar
  const int row0 = qb * p.qrows + rb * kRowsWave;
  const int rq = row0 + l32;
  const bool live = rq < p.rows;
  const int uq0 = idiv(rq, p.rcp_group);
  const int u_q = live ? uq0 : 0;
  const int h_q = kvh * p.group + (live ? rq - __mul24(uq0, p.group) : 0);
  uint32_t st_word = load_b32(a.status);  // written by earlier kernels only: a plain load
  // The query inputs of the rotation below, straight into registers with the other set-up
  // loads: of this lane's row, the dim pairs its wavefront rotates (s = 2 kp + t, t < 2:
  // layout chunk 2 s + half and its partner 2 s + 8 + half), 16 bytes each.  Rows past the
  // block read the sequence's first row and are zeroed at the rotation, as are the padding
  // chunks of a 64-wide head.
  u32x4 qin[2][2];
  {
    const bf16* qrow = static_cast<const bf16*>(a.q) + ((int64_t(b) * N + u_q) * a.Hq + h_q) * kDH;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int c = 2 * (2 * kp + t) + half;
      qin[t][0] = load_b128(qrow + 8 * src_chunk<kDH>(c));
      qin[t][1] = load_b128(qrow + 8 * src_chunk<kDH>(c + 8));
    }
  }
  uint32_t dep_q_w = load_b32(a.depth + u_q);
  uint32_t dep0_w = load_b32(a.depth + min(tid, N - 1));
  uint32_t P_lane_w = load_b32(a.prefix_len + min(lane, a.B - 1));  // sequences 0..63, checked below
  // visibility of staged tiles 2k and 2k + 1 (nodes 64 k .. 64 k + 63) for this lane's node
  u32x2 mword[kMaskLds / 2];
#pragma unroll
  for (int k = 0; k < kMaskLds / 2; ++k)
    mword[k] = load_b64(a.mask + int64_t(u_q) * a.mask_words + min(k, a.mask_words - 1));

  // ---- key tiles of the unit: n_pre prefix tiles (the last one may be partial), then the
  // staged tiles.  Stage i of this split holds tiles (s_lo + i) * n_kp + k, k < n_kp, in
  // ring slot i % S.
  const int n_pre = (P + kTile - 1) / kTile;
  const int T = n_pre + n_stg;
  const int n_stages = (T + n_kp - 1) / n_kp;
  // Split boundaries: stages holding a partial or staged tile (masks, staged-row fixes, the
  // general path) count twice, so the last split, which holds them, gets fewer stages.
  const int n_heavy = n_stages - (P / kTile) / n_kp;
  auto bound = [&](int k) __attribute__((always_inline)) {
    const int64_t num = int64_t(k) * (n_stages + n_heavy);
    const int q = num <= INT32_MAX ? udiv(int(num), p.div_splits) : int(num / p.splits);
    return k == p.splits ? n_stages : min(n_stages, q);
  };
  const int s_lo = bound(split);
  const int n_st = bound(split + 1) - s_lo;
  constexpr int S = kRing / n_kp;  // stages in the ring
  auto tile_start = [&](int i) __attribute__((always_inline)) { return (s_lo + i) * n_kp; };
  auto tile_end = [&](int i) __attribute__((always_inline)) { return min(T, (s_lo + i + 1) * n_kp); };

  const int64_t head = (int64_t(b) * a.Hkv + kvh) * a.S_max * kDH;
  const bf16* kc = static_cast<const bf16*>(a.k_cache) + head;
  const bf16* vc = static_cast<const bf16*>(a.v_cache) + head;
  bf16* kc_w = static_cast<bf16*>(a.k_cache) + head;
  bf16* vc_w = static_cast<bf16*>(a.v_cache) + head;
  const bf16* kn = static_cast<const bf16*>(a.k_new) + (int64_t(b) * N * a.Hkv + kvh) * kDH;
  const bf16* vn = static_cast<const bf16*>(a.v_new) + (int64_t(b) * N * a.Hkv + kvh) * kDH;
  // LDS buffer of stage i's k-th tile: K at +0, V at +8192
  auto tbuf = [&](int i, int k) __attribute__((always_inline)) -> unsigned char* {
    return s_ring[(i & (S - 1)) * n_kp + k];
  };

  // Rows kDmaRows w .. kDmaRows (w + 1) - 1 of one tile's K and V by direct global->LDS
  // loads (wavefront w, kDmaOps instructions of four rows per matrix): in instruction h,
  // lane l lands at byte 256 kDmaRows w + 1024 h + 16 l of the matrix, i.e. row
  // kDmaRows w + 4 h + l / 16, stored chunk l % 16, and fetches logical chunk
  // (l % 16) ^ key(row), so that the buffer holds the layout swz() reads back.
  int rt_dma[kDmaOps], chunk_dma[kDmaOps];
  uint32_t poff[kDmaOps];
#pragma unroll
  for (int h = 0; h < kDmaOps; ++h) {
    rt_dma[h] = kDmaRows * wave + 4 * h + (lane >> 4);
    chunk_dma[h] = (lane & 15) ^ swz_key(rt_dma[h]);  // logical chunk this lane fetches
    poff[h] = uint32_t(rt_dma[h] * kDH * 2 + (src_chunk<kDH>(chunk_dma[h]) << 4));
  }
  auto issue_tile = [&](int t, unsigned char* buf) __attribute__((always_inline)) {
    const uint32_t lds = lds_addr(buf) + 256 * kDmaRows * wave;
    if ((t + 1) * kTile <= P) {  // full prefix tile
      const int64_t off = int64_t(t) * kTile * kDH;
#pragma unroll
      for (int h = 0; h < kDmaOps; ++h) {
        dma16(kc + off, poff[h], lds + 1024 * h);
        dma16(vc + off, poff[h], lds + 8192 + 1024 * h);
      }
    } else if (t < n_pre) {  // the partial prefix tile: rows past P repeat row 0
      const int64_t off = int64_t(t) * kTile * kDH;
#pragma unroll
      for (int h = 0; h < kDmaOps; ++h) {
        const int r = t * kTile + rt_dma[h] < P ? rt_dma[h] : 0;
        const uint32_t o = uint32_t(r * kDH * 2 + (src_chunk<kDH>(chunk_dma[h]) << 4));
        dma16(kc + off, o, lds + 1024 * h);
        dma16(vc + off, o, lds + 8192 + 1024 * h);
      }
    } else {  // staged rows from k_new / v_new; rows past the tree repeat node 0
#pragma unroll
      for (int h = 0; h < kDmaOps; ++h) {
        const int u = (t - n_pre) * kTile + rt_dma[h];
        const uint32_t o = uint32_t(((u < N ? u : 0) * a.Hkv * kDH + 8 * src_chunk<kDH>(chunk_dma[h])) * 2);
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
  // been issued (2 kDmaOps loads per tile).  In the steady state of the ring that is always
  // the same count, tested first so that the common case costs one compare.
  constexpr int kSteadyWait = 2 * kDmaOps * kKeyPhases * (kRing / kKeyPhases - 3);
  auto wait_stage = [&](int i, int last) __attribute__((always_inline)) {
    const int n = last > i ? 2 * kDmaOps * (tile_end(last) - tile_end(i)) : 0;
    if (n == kSteadyWait)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kSteadyWait) : "memory");
    else
      wait_vm(n);
  };

  // The tile loads of the first two stages need only P (a scalar load): issue them now,
  // behind the set-up loads, unless P is out of range (checked for every sequence below,
  // which then raises the error).  Their ring slots hold nothing else during the set-up;
  // the rest of the ring is filled once every wavefront has read its query operands from
  // the slots of stages 2 and 3.
  const bool ring_ok = P >= 0 && P <= a.S_max - N && n_st > 0;
  const int early = ring_ok ? min(2, n_st) : 0;  // stages issued now
  for (int i = 0; i < early; ++i) issue_stage(i);
  const int n_ring_loads = early > 0 ? 2 * kDmaOps * (tile_end(early - 1) - tile_start(0)) : 0;

  // ---- RoPE phases (cos, sin) of positions P + d: the angle is formed and reduced modulo
  // 2 pi in binary64, then evaluated in fp32.  The depths below kEarlyDepth need only P and
  // are formed while the set-up loads and the first stage's tiles are in flight, one entry
  // per thread: (d, tid % 64) with d = tid / 64.  Deeper phases, which few trees need, are
  // formed once the node depths are known.
  static_assert(kThreads == kEarlyDepth * (kD / 2), "one early phase entry per thread");
  // the rotated query operands (16 per row block, 16 bytes per lane) fit the slots of stages
  // 2 and 3, which are issued only once every wavefront has read them
  static_assert(kRing / kKeyPhases == 4 && (kWaves / kKeyPhases) * 16 * 64 * 16 <= 2 * kKeyPhases * kTileBytes,
                "query operands overlap the first two stages");
  const double theta = exp2(-double(tid % (kD / 2)) * (2.0 / kD) * p.log2_base);
  auto phase = [&](int d) __attribute__((always_inline)) {
    const double x = double(P + d) * theta;
    const double k = rint(x * kInvTwoPi);
    const float r = float(fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, x)));
    float sn, cs;
    sincosf(r, &sn, &cs);
    s_cs[d][tid % (kD / 2)] = make_float2(cs, sn);
  };
  phase(tid / (kD / 2));
  // the set-up loads are older than the ring's tile loads, which may stay in flight
  wait_vm(n_ring_loads);
  pin(st_word);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    pin(qin[t][0]);
    pin(qin[t][1]);
  }
  pin(dep_q_w);
  pin(dep0_w);
  pin(P_lane_w);
#pragma unroll
  for (int k = 0; k < kMaskLds / 2; ++k) pin(mword[k]);
  const int dep_q = int(dep_q_w), dep0 = int(dep0_w);
  const int64_t P_lane = int32_t(P_lane_w);
  if (st_word != 0) {  // an earlier step of the round failed
    wait_vm(0);        // no load may still target LDS when the block exits
    return;
  }
  if (half == 0) {
#pragma unroll
    for (int k = 0; k < kMaskLds; ++k) s_mw[wave][k][l32] = k < n_stg ? mword[k >> 1][k & 1] : 0u;
  }
  // every sequence's staged rows [P_b, P_b + N) must lie inside the cache; all blocks
  // evaluate the same condition, so that they all store or none does
  bool unfit = lane < a.B && (P_lane < 0 || P_lane + N > a.S_max);
  for (int b2 = 64 + lane; b2 < a.B; b2 += 64) {  // batches of more than 64 sequences
    const int64_t Pb = a.prefix_len[b2];
    unfit = unfit || Pb < 0 || Pb + N > a.S_max;
  }
  if (__ballot(unfit)) {
    wait_vm(0);
    if (blockIdx.x == 0 && tid == 0) raise_status(a.status, MEDUSA_ECAPACITY);
    return;
  }
  bool bad = tid < N && (dep0 < 0 || dep0 >= kTableDepth);
  bool deep = tid < N && dep0 >= kEarlyDepth;
  if (tid < N && tid < kDepthLds) s_dep[tid] = static_cast<unsigned char>(dep0);
  for (int i = tid + kThreads; i < N; i += kThreads) {  // trees of more than 512 nodes
    const int d = a.depth[i];
    bad = bad || d < 0 || d >= kTableDepth;
    deep = deep || d >= kEarlyDepth;
    if (i < kDepthLds) s_dep[i] = static_cast<unsigned char>(d);
  }

  // one flag word per wavefront (every lane votes): bit 0 a depth outside the table, bit 1
  // a depth beyond the phases formed so far
  const int wflags = (__ballot(bad) != 0 ? 1 : 0) | (__ballot(deep) != 0 ? 2 : 0);
  if (lane == 0) s_bad[wave] = wflags;
  __syncthreads();
  int flags = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) flags |= s_bad[w];
  if (flags & 1) {  // a node deeper than the phase table: uniform over the workgroup
    wait_vm(0);     // no load may still target LDS when the block exits
    if (blockIdx.x == 0 && tid == 0) raise_status(a.status, MEDUSA_EUNSUPPORTED);
    return;
  }
  if (flags & 2) {  // deep trees: the remaining phases
    for (int d = kEarlyDepth + tid / (kD / 2); d < kTableDepth; d += kThreads / (kD / 2)) phase(d);
    __syncthreads();
  }

  // ---- this wavefront's 32 query rows: rotated, scaled to log2 units, bf16 B operands;
  // lane holds query column l32, dims 16 s + 8 half + e (e < 8).  The two wavefronts of a row
  // block (its two key phases) share the rotation: wavefront kp rotates the dim pairs of
  // s = 2 kp, 2 kp + 1 (dims 16 s.. and their partners 64 + 16 s..) and leaves its hi and lo
  // operands in LDS, in the ring slots of stages 2 and 3 (issued only after the barrier
  // that follows the operand reads); after the barrier below each wavefront reads all
  // sixteen of its row block's operands.
  const float qscale = kLog2e / sqrtf(float(kDH));
  unsigned char* const q_ops = s_ring[2 * kKeyPhases] + rb * (16 * 64 * 16);  // [operand][lane] x 16 B
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int s = 2 * kp + t;
    const bool real = live && real_chunk<kDH>(2 * s + half);  // its partner chunk 2 s + 8 + half is alike
    const bf16x8 lo = __builtin_bit_cast(bf16x8, real ? qin[t][0] : u32x4{0u, 0u, 0u, 0u});
    const bf16x8 hi = __builtin_bit_cast(bf16x8, real ? qin[t][1] : u32x4{0u, 0u, 0u, 0u});
    bf16x8 h1, h2, l1, l2;
    // element pairs, so that each bf16 rounding is one packed conversion of two values
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      f32x2 r1, r2;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const float2 cs = s_cs[dep_q][16 * s + 8 * half + e + k];
        const float x1 = float(lo[e + k]), x2 = float(hi[e + k]);
        r1[k] = (x1 * cs.x - x2 * cs.y) * qscale;
        r2[k] = (x2 * cs.x + x1 * cs.y) * qscale;
      }
      const bf16x2 a1 = __builtin_convertvector(r1, bf16x2), a2 = __builtin_convertvector(r2, bf16x2);
      const bf16x2 b1 = __builtin_convertvector(r1 - __builtin_convertvector(a1, f32x2), bf16x2);
      const bf16x2 b2 = __builtin_convertvector(r2 - __builtin_convertvector(a2, f32x2), bf16x2);
      h1[e] = a1[0];
      h1[e + 1] = a1[1];
      h2[e] = a2[0];
      h2[e + 1] = a2[1];
      l1[e] = b1[0];
      l1[e + 1] = b1[1];
      l2[e] = b2[0];
      l2[e + 1] = b2[1];
    }
    // operand o: hi s = o, lo s = 8 + o
    *reinterpret_cast<u32x4*>(q_ops + (s * 64 + lane) * 16) = __builtin_bit_cast(u32x4, h1);
    *reinterpret_cast<u32x4*>(q_ops + ((s + 4) * 64 + lane) * 16) = __builtin_bit_cast(u32x4, h2);
    *reinterpret_cast<u32x4*>(q_ops + ((8 + s) * 64 + lane) * 16) = __builtin_bit_cast(u32x4, l1);
    *reinterpret_cast<u32x4*>(q_ops + ((12 + s) * 64 + lane) * 16) = __builtin_bit_cast(u32x4, l2);
  }
  __syncthreads();  // the row block's operands are in LDS
  bf16x8 qhi[8], qlo[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    qhi[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(q_ops + (s * 64 + lane) * 16));
    qlo[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(q_ops + ((8 + s) * 64 + lane) * 16));
  }

  // Staged rows of one tile that this wavefront loaded (rows kDmaRows w ..): rotate K in
  // place to P + depth(u); query block 0 also stores K~ and V to cache rows P + u.  Lane
  // l < 8 kDmaRows takes row kDmaRows w + l / 8 and the chunk pair (l % 8, l % 8 + 8),
  // i.e. dims j and j + 64.
  // Depths come from the LDS copy; trees too large for it read them from memory, in a
  // separate instantiation so that the common path carries no wait for that load.
  auto fix_staged = [&](int t, unsigned char* buf, auto depth_in_memory) __attribute__((always_inline)) {
    if (lane >= 8 * kDmaRows) return;
    const int rt = kDmaRows * wave + (lane >> 3), c = lane & 7;
    const int uu = (t - n_pre) * kTile + rt;
    const int u = uu < N ? uu : 0;
    const int dep = decltype(depth_in_memory)::value ? a.depth[u] : int(s_dep[u]);
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
    if (qb == 0 && uu < N && real_chunk<kDH>(c)) {  // layout chunks c, c + 8 hold dims 8 c.., d_h / 2 + 8 c..
      bf16* kd = kc_w + (int64_t(P) + uu) * kDH;
      bf16* vd = vc_w + (int64_t(P) + uu) * kDH;
      *reinterpret_cast<uint4*>(kd + 8 * c) = __builtin_bit_cast(uint4, rx);
      *reinterpret_cast<uint4*>(kd + 8 * c + kDH / 2) = __builtin_bit_cast(uint4, ry);
      *reinterpret_cast<uint4*>(vd + 8 * c) = *reinterpret_cast<const uint4*>(buf + 8192 + swz(rt, c));
      *reinterpret_cast<uint4*>(vd + 8 * c + kDH / 2) = *reinterpret_cast<const uint4*>(buf + 8192 + swz(rt, c + 8));
    }
  };
  // once stage i has landed: the staged tiles of the stage get their rows fixed
  auto fix_stage = [&](int i) __attribute__((always_inline)) {
    for (int k = 0; k < n_kp; ++k) {
      const int t = tile_start(i) + k;
      if (t >= n_pre && t < T) {
        if (N <= kDepthLds)
          fix_staged(t, tbuf(i, k), std::false_type{});
        else
          fix_staged(t, tbuf(i, k), std::true_type{});
      }
    }
  };

  // K operands of one tile for S^T = K Q^T, k-steps 4 kh .. 4 kh + 3: row l32, logical
  // chunk 2 st + half.  With the swizzle its byte offset is kbase ^ (32 st), kbase being
  // that of st = 0; the tile base (a multiple of 16 KiB) is added first, which leaves the
  // XORed bits alone and keeps the per-lane offsets from being hoisted out of the loop.
  const uint32_t kbase = uint32_t(swz(l32, half));
  auto read_k = [&](const unsigned char* tb, int kh, bf16x8 (&kop)[4]) __attribute__((always_inline)) {
    const uint32_t b = lds_addr(tb) + kbase;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t addr = b ^ uint32_t(32 * (4 * kh + j));
      kop[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const __attribute__((address_space(3))) uint4*>(addr));
    }
  };
  // S^T = K Q^T for one tile, k-steps 4 kh .. 4 kh + 3 (32 keys x 32 query columns)
  auto qk = [&](int kh, const bf16x8 (&kop)[4], f32x16& s) __attribute__((always_inline)) {
    if (kh == 0) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[j], qhi[4 * kh + j], s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[j], qlo[4 * kh + j], s, 0, 0, 0);
    }
  };
  // visibility bits of a tile's 32 keys for this lane's query row (bit m = key m of the
  // tile); all ones for a full prefix tile
  auto tile_bits = [&](int t) __attribute__((always_inline)) -> uint32_t {
    if (t < n_pre) {
      const int nvalid = P - t * kTile;
      return nvalid >= 32 ? 0xffffffffu : ((1u << nvalid) - 1u);
    }
    const int ks = t - n_pre;
    if (ks < kMaskLds) {
      // the lane index passes through an empty asm so that this rarely used address is
      // formed here, not kept (and spilled) across the loop
      int l = l32;
      asm volatile("" : "+v"(l));
      return s_mw[wave][ks][l];
    }
    // wide trees: read the word from memory (the wait for it also drains the tile ring)
    return uint32_t(a.mask[int64_t(u_q) * a.mask_words + (ks >> 1)] >> (32 * (ks & 1)));
  };

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // Per-lane LDS offsets of the V^T operand reads (in the V half of a tile buffer): lane
  // (gq, gi) supplies row key0 + 8 h, dims 32 db + 16 (gq % 2) + 4 (gi % 4) .. + 3.  The
  // chunk index is 4 db + c with c < 4 and the row's swizzle key is 4 (row % 4) + k, so the
  // swizzled offset is vbase[h] ^ (64 db) with vbase[h] that of db = 0; the 16-key step t2
  // adds 16 rows (4096 bytes).
  const int gq = lane >> 4, gi = lane & 15;
  uint32_t vbase[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int dim = 16 * (gq & 1) + 4 * (gi & 3);
    const int row = 4 * (gq >> 1) + (gi >> 2) + 8 * h;
    vbase[h] = uint32_t(8192 + swz(row, dim >> 3) + ((dim & 4) << 1));
  }
  // V^T operands of one tile for the 64 output dims of half dh: 32-dim block 2 dh + j,
  // 16-key step t2
  auto read_v = [&](const unsigned char* tb, int dh, bf16x8 (&vop)[2][2]) __attribute__((always_inline)) {
    const uint32_t t0 = lds_addr(tb);
    const uint32_t b0 = t0 + vbase[0], b1 = t0 + vbase[1];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t x = uint32_t(64 * (2 * dh + j));
      const uint32_t a0 = b0 ^ x, a1 = b1 ^ x;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(size_t(a0 + 4096 * t2)));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(size_t(a1 + 4096 * t2)));
        vop[j][t2] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
  };
  // O^T += V^T P^T for output half dh: k index 8 h + e of a 16-key step pairs with key
  // 16 t2 + 8 (e / 4) + 4 h + e % 4, exactly the order in which the score accumulator holds P
  auto pv = [&](int dh, const bf16x8 (&vop)[2][2], const bf16x8 (&pop)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
        oacc[2 * dh + j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[j][t2], pop[t2], oacc[2 * dh + j], 0, 0, 0);
  };

  // running-max update of one tile's scores; rescales O and l in the rare case it moves.
  // Returns the reference the probabilities are taken against.
  auto update_max = [&](const f32x16& sc) __attribute__((always_inline)) -> float {
    float x = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
#pragma unroll
    for (int e = 4; e < 16; e += 2) x = fmaxf(x, fmaxf(sc[e], sc[e + 1]));
    float y0, y1;
    halves(x, y0, y1);
    const float tmax = fmaxf(y0, y1);
    const bool grow = tmax > m_run + kRescaleSlack;
    if (__ballot(grow)) {
      const float m_new = grow ? tmax : m_run;
      const float corr = grow ? exp2_fast(m_run - m_new) : 1.0f;
      l_run *= corr;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] *= corr;
      m_run = m_new;
    }
    return m_run == -INFINITY ? 0.f : m_run;
  };
  // probabilities of one tile as the bf16 B operands of P^T; the row sum is taken over
  // the rounded values (the ones P V uses) with packed bf16 dot products
  auto probs = [&](const f32x16& sc, float m_use, bf16x8 (&pop)[2]) __attribute__((always_inline)) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ones = {static_cast<bf16>(1.0f), static_cast<bf16>(1.0f)};
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int e = 0; e < 8; ++e) pop[t2][e] = static_cast<bf16>(exp2_fast(sc[8 * t2 + e] - m_use));
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bf16x2 pr = {pop[t2][e], pop[t2][e + 1]};
        l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_run, false);
      }
  };

  // The key loop, instantiated twice: a row block past the unit's last query row (the upper
  // half of a 128-row block when a unit has 64 rows, e.g. one query head per kv head) still
  // loads its share of every tile, fixes its staged rows and keeps every barrier, but forms
  // no scores and no output.
  auto key_loop = [&](auto dead_tag) __attribute__((always_inline)) {
    constexpr bool kDead = decltype(dead_tag)::value;
    // prep: this wavefront's tile of stage i -- visibility bits and scores
    auto prep = [&](int i, f32x16& s, uint32_t& bits) __attribute__((always_inline)) {
      if constexpr (kDead) return;
      const int t = tile_start(i) + kp;
      if (t < T) {
        bits = tile_bits(t);
  #pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          bf16x8 kop[4];
          read_k(tbuf(i, kp), kh, kop);
          qk(kh, kop, s);
        }
      }
    };
    // consume: masking, softmax and PV of this wavefront's tile of stage i
    auto consume = [&](int i, f32x16& s, uint32_t bits) __attribute__((always_inline)) {
      if constexpr (kDead) return;
      const int t = tile_start(i) + kp;
      if (t >= T) return;
      if (t >= n_pre - 1) {  // the last prefix tile or a staged tile
        // element e holds key 8 (e / 4) + 4 half + e % 4; shifting by 4 half first leaves
        // compile-time bit positions
        const uint32_t bh = bits >> (4 * half);
  #pragma unroll
        for (int e = 0; e < 16; ++e)
          if (!((bh >> (8 * (e >> 2) + (e & 3))) & 1u)) s[e] = -INFINITY;
      }
      const float m_use = update_max(s);
      bf16x8 pop[2];
      probs(s, m_use, pop);
  #pragma unroll
      for (int dh = 0; dh < 2; ++dh) {
        bf16x8 vop[2][2];
        read_v(tbuf(i, kp), dh, vop);
        pv(dh, vop, pop);
      }
    };
    // one step: publish stage i+1 and refill the slot of stage i-1, form the scores of
    // stage i+1 on the matrix core, then finish stage i
    auto step = [&](int i, f32x16& s_cur, uint32_t& b_cur, f32x16& s_nxt, uint32_t& b_nxt)
        __attribute__((always_inline)) {
      if (i + 1 < n_st) {
        wait_stage(i + 1, min(i + S - 2, n_st - 1));
        fix_stage(i + 1);
        __syncthreads();  // stage i+1 visible; every wavefront is done with stage i-1
        if (i + S - 1 < n_st) issue_stage(i + S - 1);
        prep(i + 1, s_nxt, b_nxt);
      }
      consume(i, s_cur, b_cur);
    };

    f32x16 s_cur, s_nxt;
    uint32_t b_cur = 0u, b_nxt = 0u;
    const int first = min(S - 1, n_st);  // stages in flight ahead of the loop
    if (n_st > 0) {
      wait_stage(0, early - 1);
      fix_stage(0);
      __syncthreads();  // stage 0 visible; every wavefront has read its query operands
      for (int i = early; i < first; ++i) issue_stage(i);  // fill the rest of the ring but one slot
      prep(0, s_cur, b_cur);
    }

    // Steady state.  Step i is steady when every tile it touches -- those of stages i and
    // i+1 and those of stage i+S-1, which it issues -- is a full prefix tile (index below
    // P / kTile) and the ring is full.  Such steps need no tile classification, masks,
    // staged-row fixes or variable waits, and their load addresses advance by a fixed
    // stride, so they run as a separate loop with as few instructions as possible.  The
    // remaining steps (the ring's drain, partial and staged tiles) take the general path.
    // stages of this split whose tiles are all full prefix tiles; a step over two of them
    // needs no masks, and while the stage it issues is one of them its loads advance by a
    // fixed stride with a fixed wait; the ring's drain issues through issue_stage()
    const int n_full = max(0, min(n_st, (P / kTile) / n_kp - s_lo));
    const int fast_end = max(0, n_full - 1);
    const int hot_end = max(0, n_full - S + 1);
    int i = 0;
    if (fast_end > 0) {
      // The running maximum is checked at the end of each step, on the scores just formed,
      // and moved (rarely) before they are used.
      if constexpr (!kDead) update_max(s_cur);
      f32x16 zero;
  #pragma unroll
      for (int e = 0; e < 16; ++e) zero[e] = 0.f;
      // global addresses of the tiles of stage S-1 (issued by step 0); lane offsets in poff[]
      const bf16* kq = kc + int64_t((s_lo + S - 1) * n_kp) * kTile * kDH;
      const bf16* vq = vc + int64_t((s_lo + S - 1) * n_kp) * kTile * kDH;
      const uint32_t ring0 = lds_addr(&s_ring[0][0]) + 256 * kDmaRows * wave;
      auto steady = [&](int j, f32x16& sc, f32x16& sn, auto fixed) __attribute__((always_inline)) {
        if constexpr (decltype(fixed)::value) {
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kSteadyWait) : "memory");
          __syncthreads();  // stage j+1 visible; every wavefront is done with stage j-1
          const uint32_t dst = ring0 + uint32_t(((j + S - 1) & (S - 1)) * n_kp * kTileBytes);
  #pragma unroll
          for (int k = 0; k < n_kp; ++k)
  #pragma unroll
            for (int h = 0; h < kDmaOps; ++h) {
              dma16(kq + k * kTile * kDH, poff[h], dst + k * kTileBytes + 1024 * h);
              dma16(vq + k * kTile * kDH, poff[h], dst + k * kTileBytes + 8192 + 1024 * h);
            }
          kq += n_kp * kTile * kDH;
          vq += n_kp * kTile * kDH;
        } else {
          wait_stage(j + 1, min(j + S - 2, n_st - 1));
          __syncthreads();
          if (j + S - 1 < n_st) issue_stage(j + S - 1);
        }
        if constexpr (kDead) return;
        const unsigned char* tn = s_ring[((j + 1) & (S - 1)) * n_kp + kp];
        const unsigned char* tc = s_ring[(j & (S - 1)) * n_kp + kp];
        // the operand reads of the step: the first half of the K operands and every V operand
        // up front, the second half of the K operands once the first half is in use (the
        // query rows, carried as a hi/lo pair, leave no room for all of them at once)
        bf16x8 kop[4], vop[2][2][2];
        read_k(tn, 0, kop);
        read_v(tc, 0, vop[0]);
        read_v(tc, 1, vop[1]);
        // probabilities of tile j against the running maximum
        bf16x8 pop[2];
        probs(sc, m_run, pop);
        // scores of tile j+1
  #pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          if (kh == 1) read_k(tn, 1, kop);
  #pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[jj], qhi[4 * kh + jj], kh == 0 && jj == 0 ? zero : sn, 0, 0, 0);
            sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[jj], qlo[4 * kh + jj], sn, 0, 0, 0);
          }
        }
        pv(0, vop[0], pop);
        pv(1, vop[1], pop);
        // maximum of tile j+1; the reference moves when it exceeds the slack
        float x0 = max3f(sn[0], sn[1], sn[2]), x1 = max3f(sn[3], sn[4], sn[5]);
        float x2 = max3f(sn[6], sn[7], sn[8]), x3 = max3f(sn[9], sn[10], sn[11]);
        float x4 = max3f(sn[12], sn[13], sn[14]);
        x0 = max3f(x0, x1, x2);
        x3 = max3f(x3, x4, sn[15]);
        x0 = max2f(x0, x3);
        float y0, y1;
        halves(x0, y0, y1);
        const float tmax = max2f(y0, y1);
        const bool grow = tmax > m_run + kRescaleSlack;
        if (__ballot(grow)) {
          const float m_new = grow ? tmax : m_run;
          const float corr = exp2_fast(m_run - m_new);
          l_run *= corr;
  #pragma unroll
          for (int db = 0; db < 4; ++db)
  #pragma unroll
            for (int e = 0; e < 16; ++e) oacc[db][e] *= corr;
          m_run = m_new;
        }
      };
      // unrolled twice so that the two score tiles trade places without copies
      auto run = [&](int end, auto fixed) __attribute__((always_inline)) {
        for (; i + 2 <= end; i += 2) {
          steady(i, s_cur, s_nxt, fixed);
          steady(i + 1, s_nxt, s_cur, fixed);
        }
        if (i < end) {
          steady(i, s_cur, s_nxt, fixed);
          s_cur = s_nxt;
          ++i;
        }
      };
      run(hot_end, std::true_type{});
      run(fast_end, std::false_type{});
      b_cur = 0xffffffffu;  // the current tile is a full prefix tile
    }
    // the remaining steps: the end of the ring, partial and staged tiles
    for (; i < n_st; ++i) {
      step(i, s_cur, b_cur, s_nxt, b_nxt);
      s_cur = s_nxt;
      b_cur = b_nxt;
    }

  };
  if (row0 >= p.rows)
    key_loop(std::true_type{});
  else
    key_loop(std::false_type{});

  // ---- combine the key phases.  The two wavefronts of a row block split the work: wavefront
  // kp keeps the output dims of accumulator blocks 2 kp and 2 kp + 1 and hands its partner
  // the other two blocks and its (m, l) through LDS; each then combines and stores its half.
  float lsum;
  {
    float y0, y1;
    halves(l_run, y0, y1);
    lsum = y0 + y1;
  }
  static_assert(kKeyPhases == 2, "the epilogue combines two key phases");
  __syncthreads();  // every wavefront is done with the ring
  {
    float* give = reinterpret_cast<float*>(&s_ring[0][0]) + (2 * rb + kp) * (32 * 64 + 2 * 64);
    const float* take = reinterpret_cast<const float*>(&s_ring[0][0]) + (2 * rb + (kp ^ 1)) * (32 * 64 + 2 * 64);
    // (16-byte pieces: four values of a lane side by side, so that the exchange takes 8 LDS
    // writes and reads per lane rather than 32)
    float4* const give4 = reinterpret_cast<float4*>(give);
    const float4* const take4 = reinterpret_cast<const float4*>(take);
    auto hand_over = [&](auto first) __attribute__((always_inline)) {  // blocks first, first + 1
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x16& v = oacc[decltype(first)::value + j];
          give4[(j * 4 + q) * 64 + lane] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
        }
    };
    if (kp == 0)
      hand_over(std::integral_constant<int, 2>{});
    else
      hand_over(std::integral_constant<int, 0>{});
    give[32 * 64 + lane] = m_run;
    give[32 * 64 + 64 + lane] = lsum;
    __syncthreads();
    const float m1 = take[32 * 64 + lane], l1 = take[32 * 64 + 64 + lane];
    const float M = fmaxf(m_run, m1);
    const float w0 = m_run == -INFINITY ? 0.f : exp2_fast(m_run - M);
    const float w1 = m1 == -INFINITY ? 0.f : exp2_fast(m1 - M);
    lsum = w0 * lsum + w1 * l1;
    m_run = M;
    auto combine = [&](auto first) __attribute__((always_inline)) {  // blocks first, first + 1
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 t = take4[(j * 4 + q) * 64 + lane];
          f32x16& v = oacc[decltype(first)::value + j];
          v[4 * q] = w0 * v[4 * q] + w1 * t.x;
          v[4 * q + 1] = w0 * v[4 * q + 1] + w1 * t.y;
          v[4 * q + 2] = w0 * v[4 * q + 2] + w1 * t.z;
          v[4 * q + 3] = w0 * v[4 * q + 3] + w1 * t.w;
        }
    };
    if (kp == 0)
      combine(std::integral_constant<int, 0>{});
    else
      combine(std::integral_constant<int, 2>{});
  }

  // ---- results: lane (half, l32) holds, for query row row0 + l32, dims
  // 32 db + 8 g + 4 half + 0..3 in oacc[db][4 g .. 4 g + 3]; this wavefront stores blocks
  // 2 kp and 2 kp + 1
  if (p.splits == 1) {
    if (!live) return;
    bf16* o = static_cast<bf16*>(a.out) + ((int64_t(b) * N + u_q) * a.Hq + h_q) * kDH + 4 * half;
    const float inv = 1.0f / lsum;
    auto store = [&](auto first) __attribute__((always_inline)) {
#pragma unroll
      for (int db = decltype(first)::value; db < decltype(first)::value + 2; ++db) {
        if (out_block<kDH>(db) < 0) continue;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16& v = oacc[db];
          const bf16x4 ov = {static_cast<bf16>(v[4 * g] * inv), static_cast<bf16>(v[4 * g + 1] * inv),
                             static_cast<bf16>(v[4 * g + 2] * inv), static_cast<bf16>(v[4 * g + 3] * inv)};
          *reinterpret_cast<bf16x4*>(o + out_block<kDH>(db) + 8 * g) = ov;
        }
      }
    };
    if (kp == 0)
      store(std::integral_constant<int, 0>{});
    else
      store(std::integral_constant<int, 2>{});
    return;
  }
  // Partial of a split: (m, l, s0, s1) in fp32 and O / l as 16-bit fixed point relative to s0
  // for the dims of blocks 0 and 1 and to s1 for those of blocks 2 and 3: the row's largest
  // |O / l| over each half (v_cvt_pknorm_i16_f32: round(x 32767) of x in [-1, 1]), i.e. to
  // within 2^-16 s of each value -- well inside the bf16 rounding of the output (2^-9 of |o|)
  // and half the bytes of fp32 partials, which every split writes and the merge reads back.
  // A split that saw no key of the row stores l = s = 0.
  // The O part is kept in lane order: wavefront (rb, kp) of the workgroup owns d_h / 32 KiB in
  // which lane L's 16-byte piece i sits at 1024 i + 16 L, so that each store instruction
  // writes one whole KiB straight from registers (and the merge kernel, one thread per lane
  // of a wavefront, reads it back the same way).  Row blocks past the unit's last query row
  // store nothing.
  if (row0 >= p.rows) return;
  const int64_t pgrp = (int64_t(unit) * p.qblocks + qb) * p.splits + split;  // (unit, query block, split)
  float* rec = reinterpret_cast<float*>(static_cast<float4*>(a.workspace) + pgrp * p.qrows + rb * kRowsWave + l32);
  constexpr int kPieces = kDH / 32;  // 16-byte pieces per lane
  unsigned char* const dst = static_cast<unsigned char*>(a.workspace) + p.o_offset +
                             ((pgrp * (p.qrows / kRowsWave) + rb) * 2 + kp) * (kPieces * 1024) + 16 * lane;
  auto store_partial = [&](auto first) __attribute__((always_inline)) {
    constexpr int f = decltype(first)::value;
    float amax = 0.f;  // largest |O| of this lane's dims of the half, then of the row's (two lanes)
#pragma unroll
    for (int db = f; db < f + 2; ++db) {
      if (out_block<kDH>(db) < 0) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) amax = max2f(amax, fabsf(oacc[db][e]));
    }
    {
      float y0, y1;
      halves(amax, y0, y1);
      amax = max2f(y0, y1);
    }
    if (half == 0) {
      if (f == 0) *reinterpret_cast<float2*>(rec) = make_float2(m_run, lsum);
      rec[2 + f / 2] = lsum > 0.f ? amax / lsum : 0.f;
    }
    const float k = amax > 0.f ? 1.0f / amax : 0.f;
#pragma unroll
    for (int db = f; db < f + 2; ++db) {
      if (out_block<kDH>(db) < 0) continue;
      const f32x16& v = oacc[db];
      // piece (db - f) 2 + j of a 128-wide head, j of a 64-wide one: dims
      // 32 db + 8 g + 4 half + 0..3 for g = 2 j and 2 j + 1
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        u32x4 pc;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int g = 2 * j + t;
          pc[2 * t] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pknorm_i16(v[4 * g] * k, v[4 * g + 1] * k));
          pc[2 * t + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pknorm_i16(v[4 * g + 2] * k, v[4 * g + 3] * k));
        }
        const int i = kDH == kD ? (db - f) * 2 + j : j;
        // (nontemporal: the partial is read once, by the merge kernel, mostly on another XCD)
        __builtin_nontemporal_store(pc, reinterpret_cast<u32x4*>(dst + 1024 * i));
      }
    }
  };
  if (kp == 0)
    store_partial(std::integral_constant<int, 0>{});
  else
    store_partial(std::integral_constant<int, 2>{});
}

// Merge of the splits, one thread per 16-byte piece of an attention wavefront's partial: in
// the block for wavefront (rb, kp), thread (ph, L) combines, for query row rb 32 + L % 32 of
// the query block, the eight dims of piece ph of that wavefront's lane L (layout dims
// 32 db + 8 g + 4 (L / 32) + 0..3 for g = 2 (ph % 2), 2 (ph % 2) + 1 of block db = 2 kp + ph / 2),
// weighting split s by l_s 2^(m_s - M).  The splits are visited kGroup at a time (four when
// there are at most four, else eight) with every load of a group issued before any is used,
// so that a thread waits for memory once per group rather than once per split.
// Grid: x = unit, y = query block, z = 2 rb + kp; 64 d_h / 32 threads.  Every index comes from
// the launch coordinates without a division by a run-time value.
template <int kGroup, int kDH>
__global__ __launch_bounds__(64 * (kDH / 32)) void tree_attn_merge_kernel(MergeArgs p) {
  const bool failed = round_failed(p.status);  // gates the store only
  const int lane = int(threadIdx.x) & 63, l32 = lane & 31, half = lane >> 5, ph = int(threadIdx.x) >> 6;
  const int unit = int(blockIdx.x), qb = int(blockIdx.y), rb = int(blockIdx.z) >> 1, kp = int(blockIdx.z) & 1;
  const int row0 = qb * p.qrows + rb * kRowsWave;  // the wavefront's first query row
  if (row0 >= p.rows) return;                        // a row block past the last query row
  constexpr int kPieces = kDH / 32, kPer = 1;  // pieces per lane, per thread
  const int64_t grp0 = (int64_t(unit) * p.qblocks + qb) * p.splits;  // (unit, query block, split 0)
  float M = -INFINITY, L = 0.f;
  float acc[kPer][8];
#pragma unroll
  for (int i = 0; i < kPer; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
  for (int s0 = 0; s0 < p.splits; s0 += kGroup) {
    // issued as inline assembly, every load of the group back to back and then one wait:
    // left to itself the compiler waits for each split's load before it issues the next
    u32x4 mlw[kGroup], v[kGroup][kPer];
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {  // slots past the last split re-read split 0
      const int64_t g = grp0 + (s0 + k < p.splits ? s0 + k : 0);
      mlw[k] = load_b128_nt(p.ml + g * p.qrows + rb * kRowsWave + l32);
      const unsigned char* src =
          p.o + ((g * (p.qrows / kRowsWave) + rb) * 2 + kp) * (kPieces * 1024) + 1024 * (kPer * ph) + 16 * lane;
#pragma unroll
      for (int i = 0; i < kPer; ++i) v[k][i] = load_b128_nt(src + 1024 * i);
    }
    wait_vm(0);
    float4 ml[kGroup];  // (m, l, s0, s1)
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      pin(mlw[k]);
#pragma unroll
      for (int i = 0; i < kPer; ++i) pin(v[k][i]);
      ml[k] = make_float4(__uint_as_float(mlw[k][0]), __uint_as_float(mlw[k][1]), __uint_as_float(mlw[k][2]),
                          __uint_as_float(mlw[k][3]));
    }
    float Mg = M;
#pragma unroll
    for (int k = 0; k < kGroup; ++k)
      if (s0 + k < p.splits) Mg = fmaxf(Mg, ml[k].x);
    // rescale what the earlier groups accumulated, then add this group
    const float c = M == -INFINITY ? 0.f : exp2_fast(M - Mg);
    L *= c;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[i][e] *= c;
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      const float wt = (s0 + k < p.splits && ml[k].x != -INFINITY) ? ml[k].y * exp2_fast(ml[k].x - Mg) : 0.f;
      L += wt;
      // weight of one fixed-point step: dims of blocks 0, 1 are relative to s0, the rest to s1
      const float cw = wt * (kp == 0 ? ml[k].z : ml[k].w) * (1.0f / 32767.0f);
#pragma unroll
      for (int i = 0; i < kPer; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int32_t q = int32_t(int16_t(v[k][i][e >> 1] >> (16 * (e & 1))));
          acc[i][e] += cw * float(q);
        }
    }
    M = Mg;
  }
  if (failed) return;
  // The wavefront's 32 rows x d_h / 2 dims go through LDS (rows padded by 8 bytes, so that the
  // lanes' 8-byte writes down a column spread over the banks) and leave as whole 16-byte pieces,
  // d_h / 16 threads per row: every store instruction writes whole row halves rather than 8
  // bytes on each of 32 rows.
  constexpr int kHalfDims = kDH / 2, kStride = kHalfDims * 2 + 8, kChunks = kHalfDims / 8;
  __shared__ __attribute__((aligned(16))) unsigned char tile[kRowsWave * kStride];
  const float inv = 1.0f / L;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int ig = kPer * ph + i;  // the piece of the lane
    const int db = kDH == kD ? 2 * kp + ig / 2 : 2 * kp;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int g = 2 * (ig & 1) + t;
      const bf16x4 ov = {static_cast<bf16>(acc[i][4 * t] * inv), static_cast<bf16>(acc[i][4 * t + 1] * inv),
                         static_cast<bf16>(acc[i][4 * t + 2] * inv), static_cast<bf16>(acc[i][4 * t + 3] * inv)};
      const int d = out_block<kDH>(db) - kHalfDims * kp + 8 * g + 4 * half;  // dim within the half
      *reinterpret_cast<bf16x4*>(tile + l32 * kStride + 2 * d) = ov;
    }
  }
  __syncthreads();
  const int b = udiv(unit, p.div_hkv), kvh = unit - b * p.Hkv;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int id = int(threadIdx.x) + 64 * kPieces * q, r = id / kChunks, c = id % kChunks;
    const u32x4 v = *reinterpret_cast<const u32x4*>(tile + r * kStride + 16 * c);
    const int rr = row0 + r;
    if (rr >= p.rows) continue;
    const int u = idiv(rr, p.rcp_group);
    const int h = kvh * p.group + (rr - u * p.group);
    bf16* o = static_cast<bf16*>(p.out) + ((int64_t(b) * p.N + u) * p.Hq + h) * kDH + kHalfDims * kp + 8 * c;
    *reinterpret_cast<u32x4*>(o) = v;
  }
}


}  // namespace

bool mfma_path_applies(medusa_dtype dt, int32_t Hq, int32_t Hkv, int32_t d_h, int32_t N) {
  if (dt != MEDUSA_BF16 || (d_h != kD && d_h != kD / 2)) return false;
  // one sequence's query rows are addressed with 32-bit byte offsets
  if (int64_t(N) * Hq * d_h * 2 > int64_t(UINT32_MAX)) return false;
  // query rows (those of the last query block included) stay in idiv()'s range
  const int64_t qrows = kRowsWave * kWaves / kKeyPhases;
  const int64_t rows = int64_t(N) * (Hq / Hkv), qblocks = (rows + qrows - 1) / qrows;
  return qblocks * qrows < kFastDivMax;
}

size_t attn_workspace_bytes(medusa_dtype dt, int32_t B, int32_t Hq, int32_t Hkv, int32_t d_h,
                            int32_t N, int32_t S_max) {
  if (B < 1 || Hkv < 1 || Hq < 1 || N < 1 || S_max < N) return 0;
  if (!mfma_path_applies(dt, Hq, Hkv, d_h, N)) return 256;
  return make_plan(B, Hq, Hkv, d_h, N, S_max).bytes;
}

medusa_status run_mfma(AttnArgs& a, int32_t d_h, hipStream_t stream, void* ev_start, void* ev_stop) {
  const Plan plan = make_plan(a.B, a.Hq, a.Hkv, d_h, a.N, a.S_max);
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
  // the layout's frequency j is base^(-2 j / d_h): pair i = j of the head's RoPE
  p.log2_base = std::log2(a.rope_base) * (double(kD) / d_h);
  p.rcp_group = rcp_up(plan.group);
  p.div_qblocks = make_udiv(uint32_t(plan.qblocks));
  p.div_splits = make_udiv(uint32_t(plan.splits));
  p.div_hkv = make_udiv(uint32_t(a.Hkv));
  const unsigned grid = unsigned(int64_t(plan.units) * plan.splits * plan.qblocks);
  const bool full = d_h == kD;
  const void* attn = full ? reinterpret_cast<const void*>(&tree_attn_mfma_kernel<kD>)
                          : reinterpret_cast<const void*>(&tree_attn_mfma_kernel<kD / 2>);
  if (plan.splits == 1) return launch(attn, dim3(grid), dim3(kThreads), 0, stream, p, ev_start, ev_stop);
  const medusa_status st = launch(attn, dim3(grid), dim3(kThreads), 0, stream, p, ev_start, nullptr);
  if (st != MEDUSA_OK) return st;
  MergeArgs m{};
  m.ml = static_cast<const float4*>(a.workspace);
  m.o = static_cast<const unsigned char*>(a.workspace) + plan.o_offset;
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
  m.rcp_group = rcp_up(plan.group);
  m.div_hkv = make_udiv(uint32_t(a.Hkv));
  const void* merge =
      full ? (plan.splits <= 4 ? reinterpret_cast<const void*>(&tree_attn_merge_kernel<4, kD>)
                               : reinterpret_cast<const void*>(&tree_attn_merge_kernel<8, kD>))
           : (plan.splits <= 4 ? reinterpret_cast<const void*>(&tree_attn_merge_kernel<4, kD / 2>)
                               : reinterpret_cast<const void*>(&tree_attn_merge_kernel<8, kD / 2>));
  static_assert(kRowsWave * kWaves / kKeyPhases == 4 * kRowsWave && kKeyPhases == 2,
                "one merge block per attention wavefront: 4 row blocks x 2 key phases");
  return launch(merge, dim3(unsigned(plan.units), unsigned(plan.qblocks), unsigned(2 * (plan.qrows / kRowsWave))),
                dim3(unsigned(64 * (d_h / 32))), 0, stream, m, nullptr, ev_stop);
}

}  // namespace medusa
