/*
 * medusa.h -- C ABI of one Medusa tree-verification round on an MI355X (gfx950).
 *
 * A round has four steps, one entry point each:
 *   medusa_tree_compile  host:   rank-path tree -> flattened buffers (once per tree)
 *   medusa_tree_attn     device: RoPE at P+depth, staged K/V rows, tree attention
 *   medusa_accept        device: greedy longest-prefix acceptance
 *   medusa_kv_compact    device: gather the winning path's K/V rows into the cache
 * and, around them:
 *   medusa_accept_typical   device: typical acceptance instead of greedy
 *   medusa_accept_commit    device: greedy acceptance, compaction and the frontier carry
 *                           in one call
 *   medusa_head_candidates  device: the Medusa heads' top-k candidate rows
 *   medusa_tree_budget      host:   the node budget with the most tokens per unit time
 *
 * Pages cited (by title and section):
 *   [M7.2]  "M7.2 - Medusa: Multi-Head Candidates, Tree Attention, and Verification"
 *   [Chai]  "Medusa 完全拆解：多头树式候选如何用一次验证解码多个 Token"
 *   [PartII] "Medusa Part II: Candidate Trees, Verification, and Acceptance"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Ownership: the caller owns every buffer.  The library allocates no device
 *   memory and keeps no global mutable state; calls are re-entrant.
 * Pointers: "device" pointers are HIP device allocations on the current
 *   device; "host" pointers are ordinary host memory.  All tensors are dense,
 *   row-major (last index fastest), without padding.
 * Streams: device work is enqueued on `stream` (a hipStream_t; NULL = the
 *   null stream) and ordered with the caller's other work on it.  No call
 *   synchronises the host.
 * Errors: a negative medusa_status returned by a call means nothing was
 *   launched and no buffer was touched.  Conditions that only the device can
 *   see (values held in device memory) are reported through the device word
 *   `d_status` (int32, device): kernels leave it unchanged on success; on a
 *   violation they store a negative medusa_status code and perform no store to
 *   any output, cache or length buffer.  `d_status` is sticky: every device
 *   entry point first reads it and does nothing when it is non-zero, so one
 *   failed step voids the rest of the round.  The caller zeroes it before a
 *   round and reads it when it needs to know.
 * Timing: `ev_start` / `ev_stop` are optional hipEvent_t handles (NULL to
 *   skip).  When given, they are recorded at the start of the call's first
 *   kernel and at the end of its last kernel, from the kernel dispatch itself.
 */
#ifndef MEDUSA_H
#define MEDUSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MEDUSA_OK = 0,
  MEDUSA_EINVAL = -1,             /* malformed argument, shape, index or NaN input */
  MEDUSA_ENOT_PREFIX_CLOSED = -2, /* a path is present without one of its prefixes */
  MEDUSA_ECAPACITY = -3,          /* a budget or cache capacity is exceeded */
  MEDUSA_EUNSUPPORTED = -4,       /* valid but not implemented (head size, dtype, group) */
  MEDUSA_EBUFSIZE = -5,           /* a caller buffer or workspace is too small */
  MEDUSA_EHIP = -6                /* the HIP runtime refused a launch */
} medusa_status;

typedef enum { MEDUSA_F32 = 0, MEDUSA_BF16 = 1 } medusa_dtype;

/* ------------------------------------------------------------------ tree compile
 *
 * [M7.2] §0x04A "Sparse Tree Construction": a tree is a prefix-closed set of
 * rank paths (r_1..r_d), "rank r_i of head i-1 at depth i".  Non-root paths are
 * sorted by (length, path); row 0 is the LM root and row(p) = 1 + index.
 * Every buffer below is a function of that row:
 *   tree_indices[row(p)] = 1 + (len(p)-1)*topk + p[-1], tree_indices[0] = 0
 *       (candidate slot, [M7.2] §0x01B: slot(j,r) = 1 + j*TOPK + r)
 *   depth[u] = len(path(u)); the logical position is prefix_len + depth[u]
 *   parent[u] = row of path(u) without its last rank; parent[0] = -1
 *   tree_mask bit v of row u set iff path(v) is a prefix of path(u)
 *       (reflexive; the root is visible to every row)
 *   retrieve_indices: one row per maximal path (a leaf), leaves in ascending
 *       row order, [0, row(p[:1]), ..., row(p)] padded with -1 to
 *       path_width = max depth + 1.
 *
 * Two ways to name the tree (exactly one):
 *  A. explicit paths: n_paths paths, path_len[i] ranks each, ranks
 *     concatenated in path_ranks.  Any order; validated for 1 <= len <= num_heads,
 *     0 <= rank < topk, no duplicates, prefix closure.
 *  B. greedy growth ([M7.2] §0x04B/§0x04C; [PartII] Part 3): path_len == NULL,
 *     rank_hit = a[num_heads*topk] (row-major by head; a[k*topk+i] = probability
 *     that head k's rank-i token is the exact hit, each in [0,1]) and n_nodes =
 *     rows including the root.  Starting from the depth-1 paths, the path with
 *     the largest weight w(p) = a[0][p0]*a[1][p1]*... (binary64, left to right)
 *     whose parent is present is admitted until n_nodes-1 paths are in; ties go
 *     to the shorter path, then the lexicographically smaller one.
 *
 * Outputs (host buffers owned by the caller).  Call once with every output
 * pointer NULL: the sizes are written to n_nodes, n_paths, path_width and
 * mask_words (= ceil(n_nodes/64)) and nothing else happens.  On the second
 * call those four fields must hold the capacities of the caller's buffers
 * (rows, paths, width, words); MEDUSA_EBUFSIZE if any is smaller than needed.
 * Layouts: tree_indices, depth, parent: int32[n_nodes]; tree_mask:
 * uint64[n_nodes][mask_words] with bit (v % 64) of word (v / 64) in row u;
 * retrieve_indices: int32[n_paths][path_width]; node_weight (optional, mode B,
 * may be NULL): double[n_nodes] with w(root) = 1.
 *
 * Errors: MEDUSA_EINVAL (bad field, rank/length out of range, duplicate, rank_hit
 * outside [0,1] or NaN, n_nodes < 1), MEDUSA_ENOT_PREFIX_CLOSED, MEDUSA_ECAPACITY
 * (mode B: n_nodes-1 exceeds the number of rank tuples or n_nodes > 16384; mode
 * A: 16384 or more explicit paths, i.e. more than 16384 rows; either mode: host
 * memory for the search or the tree runs out), MEDUSA_EBUFSIZE.  No exception
 * leaves the call.
 */
typedef struct {
  int32_t num_heads;           /* K: Medusa heads = maximum depth, >= 1 */
  int32_t topk;                /* TOPK: candidate pool width per head, >= 1 */
  int32_t n_paths;             /* mode A: number of explicit paths (may be 0) */
  const int32_t* path_len;     /* mode A: [n_paths]; NULL selects mode B */
  const int32_t* path_ranks;   /* mode A: concatenated ranks, sum(path_len) entries */
  const double* rank_hit;      /* mode B: [num_heads*topk] */
  int32_t n_nodes;             /* mode B: rows including the root, >= 1 */
} medusa_tree_spec;

typedef struct {
  int32_t n_nodes, n_paths, path_width, mask_words;   /* in: capacities, out: sizes */
  int32_t* tree_indices;
  int32_t* depth;
  int32_t* parent;
  uint64_t* tree_mask;
  int32_t* retrieve_indices;
  double* node_weight;
} medusa_tree;

medusa_status medusa_tree_compile(const medusa_tree_spec* spec, medusa_tree* out);

/* ------------------------------------------------------------------ tree budget (host)
 *
 * [M7.2] §0x04C: maximising the expected accepted length per round is not maximising tokens
 * per second, because nodes carry kernel and cache costs; [Chai] "局限与适用场景": attention
 * traffic grows with context length and node count, so the best node count changes with the
 * context length.  For the nested greedy trees T_N of medusa_tree_compile (mode B: T_N is
 * the first N - 1 admissions of the growth), N rows including the root:
 *   E[A](N) = sum of T_N's non-root path weights ([M7.2] §0x04B)
 *   t(N)    = the per-layer cost of the tree-dependent work at the round's context length,
 *             linear between the measured points (cost_nodes[i], cost_us[i]), cost_nodes
 *             strictly increasing
 *   rate(N) = (1 + E[A](N)) / (fixed_us + n_layers * t(N))   (published tokens per us)
 * *best_n = the N in [cost_nodes[0], cost_nodes[n_costs - 1]] with the largest rate, the
 * smallest on ties.  Optional host outputs of cost_nodes[n_costs - 1] + 1 doubles, indexed
 * by N: expected_tokens[N] = 1 + E[A](N), rate[N] (0 outside the measured range).
 * fixed_us is the tree-independent cost of a round (for example the backbone weight stream).
 * Errors: MEDUSA_EINVAL (NULL pointer, non-increasing or non-positive node counts, a negative
 * or non-finite cost, rank_hit outside [0, 1], a round that would cost nothing),
 * MEDUSA_ECAPACITY (more rows than the rank table can hold, or host memory for the search
 * runs out).  Host only; no exception leaves the call.
 */
medusa_status medusa_tree_budget(const double* rank_hit, int32_t num_heads, int32_t topk, int32_t n_costs,
                                 const int32_t* cost_nodes, const double* cost_us, double fixed_us,
                                 int32_t n_layers, int32_t* best_n, double* expected_tokens,
                                 double* rate);

/* ------------------------------------------------------------------ tree attention
 *
 * [Chai] section "Tree Attention：把一棵树压进一次并行前向" and [M7.2] §0x03C
 * "Target Verification Is A Rectangular Forward Contract": each tree row u of
 * sequence b attends to all P_b committed cache rows and, among the N staged
 * rows, to exactly its ancestors and itself; the result equals running the
 * root-to-u sequence through ordinary causal attention on its own.
 *   pos(u)  = P_b + depth[u]                        ([M7.2] §0x03A)
 *   q~      = RoPE(q[b,u,h], pos(u))
 *   K~_u    = RoPE(k_new[b,u,g], pos(u)); stored to k_cache[b,g,P_b+u,:]
 *   V_u     = v_new[b,u,g];               stored to v_cache[b,g,P_b+u,:]
 *   out[b,u,h] = softmax_j(q~ . key_j / sqrt(d_h)) over {cache rows 0..P_b-1}
 *                U {staged rows P_b+v : tree_mask bit v of row u}, times values
 * with g = h / (Hq/Hkv).  RoPE pairs element i with element i + d_h/2 and
 * rotates them by pos * rope_base^(-2i/d_h); the angles are formed in
 * binary64.  Committed rows 0..P_b-1 are used as stored (already rotated).
 *
 * Layouts (dtype dt for every float tensor; arithmetic in fp32):
 *   q, out           [B][N][Hq][d_h]        device
 *   k_new, v_new     [B][N][Hkv][d_h]       device
 *   k_cache, v_cache [B][Hkv][S_max][d_h]   device; rows P_b..P_b+N-1 are written
 *   d_depth          int32[N]               device
 *   d_tree_mask      uint64[N][mask_words]  device
 *   d_prefix_len     int32[B]               device, P_b (read only)
 * Supported: d_h in {64, 128}; Hq % Hkv == 0; 1 <= N <= 64*mask_words;
 * dt in {MEDUSA_F32, MEDUSA_BF16}.
 * Workspace: device memory of at least medusa_tree_attn_workspace_size(...)
 * bytes, owned by the caller.  For bf16 (d_h 64 or 128) it receives the partial
 * results of the key-range splits ((m, l) in fp32 and O / l in 16-bit fixed point per query
 * row and split), merged into out by a second kernel of the same call; no state
 * carries from one call to the next.  Calls sharing a workspace must be ordered
 * (same stream).
 * Device-detected errors (d_status): any P_b < 0 or P_b + N > S_max
 * -> MEDUSA_ECAPACITY; for bf16, a depth[u] outside [0, 32)
 * -> MEDUSA_EUNSUPPORTED (the RoPE phase table holds 32 depths); both with no
 * stores to the cache or out.
 */
size_t medusa_tree_attn_workspace_size(medusa_dtype dt, int32_t B, int32_t Hq, int32_t Hkv,
                                       int32_t d_h, int32_t N, int32_t S_max);

medusa_status medusa_tree_attn(void* stream, medusa_dtype dt, int32_t B, int32_t Hq, int32_t Hkv,
                               int32_t d_h, int32_t N, const int32_t* d_depth,
                               const uint64_t* d_tree_mask, int32_t mask_words,
                               const int32_t* d_prefix_len, const void* q, const void* k_new,
                               const void* v_new, void* k_cache, void* v_cache, int32_t S_max,
                               double rope_base, void* out, void* workspace,
                               size_t workspace_bytes, int32_t* d_status, void* ev_start,
                               void* ev_stop);

/* ------------------------------------------------------------------ tree attention, no allocation
 *
 * For callers that cannot allocate device memory or pass a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  Computes exactly what
 * medusa_tree_attn computes, with the same arguments except the workspace; the split
 * partials go to a device array of MEDUSA_TREE_ATTN_SCRATCH_BYTES bytes that the library
 * holds on every GPU it runs on until the process ends (its address is taken on the first
 * call made with that GPU current; that call and no later one may load the library's code
 * object on the device).  No call allocates or frees memory.
 * The array is shared by every call on one GPU: calls that overlap on one GPU (different
 * streams, no ordering between them) race and their outputs are undefined; calls on one
 * stream are ordered and independent.
 * Limit: a shape whose workspace (medusa_tree_attn_workspace_size) exceeds the array gets
 * MEDUSA_ECAPACITY before any launch; every shape medusa_tree_attn supports fits.
 * Errors: those of medusa_tree_attn, plus MEDUSA_EHIP if the array's address cannot be
 * taken on the current GPU.
 */
#define MEDUSA_TREE_ATTN_SCRATCH_BYTES ((size_t)256 * 128 * (16 + 128 * 2))

medusa_status medusa_tree_attn_noalloc(void* stream, medusa_dtype dt, int32_t B, int32_t Hq, int32_t Hkv,
                                       int32_t d_h, int32_t N, const int32_t* d_depth,
                                       const uint64_t* d_tree_mask, int32_t mask_words,
                                       const int32_t* d_prefix_len, const void* q, const void* k_new,
                                       const void* v_new, void* k_cache, void* v_cache, int32_t S_max,
                                       double rope_base, void* out, int32_t* d_status, void* ev_start,
                                       void* ev_stop);

/* ------------------------------------------------------------------ acceptance
 *
 * [M7.2] §0x03D and §0x04D; [PartII] Part 7.  Per sequence b:
 *   token[u]  = candidates[b][tree_indices[u]]            (slot 0 = LM root)
 *   t[u]      = argmax_v logits[b][u][v] (lowest index on ties), or
 *               target_ids[b][u] when logits is NULL
 *   a_i       = number of leading j with retrieve[i][j+1] != -1 and
 *               token[retrieve[i][j+1]] == t[retrieve[i][j]]  (a sentinel ends
 *               the path; it never matches)
 *   a*        = max_i a_i; best = the smallest i with a_i == a* (0 when a* = 0)
 * Outputs (device): best_path[b] = best, accept_len[b] = a* (suffix edges; the
 * round publishes G = a*+1 tokens including the root), accepted_tokens[b][j] =
 * token[retrieve[best][j]] for j < G and -1 for G <= j < path_width,
 * frontier_row[b] = retrieve[best][a*] (the row whose logits seed the next
 * round, [M7.2] §0x06C).
 * Layouts: logits float32 [B][N][V]; target_ids int32 [B][N]; candidates int32
 * [B][n_slots]; d_tree_indices int32 [N]; d_retrieve int32 [n_paths][path_width]; all device.
 * Workspace: at least medusa_accept_workspace_size(B, N) bytes of device memory.
 * Device-detected errors (d_status): a NaN logit, a tree index outside
 * [0, n_slots), a retrieve entry outside [-1, N) or a path not starting at row 0
 * -> MEDUSA_EINVAL, with no output stores.
 */
size_t medusa_accept_workspace_size(int32_t B, int32_t N);

medusa_status medusa_accept(void* stream, int32_t B, int32_t N, int32_t V, const float* logits,
                            const int32_t* target_ids, const int32_t* candidates, int32_t n_slots,
                            const int32_t* d_tree_indices, const int32_t* d_retrieve,
                            int32_t n_paths, int32_t path_width, int32_t* best_path,
                            int32_t* accept_len, int32_t* accepted_tokens, int32_t* frontier_row,
                            void* workspace, size_t workspace_bytes, int32_t* d_status,
                            void* ev_start, void* ev_stop);

/* ------------------------------------------------------------------ typical acceptance
 *
 * [M7.2] §0x04E "Fast Typical Acceptance Derivation"; defaults from [Chai] section
 * "接受机制" (posterior_threshold = 0.3 = epsilon, posterior_alpha = 0.09 = alpha).
 * Per sequence b, with token[u] = candidates[b][tree_indices[u]] as for medusa_accept
 * and p_r = softmax(logits[b][r] / temperature) for row r:
 *   H_r    = -sum_x p_r(x) log(p_r(x) + 1e-5)
 *   tau_r  = min(epsilon, alpha * exp(-H_r))
 *   edge (r, child) passes iff p_r(token[child]) > tau_r  (strict)
 *   a_i    = number of leading passing edges of retrieve row i (a sentinel ends it)
 *   among the i with a_i = max a, the largest sum over its accepted edges of
 *   log p_r(token[child]) wins; the smallest such i on exact ties.
 * Outputs and layouts as for medusa_accept (logits are required).  The statistics are
 * formed in fp32; a pass decision whose margin |p - tau| is below fp32 rounding may differ
 * from a binary64 evaluation.
 * Workspace: at least medusa_accept_workspace_size(B, N) bytes of device memory.
 * Host errors: MEDUSA_EINVAL for temperature <= 0 or a non-finite temperature, epsilon or
 * alpha, negative epsilon or alpha, or a NULL pointer; MEDUSA_EBUFSIZE for a short
 * workspace.  Device-detected errors (d_status): a NaN logit, a tree index outside
 * [0, n_slots), a candidate id outside [0, V), a retrieve entry outside [-1, N) or a path
 * not starting at row 0 -> MEDUSA_EINVAL, with no output stores.
 */
medusa_status medusa_accept_typical(void* stream, int32_t B, int32_t N, int32_t V, const float* logits,
                                    double temperature, double epsilon, double alpha,
                                    const int32_t* candidates, int32_t n_slots,
                                    const int32_t* d_tree_indices, const int32_t* d_retrieve,
                                    int32_t n_paths, int32_t path_width, int32_t* best_path,
                                    int32_t* accept_len, int32_t* accepted_tokens,
                                    int32_t* frontier_row, void* workspace, size_t workspace_bytes,
                                    int32_t* d_status, void* ev_start, void* ev_stop);

/* ------------------------------------------------------------------ accept, commit, carry
 *
 * Greedy acceptance (exactly as medusa_accept, same outputs), then, per sequence and with
 * the chosen path, the compaction of medusa_kv_compact ([M7.2] §0x06A-§0x06B: for j < G_b
 * = accept_len[b] + 1, cache rows P_b + j <- P_b + retrieve[best][j] of every layer, kv
 * head, K and V, all source rows read before any is written; then prefix_len[b] += G_b)
 * and the frontier carry ([M7.2] §0x06C: the next round starts from the terminal row
 * f_b = frontier_row[b]):
 *   next_root[b]  = the target token of row f_b (argmax of logits[b][f_b], lowest index on
 *                   ties; target_ids[b][f_b] when target ids are given)   (optional)
 *   h_next[b][:]  = hidden[b][f_b][:]                                     (optional)
 * One call replaces medusa_accept + medusa_kv_compact and launches two kernels.  Nothing in
 * it allocates, copies through the host or synchronises, so a round built from it can be
 * captured in a HIP graph and replayed ([Chai] "把 Python 控制流赶出热路径").
 * Arguments as medusa_accept and medusa_kv_compact (k_cache / v_cache: host arrays of
 * n_layers device pointers, each [B][Hkv][S_max][d_h] of dtype dt, 16-byte aligned;
 * d_prefix_len int32 [B] device, in: P_b, out: P_b + G_b), plus:
 *   hidden     device [B][N][hidden_dim] of dtype dt (the tree rows' hidden states), or NULL
 *   h_next     device [B][hidden_dim] of dtype dt, or NULL (together with hidden)
 *   next_root  device int32 [B], or NULL
 * Limits: n_layers <= 32, path_width <= 8, d_h * size(dt) and hidden_dim * size(dt)
 * multiples of 16 bytes (else MEDUSA_EUNSUPPORTED).  The copy runs in one workgroup per
 * sequence: with many layers and few sequences medusa_kv_compact spreads it wider.
 * Workspace: medusa_accept_workspace_size(B, N) bytes when logits are given.
 * Device-detected errors (d_status), all before any store of the call: those of
 * medusa_accept, and P_b < 0 or P_b + N > S_max for any sequence -> MEDUSA_ECAPACITY.
 */
medusa_status medusa_accept_commit(void* stream, int32_t B, int32_t N, int32_t V, const float* logits,
                                   const int32_t* target_ids, const int32_t* candidates, int32_t n_slots,
                                   const int32_t* d_tree_indices, const int32_t* d_retrieve,
                                   int32_t n_paths, int32_t path_width, int32_t* best_path,
                                   int32_t* accept_len, int32_t* accepted_tokens, int32_t* frontier_row,
                                   medusa_dtype dt, int32_t n_layers, int32_t Hkv, int32_t d_h,
                                   int32_t S_max, void* const* k_cache, void* const* v_cache,
                                   int32_t* d_prefix_len, int32_t hidden_dim, const void* hidden,
                                   void* h_next, int32_t* next_root, void* workspace,
                                   size_t workspace_bytes, int32_t* d_status, void* ev_start,
                                   void* ev_stop);

/* ------------------------------------------------------------------ head step and candidates
 *
 * [Chai] section "Medusa 的核心思路与系统位置" and [Math] section "The Medusa head: math and
 * shapes": head k maps the last hidden state h of sequence b to the logits
 *   l_k[b] = W2_k (SiLU(W1_k h_b) + h_b)       (no bias; [M7.2] §0x02A adds one in general)
 * "Medusa Part II ...", Part 4: each head contributes its topk ranked ids; [M7.2] §0x01B:
 *   candidates[b][0]                   = root_tokens[b]   (the LM head's token, [Chai]
 *                                                          "一次完整解码迭代")
 *   candidates[b][1 + k*topk + r]      = id of the r-th largest entry of l_k[b]
 * the lower id first among equal logits.  This is the candidates[] input of medusa_accept.
 * Layouts (bf16 = IEEE binary32 truncated to its high 16 bits with round-to-nearest-even):
 *   h          bf16 [B][d]      device (16-byte aligned)
 *   W1         bf16 [K][d][d]   device, row o of head k is W1_k[o][:] (16-byte aligned)
 *   W2         bf16 [K][V][d]   device, row v of head k is W2_k[v][:] (16-byte aligned)
 *   d_root_tokens int32 [B]; candidates int32 [B][1 + K*topk]; device
 *   head_logits   optional fp32 [K][B][V] device output (NULL: kept in the workspace)
 * Arithmetic in fp32 (inputs widened, products accumulated in fp32).  Weights are read once
 * per group of four sequences.
 * Workspace: at least medusa_head_workspace_size(B, K, d, V) bytes of device memory; it
 * receives u = SiLU(W1 h) + h and the ranked lists of the unembedding row blocks (the
 * logits are ranked where they are computed and written to memory only into head_logits).
 * Host errors: MEDUSA_EINVAL (non-positive size, NULL pointer, h, W1 or W2 not 16-byte
 * aligned), MEDUSA_EUNSUPPORTED (d not a multiple of 8 or above 8192, topk above 64 or above
 * V, one head's W2 or the fp32 inputs of one head 4 GiB or larger), MEDUSA_EBUFSIZE.
 * Device-detected error (d_status): a NaN logit -> MEDUSA_EINVAL, and no candidate is written
 * by a call whose status word is already nonzero when its last kernel starts.
 */
size_t medusa_head_workspace_size(int32_t B, int32_t K, int32_t d, int32_t V);

medusa_status medusa_head_candidates(void* stream, int32_t B, int32_t K, int32_t d, int32_t V,
                                     int32_t topk, const void* h, const void* W1, const void* W2,
                                     const int32_t* d_root_tokens, int32_t* candidates,
                                     float* head_logits, void* workspace, size_t workspace_bytes,
                                     int32_t* d_status, void* ev_start, void* ev_stop);

/* ------------------------------------------------------------------ KV compaction
 *
 * [M7.2] §0x06A-§0x06D: with G_b = accept_len[b] + 1, u_j = retrieve[best_path[b]][j],
 * for every layer, kv head and both K and V:
 *   cache[b][g][P_b + j] <- cache[b][g][P_b + u_j]   for j < G_b
 * all G_b source rows being read before any is written (sources and
 * destinations may overlap), then prefix_len[b] <- P_b + G_b.  Rows beyond the
 * new length keep their stale staged bytes.
 * k_cache / v_cache: host arrays of n_layers device pointers, each cache
 * [B][Hkv][S_max][d_h] of dtype dt.  d_retrieve int32 [n_paths][path_width],
 * best_path / accept_len int32 [B], d_prefix_len int32 [B] (in: P_b, out:
 * P_b + G_b); all device.
 * Device-detected errors (d_status), checked for every sequence before any
 * store: best_path outside [0, n_paths), accept_len outside [0, path_width),
 * a sentinel or row >= n_nodes among the G_b published rows, P_b < 0 or
 * P_b + n_nodes > S_max -> MEDUSA_EINVAL / MEDUSA_ECAPACITY.
 */
medusa_status medusa_kv_compact(void* stream, medusa_dtype dt, int32_t n_layers, int32_t B,
                                int32_t Hkv, int32_t d_h, int32_t S_max, int32_t n_nodes,
                                void* const* k_cache, void* const* v_cache,
                                const int32_t* d_retrieve, int32_t n_paths, int32_t path_width,
                                const int32_t* best_path, const int32_t* accept_len,
                                int32_t* d_prefix_len, int32_t* d_status, void* ev_start,
                                void* ev_stop);

/* ------------------------------------------------------------------ measurement utility
 *
 * Not a step of the round: a streaming read of `bytes` (a multiple of 16) of device memory at
 * `src` (16-byte aligned), every thread keeping eight 16-byte loads in flight, with one word
 * per workgroup stored to `sink` (device, medusa_read_probe_sink_size() bytes).  Timed on a
 * buffer larger than the 256 MB Infinity Cache it gives the practical read bandwidth of the
 * chip, against which the round's memory-bound kernels are compared.
 * Host errors: MEDUSA_EINVAL (NULL pointer, size or alignment).
 */
size_t medusa_read_probe_sink_size(void);

medusa_status medusa_read_probe(void* stream, const void* src, size_t bytes, uint32_t* sink,
                                void* ev_start, void* ev_stop);

#ifdef __cplusplus
}
#endif

#endif /* MEDUSA_H */
