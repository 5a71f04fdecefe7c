// Host tree compiler: rank paths (explicit, or grown greedily from rank-hit
// probabilities) -> the flattened buffers every round reads.
//
// [M7.2] = "M7.2 - Medusa: Multi-Head Candidates, Tree Attention, and Verification"
//   §0x04A "Sparse Tree Construction": prefix closure; canonical row order by
//     (length, path); candidate gather slot 1 + (len-1)*TOPK + last rank;
//     ancestry mask; depth; maximal retrieve rows with a negative sentinel.
//   §0x04B "Calibration Probabilities And Expected Accepted Length": the path
//     weight is the product of the per-depth exact-rank hit probabilities.
//   §0x04C "Greedy Frontier Search And Its Boundary": admit the best frontier
//     path whose parent is present until the budget is spent.
// "Medusa Part II: Candidate Trees, Verification, and Acceptance", Part 3
//   Step 3, describes the same budgeted growth.
//
// This is integer work plus binary64 products; it runs once per tree shape on
// the host (the pages build these buffers at start-up and keep them resident).
// Built with -ffp-contract=off so every weight is the plain left-to-right
// product of IEEE binary64 multiplications.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <climits>
#include <new>
#include <queue>
#include <vector>

#include "medusa.h"

namespace {

constexpr int32_t kMaxNodes = 16384;  // mask alone is N*N/8 bytes (32 MiB here)

using Path = std::vector<int32_t>;

// A path of the greedy search, stored once in a pool as (parent, last rank): the frontier
// holds pool ids, so a push copies no path.
struct PoolNode {
  int32_t parent;  // pool id, -1 for the root's children
  int32_t rank;
  int32_t depth;
  double w;
};

// ranks of a pool path from the root down, into r[0 .. depth)
void ranks_of(const std::vector<PoolNode>& pool, int32_t id, int32_t* r) {
  for (int32_t v = id; v >= 0; v = pool[v].parent) r[pool[v].depth - 1] = pool[v].rank;
}

// Priority of the greedy loop: larger weight first, then the shorter path,
// then the lexicographically smaller one.  Only exact weight ties compare paths.
struct LowerPriority {
  const std::vector<PoolNode>* pool;
  bool operator()(int32_t a, int32_t b) const {
    const PoolNode& x = (*pool)[a];
    const PoolNode& y = (*pool)[b];
    if (x.w != y.w) return x.w < y.w;
    if (x.depth != y.depth) return x.depth > y.depth;
    int32_t ra[64], rb[64];  // depth <= num_heads <= 64
    ranks_of(*pool, a, ra);
    ranks_of(*pool, b, rb);
    return std::lexicographical_compare(rb, rb + y.depth, ra, ra + x.depth);
  }
};

bool canonical_less(const Path& a, const Path& b) {
  if (a.size() != b.size()) return a.size() < b.size();
  return a < b;
}

// canonical order of a stored path against the first n ranks of another
bool canonical_less_prefix(const Path& a, const int32_t* b, size_t n) {
  if (a.size() != n) return a.size() < n;
  return std::lexicographical_compare(a.begin(), a.end(), b, b + n);
}

// Number of rank tuples of length 1..K, saturated at `cap`.
int64_t tuple_count(int32_t K, int32_t topk, int64_t cap) {
  int64_t total = 0, level = 1;
  for (int32_t d = 0; d < K; ++d) {
    level = (level > cap / topk) ? cap : level * topk;
    total = std::min<int64_t>(cap, total + level);
  }
  return total;
}

medusa_status grow_greedy(const medusa_tree_spec& s, std::vector<Path>& paths,
                          std::vector<double>* weights = nullptr) {
  const int32_t K = s.num_heads, topk = s.topk;
  for (int64_t i = 0; i < int64_t(K) * topk; ++i) {
    const double a = s.rank_hit[i];
    if (!(a >= 0.0 && a <= 1.0)) return MEDUSA_EINVAL;  // also rejects NaN
  }
  if (s.n_nodes < 1) return MEDUSA_EINVAL;
  if (s.n_nodes > kMaxNodes) return MEDUSA_ECAPACITY;
  const int64_t budget = int64_t(s.n_nodes) - 1;
  if (budget > tuple_count(K, topk, int64_t(1) << 40)) return MEDUSA_ECAPACITY;
  // every admitted path adds at most topk pool entries, addressed by int32 ids
  if ((budget + 1) * int64_t(topk) > int64_t(INT32_MAX)) return MEDUSA_ECAPACITY;

  std::vector<PoolNode> pool;
  // a modest reservation; larger searches grow the vectors (an allocation failure is
  // reported as MEDUSA_ECAPACITY by the entry points)
  const size_t want = size_t(std::min<int64_t>((budget + 1) * int64_t(topk), int64_t(1) << 16));
  pool.reserve(want);
  std::vector<int32_t> heap_store;
  heap_store.reserve(want);
  std::priority_queue<int32_t, std::vector<int32_t>, LowerPriority> frontier(LowerPriority{&pool},
                                                                              std::move(heap_store));
  for (int32_t r = 0; r < topk; ++r) {
    pool.push_back({-1, r, 1, 1.0 * s.rank_hit[r]});
    frontier.push(int32_t(pool.size()) - 1);
  }
  int32_t buf[64];
  while (int64_t(paths.size()) < budget) {
    const int32_t best = frontier.top();
    frontier.pop();
    const PoolNode node = pool[best];
    if (node.depth < K) {
      for (int32_t r = 0; r < topk; ++r) {
        pool.push_back({best, r, node.depth + 1, node.w * s.rank_hit[int64_t(node.depth) * topk + r]});
        frontier.push(int32_t(pool.size()) - 1);
      }
    }
    ranks_of(pool, best, buf);
    paths.emplace_back(buf, buf + node.depth);
    if (weights) weights->push_back(node.w);
  }
  return MEDUSA_OK;
}

medusa_status read_explicit(const medusa_tree_spec& s, std::vector<Path>& paths) {
  if (s.n_paths < 0) return MEDUSA_EINVAL;
  if (s.n_paths >= kMaxNodes) return MEDUSA_ECAPACITY;
  if (s.n_paths > 0 && s.path_ranks == nullptr) return MEDUSA_EINVAL;
  int64_t off = 0;
  for (int32_t i = 0; i < s.n_paths; ++i) {
    const int32_t len = s.path_len[i];
    if (len < 1 || len > s.num_heads) return MEDUSA_EINVAL;
    Path p(s.path_ranks + off, s.path_ranks + off + len);
    off += len;
    for (int32_t r : p)
      if (r < 0 || r >= s.topk) return MEDUSA_EINVAL;
    paths.push_back(std::move(p));
  }
  return MEDUSA_OK;
}

}  // namespace

static medusa_status tree_compile_impl(const medusa_tree_spec* spec, medusa_tree* out) {
  if (spec == nullptr || out == nullptr) return MEDUSA_EINVAL;
  const medusa_tree_spec& s = *spec;
  if (s.num_heads < 1 || s.topk < 1 || s.num_heads > 64) return MEDUSA_EINVAL;

  std::vector<Path> paths;
  medusa_status st;
  if (s.path_len != nullptr) {
    st = read_explicit(s, paths);
  } else {
    if (s.rank_hit == nullptr) return MEDUSA_EINVAL;
    st = grow_greedy(s, paths);
  }
  if (st != MEDUSA_OK) return st;

  // canonical order, duplicates, prefix closure: row u holds paths[u - 1], and the parent
  // of a path is found by binary search for its prefix among the sorted paths
  std::sort(paths.begin(), paths.end(), canonical_less);
  for (size_t i = 1; i < paths.size(); ++i)
    if (paths[i] == paths[i - 1]) return MEDUSA_EINVAL;
  const int32_t n = int32_t(paths.size()) + 1;
  std::vector<int32_t> parent(n, -1), depth(n, 0), slot(n, 0);
  for (int32_t u = 1; u < n; ++u) {
    const Path& p = paths[u - 1];
    const size_t L = p.size() - 1;  // prefix length
    if (L == 0) {
      parent[u] = 0;
    } else {
      auto it = std::lower_bound(paths.begin(), paths.end(), p.data(),
                                 [L](const Path& x, const int32_t* b) { return canonical_less_prefix(x, b, L); });
      if (it == paths.end() || it->size() != L || !std::equal(it->begin(), it->end(), p.begin()))
        return MEDUSA_ENOT_PREFIX_CLOSED;
      parent[u] = int32_t(it - paths.begin()) + 1;
    }
    depth[u] = int32_t(p.size());
    slot[u] = 1 + (depth[u] - 1) * s.topk + p.back();
  }
  std::vector<char> has_child(n, 0);
  for (int32_t u = 1; u < n; ++u) has_child[parent[u]] = 1;
  std::vector<int32_t> leaves;
  int32_t max_depth = 0;
  for (int32_t u = 0; u < n; ++u) {
    if (!has_child[u]) leaves.push_back(u);
    max_depth = std::max(max_depth, depth[u]);
  }
  const int32_t words = (n + 63) / 64;
  const int32_t width = max_depth + 1;
  const int32_t n_leaves = int32_t(leaves.size());

  const bool query = out->tree_indices == nullptr && out->depth == nullptr &&
                     out->parent == nullptr && out->tree_mask == nullptr &&
                     out->retrieve_indices == nullptr && out->node_weight == nullptr;
  if (query) {
    out->n_nodes = n;
    out->n_paths = n_leaves;
    out->path_width = width;
    out->mask_words = words;
    return MEDUSA_OK;
  }
  if (out->tree_indices == nullptr || out->depth == nullptr || out->parent == nullptr ||
      out->tree_mask == nullptr || out->retrieve_indices == nullptr)
    return MEDUSA_EINVAL;
  if (out->n_nodes < n || out->n_paths < n_leaves || out->path_width < width ||
      out->mask_words < words)
    return MEDUSA_EBUFSIZE;
  if (out->node_weight != nullptr && s.rank_hit == nullptr) return MEDUSA_EINVAL;
  if (out->node_weight != nullptr) {
    for (int64_t i = 0; i < int64_t(s.num_heads) * s.topk; ++i)
      if (!(s.rank_hit[i] >= 0.0 && s.rank_hit[i] <= 1.0)) return MEDUSA_EINVAL;
  }

  // every check passed: emit
  for (int32_t u = 0; u < n; ++u) {
    out->tree_indices[u] = slot[u];
    out->depth[u] = depth[u];
    out->parent[u] = parent[u];
  }
  std::memset(out->tree_mask, 0, sizeof(uint64_t) * size_t(n) * size_t(words));
  for (int32_t u = 0; u < n; ++u) {
    uint64_t* m = out->tree_mask + size_t(u) * words;
    for (int32_t v = u; v >= 0; v = parent[v]) m[v / 64] |= uint64_t(1) << (v % 64);
  }
  for (int32_t i = 0; i < n_leaves; ++i) {
    int32_t* r = out->retrieve_indices + size_t(i) * width;
    std::fill(r, r + width, -1);
    for (int32_t v = leaves[i]; v >= 0; v = parent[v]) r[depth[v]] = v;
  }
  if (out->node_weight != nullptr) {
    out->node_weight[0] = 1.0;
    for (int32_t u = 1; u < n; ++u) {
      const Path& p = paths[u - 1];
      double w = 1.0;
      for (size_t j = 0; j < p.size(); ++j) w = w * s.rank_hit[int64_t(j) * s.topk + p[j]];
      out->node_weight[u] = w;
    }
  }
  out->n_nodes = n;
  out->n_paths = n_leaves;
  out->path_width = width;
  out->mask_words = words;
  return MEDUSA_OK;
}

// Context-dependent budget.  [M7.2] §0x04C: the greedy search maximises the expected accepted
// length per round, which is not tokens per second, since nodes carry kernel costs; [Chai]
// "局限与适用场景": the attention traffic grows with context length and node count, so the best
// node count changes with context length.  The tree of budget N is the first N - 1
// admissions of the greedy growth, so E[A](N) is their weights' running sum (admission
// order, binary64), and the round rate is (1 + E[A](N)) / (fixed_us + n_layers * t(N)).
static medusa_status tree_budget_impl(const double* rank_hit, int32_t num_heads, int32_t topk, int32_t n_costs,
                                      const int32_t* cost_nodes, const double* cost_us, double fixed_us,
                                      int32_t n_layers, int32_t* best_n, double* expected_tokens, double* rate) {
  if (!rank_hit || !cost_nodes || !cost_us || !best_n || num_heads < 1 || topk < 1 || n_costs < 1 ||
      n_layers < 0 || !(fixed_us >= 0.0) || !std::isfinite(fixed_us))
    return MEDUSA_EINVAL;
  for (int32_t i = 0; i < n_costs; ++i) {
    if (cost_nodes[i] < 1 || (i > 0 && cost_nodes[i] <= cost_nodes[i - 1])) return MEDUSA_EINVAL;
    if (!(cost_us[i] >= 0.0) || !std::isfinite(cost_us[i])) return MEDUSA_EINVAL;
  }
  const int32_t lo = cost_nodes[0], hi = cost_nodes[n_costs - 1];
  medusa_tree_spec s{};
  s.num_heads = num_heads;
  s.topk = topk;
  s.rank_hit = rank_hit;
  s.n_nodes = hi;
  std::vector<Path> paths;
  std::vector<double> w;
  const medusa_status st = grow_greedy(s, paths, &w);
  if (st != MEDUSA_OK) return st;
  if (fixed_us == 0.0 && n_layers == 0) return MEDUSA_EINVAL;  // a round would cost nothing
  int32_t seg = 0;
  double ea = 0.0, best_rate = -1.0;
  int32_t best = lo;
  for (int32_t n = 1; n <= hi; ++n) {
    if (n >= 2) ea += w[size_t(n) - 2];
    if (n < lo) {
      if (expected_tokens) expected_tokens[n] = 1.0 + ea;
      if (rate) rate[n] = 0.0;
      continue;
    }
    while (seg + 1 < n_costs - 1 && cost_nodes[seg + 1] < n) ++seg;
    double t = cost_us[seg];
    if (n_costs > 1) {
      const int32_t n0 = cost_nodes[seg], n1 = cost_nodes[seg + 1];
      t = cost_us[seg] + (cost_us[seg + 1] - cost_us[seg]) * double(n - n0) / double(n1 - n0);
    }
    const double r = (1.0 + ea) / (fixed_us + double(n_layers) * t);
    if (expected_tokens) expected_tokens[n] = 1.0 + ea;
    if (rate) rate[n] = r;
    if (r > best_rate) {
      best_rate = r;
      best = n;
    }
  }
  if (expected_tokens) expected_tokens[0] = 0.0;
  if (rate) rate[0] = 0.0;
  *best_n = best;
  return MEDUSA_OK;
}

// C entry points: no exception crosses the ABI (an allocation failure of a very large
// search or tree is reported as MEDUSA_ECAPACITY)
extern "C" medusa_status medusa_tree_compile(const medusa_tree_spec* spec, medusa_tree* out) {
  try {
    return tree_compile_impl(spec, out);
  } catch (const std::bad_alloc&) {
    return MEDUSA_ECAPACITY;
  } catch (...) {
    return MEDUSA_EINVAL;
  }
}

extern "C" medusa_status medusa_tree_budget(const double* rank_hit, int32_t num_heads, int32_t topk,
                                            int32_t n_costs, const int32_t* cost_nodes,
                                            const double* cost_us, double fixed_us, int32_t n_layers,
                                            int32_t* best_n, double* expected_tokens, double* rate) {
  try {
    return tree_budget_impl(rank_hit, num_heads, topk, n_costs, cost_nodes, cost_us, fixed_us, n_layers,
                            best_n, expected_tokens, rate);
  } catch (const std::bad_alloc&) {
    return MEDUSA_ECAPACITY;
  } catch (...) {
    return MEDUSA_EINVAL;
  }
}
