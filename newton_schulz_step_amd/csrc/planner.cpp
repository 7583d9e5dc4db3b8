// Owner planning for dedicated ownership (host only).
//
// DMuon ("Z2 与 Z3 模式", sections on the packed-buffer lifecycles and on the
// relation to ZeRO-2/3): every Muon-target matrix has one owner, which alone
// runs its Newton-Schulz; an owner's matrices are packed into one contiguous
// buffer, broadcast layer by layer. The owner choice is not given there: the
// planner balances nominal Newton-Schulz FLOPs with the largest-first greedy
// rule (LPT) and packs each owner's matrices layer by layer.
#include <algorithm>
#include <functional>
#include <numeric>
#include <queue>
#include <string>
#include <utility>
#include <vector>

#include "planner.hpp"

namespace muon {

static bool mul_ok(int64_t a, int64_t b, int64_t& out) { return !__builtin_mul_overflow(a, b, &out); }
static bool add_ok(int64_t a, int64_t b, int64_t& out) { return !__builtin_add_overflow(a, b, &out); }

int64_t ns_flops(int64_t m, int64_t n, int method, int steps) {
  if (m < 1 || n < 1 || steps < 1 || steps > 64) return -1;
  if (method != MUON_NS_STANDARD && method != MUON_NS_GRAM) return -1;
  int64_t mm, m2n, m3;
  if (!mul_ok(m, m, mm) || !mul_ok(mm, n, m2n) || !mul_ok(mm, m, m3)) return -1;
  // standard: steps x (4 m^2 n + 2 m^3); gram: 4 m^2 n + (8 steps - 6) m^3
  int64_t a, b, out;
  if (method == MUON_NS_STANDARD) {
    if (!mul_ok(m2n, 4 * static_cast<int64_t>(steps), a) || !mul_ok(m3, 2 * static_cast<int64_t>(steps), b)) return -1;
  } else {
    if (!mul_ok(m2n, 4, a) || !mul_ok(m3, 8 * static_cast<int64_t>(steps) - 6, b)) return -1;
  }
  return add_ok(a, b, out) ? out : -1;
}

int plan_owners(const muon_param_t* params, int32_t n_params, int32_t n_owners, int32_t method, int32_t steps,
                int64_t align, muon_assign_t* assign, muon_owner_t* owners, std::string& err) {
  if (n_params < 0) { err = "n_params < 0"; return MUON_ERR_BAD_SHAPE; }
  if (n_owners < 1) { err = "n_owners must be >= 1"; return MUON_ERR_BAD_SHAPE; }
  if ((n_params > 0 && (params == nullptr || assign == nullptr)) || owners == nullptr) {
    err = "params, assign and owners must not be NULL";
    return MUON_ERR_NULL;
  }
  if (method != MUON_NS_STANDARD && method != MUON_NS_GRAM) {
    err = "ns_method must be MUON_NS_STANDARD or MUON_NS_GRAM, got " + std::to_string(method);
    return MUON_ERR_BAD_METHOD;
  }
  if (steps < 1 || steps > 64) { err = "ns_steps outside [1, 64]"; return MUON_ERR_BAD_HYPER; }
  if (align < 8 || align % 8 != 0) { err = "align must be a positive multiple of 8"; return MUON_ERR_ALIGN; }

  // FLOPs and elements per matrix
  std::vector<int64_t> cost(n_params), size(n_params);
  for (int32_t i = 0; i < n_params; ++i) {
    const muon_param_t& p = params[i];
    const std::string at = " (param " + std::to_string(i) + ")";
    if (p.rows < 1 || p.cols < 1) { err = "rows and cols must be >= 1" + at; return MUON_ERR_BAD_SHAPE; }
    if (p.split_rows < 0 || (p.split_rows > 0 && p.rows % p.split_rows != 0)) {
      err = "split_rows must be 0 or divide rows" + at;
      return MUON_ERR_BAD_SHAPE;
    }
    if (p.split_cols < 0 || (p.split_cols > 0 && p.cols % p.split_cols != 0)) {
      err = "split_cols must be 0 or divide cols" + at;
      return MUON_ERR_BAD_SHAPE;
    }
    if (p.layer < 0) { err = "layer < 0" + at; return MUON_ERR_BAD_SHAPE; }
    const int64_t pr = p.split_rows > 0 ? p.split_rows : p.rows;
    const int64_t pc = p.split_cols > 0 ? p.split_cols : p.cols;
    const int64_t m = std::min(pr, pc), n = std::max(pr, pc);
    if (m > MUON_MAX_SHORT_SIDE || n > MUON_MAX_LONG_SIDE || p.cols > MUON_MAX_LONG_SIDE) {
      err = "matrix beyond the size limits" + at;
      return MUON_ERR_BAD_SHAPE;
    }
    const int64_t f = ns_flops(m, n, method, steps);
    if (f < 0 || !mul_ok(f, (p.rows / pr) * (p.cols / pc), cost[i])) {
      err = "FLOP count overflows int64" + at;
      return MUON_ERR_RANGE;
    }
    size[i] = p.rows * p.cols;
  }

  // largest first; ties: more elements, then lower index
  std::vector<int32_t> order(n_params);
  std::iota(order.begin(), order.end(), 0);
  std::sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
    if (cost[x] != cost[y]) return cost[x] > cost[y];
    if (size[x] != size[y]) return size[x] > size[y];
    return x < y;
  });
  // each to the least-loaded owner; ties: lower owner index
  using Load = std::pair<int64_t, int32_t>;
  std::priority_queue<Load, std::vector<Load>, std::greater<Load>> heap;
  for (int32_t o = 0; o < n_owners; ++o) heap.push({0, o});
  std::vector<int32_t> owner_of(n_params);
  std::vector<int64_t> load(n_owners, 0);
  for (int32_t i : order) {
    const Load top = heap.top();
    heap.pop();
    int64_t nl;
    if (!add_ok(top.first, cost[i], nl)) { err = "owner FLOP total overflows int64"; return MUON_ERR_RANGE; }
    owner_of[i] = top.second;
    load[top.second] = nl;
    heap.push({nl, top.second});
  }

  // per owner: (layer, index) order, each matrix at the next multiple of align
  std::vector<std::vector<int32_t>> held(n_owners);
  for (int32_t i = 0; i < n_params; ++i) held[owner_of[i]].push_back(i);
  std::vector<int64_t> offset(n_params);
  std::vector<muon_owner_t> res(n_owners);
  for (int32_t o = 0; o < n_owners; ++o) {
    auto& v = held[o];
    std::stable_sort(v.begin(), v.end(), [&](int32_t x, int32_t y) { return params[x].layer < params[y].layer; });
    int64_t cur = 0, layer_start = 0, max_layer = 0;
    for (size_t k = 0; k < v.size(); ++k) {
      const int32_t i = v[k];
      int64_t padded;
      if (!add_ok(cur, align - 1, padded)) { err = "packed buffer length overflows int64"; return MUON_ERR_RANGE; }
      cur = padded / align * align;
      if (k == 0 || params[i].layer != params[v[k - 1]].layer) layer_start = cur;
      offset[i] = cur;
      if (!add_ok(cur, size[i], cur)) { err = "packed buffer length overflows int64"; return MUON_ERR_RANGE; }
      max_layer = std::max(max_layer, cur - layer_start);
    }
    res[o] = muon_owner_t{cur, max_layer, load[o], static_cast<int32_t>(v.size()), 0};
  }

  for (int32_t i = 0; i < n_params; ++i) assign[i] = muon_assign_t{owner_of[i], 0, offset[i]};
  for (int32_t o = 0; o < n_owners; ++o) owners[o] = res[o];
  return MUON_OK;
}

double comm_elements(int64_t p_m, int32_t n_ranks, int32_t zero_stage, int32_t dedicated) {
  if (p_m < 0 || n_ranks < 1 || (zero_stage != 2 && zero_stage != 3) || (dedicated != 0 && dedicated != 1))
    return -1.0;
  // collectives over the shard group: DMuon-Z2 reduce + forward broadcast; Z3
  // adds the backward re-broadcast; without owners, one more gradient all-gather
  const int k = (zero_stage == 2 ? 2 : 3) + (dedicated ? 0 : 1);
  return static_cast<double>(k) * static_cast<double>(n_ranks - 1) / static_cast<double>(n_ranks) *
         static_cast<double>(p_m);
}

}  // namespace muon
