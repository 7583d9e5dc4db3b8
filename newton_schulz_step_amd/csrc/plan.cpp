#include "plan.hpp"

#include <algorithm>
#include <cmath>
#include <map>
#include <utility>

#include "common_host.hpp"

namespace muon {

int element_size(int dtype) {
  switch (dtype) {
    case MUON_DTYPE_F32: return 4;
    case MUON_DTYPE_BF16:
    case MUON_DTYPE_F16: return 2;
    default: return 0;
  }
}

// 256 x 256 tiles (one workgroup per CU) for short sides from 512 up, unless the
// group's smallest launch, the symmetric X X^T over the lower tiles, would then
// fill fewer than 1.5 waves of the 256 CUs: 128 x 128 tiles (two workgroups per
// CU, four times the tiles) keep small groups from idling most of the chip.
int tile_for(int64_t m, int64_t count) {
  if (m < 512) return 128;
  const int64_t t = (m + 255) / 256;
  return count * t * (t + 1) / 2 >= 384 ? 256 : 128;
}

// The symmetric launches only need tiles up to m rounded to 128 (their K
// loops stop there too), so with 128-tiles a short side of 1408 costs 66 tiles
// of 128^2 instead of 21 of 256^2 (84 of 128^2); the full launches keep
// 256-tiles, whose operand reuse the 128-tiles lack.
int sym_tile_for(int64_t m, int tile) {
  return (tile == 256 && m % 256 != 0 && m % 256 <= 128) ? 128 : tile;
}

static int64_t round_up(int64_t v, int64_t q) { return (v + q - 1) / q * q; }
static size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

int validate(const muon_matrix_t* table, int32_t n_entries, const muon_hyper_t* h, std::string& err) {
  if (h == nullptr) { err = "hyperparameter pointer is NULL"; return MUON_ERR_NULL; }
  if (n_entries < 0) { err = "n_entries < 0"; return MUON_ERR_BAD_SHAPE; }
  if (n_entries > 0 && table == nullptr) { err = "table is NULL"; return MUON_ERR_NULL; }
  if (h->ns_method != MUON_NS_STANDARD && h->ns_method != MUON_NS_GRAM) {
    err = "ns_method must be MUON_NS_STANDARD (\"standard\") or MUON_NS_GRAM (\"gram\"), got " +
          std::to_string(h->ns_method);
    return MUON_ERR_BAD_METHOD;
  }
  const float fs[] = {h->lr, h->momentum, h->weight_decay, h->ns_a, h->ns_b, h->ns_c, h->ns_eps};
  for (float f : fs)
    if (!std::isfinite(f)) { err = "a hyperparameter is not finite"; return MUON_ERR_BAD_HYPER; }
  if (h->ns_eps < 0.0f) { err = "ns_eps < 0"; return MUON_ERR_BAD_HYPER; }
  if (h->ns_steps < 1 || h->ns_steps > 64) { err = "ns_steps outside [1, 64]"; return MUON_ERR_BAD_HYPER; }
  if (h->param_dtype != MUON_DTYPE_F32 && h->param_dtype != MUON_DTYPE_BF16) {
    err = "param_dtype must be F32 or BF16";
    return MUON_ERR_UNSUPPORTED;
  }
  if (element_size(h->grad_dtype) == 0) { err = "grad_dtype must be F32, BF16 or F16"; return MUON_ERR_UNSUPPORTED; }
  if (element_size(h->ns_dtype) == 0) { err = "ns_dtype must be F32, BF16 or F16"; return MUON_ERR_UNSUPPORTED; }
  if (h->ns_method == MUON_NS_GRAM && h->ns_dtype == MUON_DTYPE_BF16) {
    err = "gram Newton-Schulz with bf16 storage is not supported (it diverges); use F16 or F32";
    return MUON_ERR_UNSUPPORTED;
  }
  std::vector<std::pair<int64_t, int64_t>> spans;
  spans.reserve(n_entries);
  int64_t elements = 0, problems = 0;
  for (int32_t i = 0; i < n_entries; ++i) {
    const muon_matrix_t& e = table[i];
    const std::string at = " (entry " + std::to_string(i) + ")";
    if (e.rows < 1 || e.cols < 1) { err = "rows and cols must be >= 1" + at; return MUON_ERR_BAD_SHAPE; }
    if (e.split_rows < 0) { err = "split_rows < 0" + at; return MUON_ERR_BAD_SHAPE; }
    if (e.split_rows > 0 && e.rows % e.split_rows != 0) { err = "split_rows does not divide rows" + at; return MUON_ERR_BAD_SHAPE; }
    if (e.split_cols < 0) { err = "split_cols < 0" + at; return MUON_ERR_BAD_SHAPE; }
    if (e.split_cols > 0 && e.cols % e.split_cols != 0) { err = "split_cols does not divide cols" + at; return MUON_ERR_BAD_SHAPE; }
    const int64_t pr = e.split_rows > 0 ? e.split_rows : e.rows;
    const int64_t pc = e.split_cols > 0 ? e.split_cols : e.cols;
    const int64_t m = std::min(pr, pc), n = std::max(pr, pc);
    if (m > MUON_MAX_SHORT_SIDE || n > MUON_MAX_LONG_SIDE || e.cols > MUON_MAX_LONG_SIDE) {
      err = "matrix beyond the size limits" + at;
      return MUON_ERR_BAD_SHAPE;
    }
    // running totals, compared without overflow: rows <= (limit - elements) / cols
    if (e.rows > (MUON_MAX_TABLE_ELEMENTS - elements) / e.cols) {
      err = "the table holds more than MUON_MAX_TABLE_ELEMENTS elements" + at;
      return MUON_ERR_BAD_SHAPE;
    }
    elements += e.rows * e.cols;
    problems += (e.rows / pr) * (e.cols / pc);
    if (problems > MUON_MAX_PROBLEMS) { err = "the table expands to more than MUON_MAX_PROBLEMS problems" + at; return MUON_ERR_BAD_SHAPE; }
    if (e.offset < 0) { err = "offset < 0" + at; return MUON_ERR_RANGE; }
    if (e.offset > INT64_MAX - MUON_MAX_TABLE_ELEMENTS) { err = "offset beyond the addressable range" + at; return MUON_ERR_RANGE; }
    if (e.offset % 8 != 0) { err = "offset is not a multiple of 8 elements" + at; return MUON_ERR_ALIGN; }
    spans.emplace_back(e.offset, e.rows * e.cols);
  }
  std::sort(spans.begin(), spans.end());
  for (size_t i = 1; i < spans.size(); ++i)
    if (spans[i - 1].first + spans[i - 1].second > spans[i].first) { err = "table entries overlap"; return MUON_ERR_OVERLAP; }
  return MUON_OK;
}

int validate_windows(const muon_matrix_t* table, const muon_window_t* windows, int32_t n_entries,
                     int64_t partition_numel, std::string& err) {
  if (n_entries > 0 && windows == nullptr) { err = "windows is NULL"; return MUON_ERR_NULL; }
  if (partition_numel < 0) { err = "partition_numel < 0"; return MUON_ERR_RANGE; }
  std::vector<std::pair<int64_t, int64_t>> spans;
  for (int32_t i = 0; i < n_entries; ++i) {
    const muon_window_t& w = windows[i];
    const std::string at = " (window " + std::to_string(i) + ")";
    const int64_t total = table[i].rows * table[i].cols;
    if (w.lo < 0 || w.lo > w.hi || w.hi > total) { err = "window outside [0, rows * cols] or lo > hi" + at; return MUON_ERR_RANGE; }
    if (w.hi > w.lo && (w.param_offset < 0 || w.param_offset + (w.hi - w.lo) > partition_numel)) {
      err = "window does not fit in the partition" + at;
      return MUON_ERR_RANGE;
    }
    if (w.hi > w.lo) spans.emplace_back(w.param_offset, w.hi - w.lo);
  }
  std::sort(spans.begin(), spans.end());
  for (size_t i = 1; i < spans.size(); ++i)
    if (spans[i - 1].first + spans[i - 1].second > spans[i].first) { err = "windows overlap in the partition"; return MUON_ERR_OVERLAP; }
  return MUON_OK;
}

Layout build_layout(const muon_matrix_t* table, int32_t n_entries, const muon_hyper_t* h,
                    const muon_window_t* windows) {
  Layout L;
  // canonical shape -> group, in order of first appearance
  std::map<std::pair<int64_t, int64_t>, int> gid;
  std::vector<std::vector<HostProblem>> per_group;
  std::vector<std::pair<int, size_t>> entry_pos;   // (group, index of its first problem in the group)
  // block geometry of entry i: pr x pc blocks, nrb x ncb of them
  struct Geom { int64_t pr, pc, nrb, ncb; };
  auto geom = [&](const muon_matrix_t& e) {
    Geom q;
    q.pr = e.split_rows > 0 ? e.split_rows : e.rows;
    q.pc = e.split_cols > 0 ? e.split_cols : e.cols;
    q.nrb = e.rows / q.pr;
    q.ncb = e.cols / q.pc;
    return q;
  };
  for (int32_t i = 0; i < n_entries; ++i) {
    const muon_matrix_t& e = table[i];
    const Geom q = geom(e);
    const int64_t m = std::min(q.pr, q.pc), n = std::max(q.pr, q.pc);
    const auto key = std::make_pair(m, n);
    auto it = gid.find(key);
    int g;
    if (it == gid.end()) {
      g = static_cast<int>(L.groups.size());
      gid[key] = g;
      Group G;
      G.m = m; G.n = n;
      L.groups.push_back(G);
      per_group.emplace_back();
    } else {
      g = it->second;
    }
    entry_pos.emplace_back(g, per_group[g].size());
    const int64_t span = (q.pr - 1) * e.cols + q.pc;   // a block's last local index + 1
    for (int64_t b = 0; b < q.nrb * q.ncb; ++b) {
      HostProblem p;
      const int64_t first = (b / q.ncb) * q.pr * e.cols + (b % q.ncb) * q.pc;   // matrix flat index of element 0
      p.src_off = e.offset + first;
      p.ld = static_cast<int32_t>(e.cols);
      p.transposed = q.pr > q.pc ? 1 : 0;
      p.entry = i;
      if (windows == nullptr) {
        p.lo = 0;
        p.hi = span;
        p.p_base = p.src_off;
      } else {
        const muon_window_t& w = windows[i];
        p.lo = std::min(std::max(w.lo - first, int64_t(0)), span);
        p.hi = std::min(std::max(w.hi - first, int64_t(0)), span);
        p.p_base = w.param_offset - w.lo + first;
      }
      per_group[g].push_back(p);
    }
  }
  for (size_t g = 0; g < L.groups.size(); ++g) {
    Group& G = L.groups[g];
    G.tile = tile_for(G.m, static_cast<int64_t>(per_group[g].size()));
    G.sym_tile = sym_tile_for(G.m, G.tile);
    G.mp = round_up(G.m, G.tile);
    G.np = round_up(G.n, G.tile);
    L.groups[g].first = static_cast<int>(L.problems.size());
    L.groups[g].count = static_cast<int>(per_group[g].size());
    L.problems.insert(L.problems.end(), per_group[g].begin(), per_group[g].end());
  }
  for (int32_t i = 0; i < n_entries; ++i) {
    const muon_matrix_t& e = table[i];
    const Geom q = geom(e);
    EntryRec r{};
    r.offset = e.offset;
    r.rstep = q.pr * e.cols;
    r.span = (q.pr - 1) * e.cols + q.pc;
    r.cstep = static_cast<int32_t>(q.pc);
    r.ncb = static_cast<int32_t>(q.ncb);
    r.ld = static_cast<int32_t>(e.cols);
    r.w = static_cast<int32_t>(q.pc);
    if (windows == nullptr) {
      r.lo = 0;
      r.hi = e.rows * e.cols;
      r.p0 = e.offset;
    } else {
      r.lo = windows[i].lo;
      r.hi = windows[i].hi;
      r.p0 = windows[i].param_offset - windows[i].lo;
    }
    r.first = L.groups[entry_pos[i].first].first + static_cast<int32_t>(entry_pos[i].second);
    r.nblk_t = static_cast<int32_t>(((q.nrb * q.ncb) << 1) | (q.pr > q.pc ? 1 : 0));
    L.entries.push_back(r);
  }
  // momentum blocks: each problem is cut into blocks of kMomChunk elements; the
  // per-block partial sums of squares are laid out group by group, problem by problem
  for (Group& G : L.groups) {
    G.chunks = (G.m * G.n + kMomChunk - 1) / kMomChunk;
    G.partial_first = L.n_partials;
    L.n_partials += static_cast<size_t>(G.count) * static_cast<size_t>(G.chunks);
  }

  // workspace
  const size_t esz = static_cast<size_t>(element_size(h->ns_dtype));
  size_t off = 0;
  L.off_desc = off;
  off = align256(off + std::max<size_t>(L.problems.size(), 1) * kProblemDescBytes);
  L.off_partials = off;
  off = align256(off + L.n_partials * sizeof(double));
  L.off_invnorm = off;
  off = align256(off + L.problems.size() * sizeof(float));
  for (Group& G : L.groups) {
    const size_t cnt = static_cast<size_t>(G.count);
    const size_t xbytes = cnt * static_cast<size_t>(G.mp * G.np) * esz;
    const size_t sbytes = cnt * static_cast<size_t>(G.mp * G.mp) * esz;
    G.x[0] = off; off = align256(off + xbytes);
    if (h->ns_method == MUON_NS_STANDARD) {
      G.x[1] = off; off = align256(off + xbytes);
      G.a = off; off = align256(off + sbytes);
      G.b = off; off = align256(off + sbytes);
    } else if (G.mp == G.tile && h->ns_dtype != MUON_DTYPE_F32) {
      // single tile row in 16-bit: the chain runs in LDS; R0 and the final P
      G.a = off; off = align256(off + sbytes);      // R0
      G.p[0] = off; off = align256(off + sbytes);   // P
    } else {
      G.a = off; off = align256(off + sbytes);      // R
      G.r2 = off; off = align256(off + sbytes);     // next R
      G.b = off; off = align256(off + sbytes);      // Q
      G.p[0] = off; off = align256(off + sbytes);   // P
      G.p[1] = off; off = align256(off + sbytes);   // next P
      G.t = off; off = align256(off + sbytes);      // R Q
    }
  }
  L.ws_bytes = std::max<size_t>(off, 256);
  return L;
}

}  // namespace muon
