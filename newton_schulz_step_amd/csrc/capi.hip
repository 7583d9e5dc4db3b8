// C ABI of libmuonstep: argument checks, the per-table plan cache, and the
// launch sequence of one Muon step (momentum -> norms -> X0 -> Newton-Schulz
// chain -> fused apply), plus AdamW and pack/unpack.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "common.hpp"
#include "kernels.hpp"
#include "plan.hpp"
#include "planner.hpp"

namespace muon {

static thread_local std::string g_err;

static int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

// ---------------------------------------------------------------------------
// kernel timing (measurement hooks)

struct ProfRec {
  const char* kind;
  hipEvent_t a, b;
};

static std::mutex g_prof_mu;
static std::atomic<bool> g_prof_active{false};
static std::vector<ProfRec> g_prof;

template <typename F>
static hipError_t timed(const char* kind, hipStream_t s, F&& launch) {
  if (!g_prof_active.load(std::memory_order_acquire)) return launch();
  hipEvent_t a = nullptr, b = nullptr;
  if (hipEventCreate(&a) != hipSuccess) return hipErrorOutOfMemory;
  if (hipEventCreate(&b) != hipSuccess) {
    (void)hipEventDestroy(a);
    return hipErrorOutOfMemory;
  }
  (void)hipEventRecord(a, s);
  const hipError_t r = launch();
  (void)hipEventRecord(b, s);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof.push_back({kind, a, b});
  return r;
}

// A set of shape groups that share the tile edge; each NS product is one launch
// over all of them. Groups are ordered by decreasing n, so the tiles with the
// longest K (X X^T) are dispatched first and the short ones fill the tail.
// Groups with a single tile row (m <= 128) form sets of their own, which the
// standard iteration runs with the fused update + Gram kernel.
using GroupSet = std::vector<const Group*>;

static bool single_row(const Group& G) { return G.mp == G.tile; }

static std::vector<GroupSet> group_sets(const Layout& L) {
  std::vector<GroupSet> sets;
  for (int kind = 0; kind < 4; ++kind) {
    // 256-tiles with 256- or 128-tile symmetric launches; 128-tiles with more
    // than one tile row; single-tile-row groups
    const int tile = kind < 2 ? 256 : 128;
    GroupSet all;
    for (const Group& G : L.groups)
      if (G.tile == tile && (kind >= 2 ? single_row(G) == (kind == 3) : G.sym_tile == (kind == 0 ? 256 : 128)))
        all.push_back(&G);
    std::stable_sort(all.begin(), all.end(), [](const Group* x, const Group* y) { return x->n > y->n; });
    for (size_t i = 0; i < all.size(); i += kBatchGroups)
      sets.emplace_back(all.begin() + i, all.begin() + std::min(all.size(), i + kBatchGroups));
  }
  return sets;
}

// ---------------------------------------------------------------------------
// plan cache: the host layout of a step per (table, windows, method, dtypes).
// It is host memory only: a step writes its per-problem descriptors into the
// caller's workspace on the stream, so no device memory is owned here and
// dropping a plan (cache full, or muon_release_plans) never touches the device.
// A plan is shared: a call holds it while it enqueues its launches.

struct Plan {
  Layout L;
  std::vector<GroupSet> sets;   // shape groups launched together
};

// The cache is never destroyed (calls may still run during process teardown).
static std::mutex g_plan_mu;
static auto& g_plans = *new std::map<std::string, std::shared_ptr<const Plan>>();
static constexpr size_t kMaxPlans = 1024;

static std::string plan_key(const muon_matrix_t* t, const muon_window_t* w, int32_t n, const muon_hyper_t* h) {
  std::string k;
  const int32_t hdr[5] = {n, h->ns_method, h->ns_dtype, h->grad_dtype, w != nullptr};
  k.append(reinterpret_cast<const char*>(hdr), sizeof(hdr));
  if (n > 0) k.append(reinterpret_cast<const char*>(t), sizeof(muon_matrix_t) * static_cast<size_t>(n));
  if (n > 0 && w) k.append(reinterpret_cast<const char*>(w), sizeof(muon_window_t) * static_cast<size_t>(n));
  return k;
}

static int get_plan(const muon_matrix_t* t, const muon_window_t* w, int32_t n, const muon_hyper_t* h,
                    size_t workspace_bytes, std::shared_ptr<const Plan>& out) {
  const std::string key = plan_key(t, w, n, h);
  {
    std::lock_guard<std::mutex> lk(g_plan_mu);
    auto it = g_plans.find(key);
    if (it != g_plans.end()) out = it->second;
  }
  if (!out) {
    auto p = std::make_shared<Plan>();
    p->L = build_layout(t, n, h, w);
    p->sets = group_sets(p->L);
    std::lock_guard<std::mutex> lk(g_plan_mu);
    if (g_plans.size() >= kMaxPlans) g_plans.clear();
    auto ins = g_plans.emplace(key, std::move(p));   // another thread may have built it first
    out = ins.first->second;
  }
  if (workspace_bytes < out->L.ws_bytes)
    return fail(MUON_ERR_WORKSPACE, "workspace too small: need " + std::to_string(out->L.ws_bytes) + " bytes");
  return MUON_OK;
}

// ---------------------------------------------------------------------------
// helpers

static bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

struct Span {
  const char* lo;
  const char* hi;
  const char* name;
};

static bool overlapping(const std::vector<Span>& v, std::string& which) {
  for (size_t i = 0; i < v.size(); ++i)
    for (size_t j = i + 1; j < v.size(); ++j)
      if (v[i].lo < v[j].hi && v[j].lo < v[i].hi) {
        which = std::string(v[i].name) + " and " + v[j].name;
        return true;
      }
  return false;
}

#define MUON_LAUNCH(kind, stream, expr)                                                        \
  do {                                                                                         \
    const hipError_t _e = timed(kind, stream, [&]() { return (expr); });                      \
    if (_e != hipSuccess)                                                                      \
      return fail(MUON_ERR_HIP, std::string(kind) + " launch failed: " + hipGetErrorString(_e)); \
  } while (0)

static float gram_scale(int64_t m) {
  int e = 0;
  while ((int64_t(1) << e) < m && e < 15) ++e;
  return static_cast<float>(int64_t(1) << e);
}

// Contraction length of a product over a dimension of `len` valid elements: the
// buffers are zero beyond `len` (up to the tile-padded extent), so the K loop
// stops at the next multiple of two 128-byte slices instead of the padded extent.
// (Gram's Q carries a on its padded diagonal, but padded and valid indices never
// meet in one product term: the valid block of every result is unchanged.)
static int64_t kext(int64_t len, int dtype) {
  const int64_t q = dtype == MUON_DTYPE_F32 ? 64 : 128;
  return (len + q - 1) / q * q;
}

struct StepCtx {
  const Plan* P;
  const ProblemDesc* probs;   // the step's descriptors, in the workspace
  const muon_hyper_t* h;
  char* ws;
  const float* M;
  void* params;               // fp32 or bf16 (h->param_dtype)
  float* update_out;
  uint16_t* shadow;
  float decay;
  hipStream_t s;
};

static int apply_epi(const StepCtx& c) { return c.h->param_dtype == MUON_DTYPE_BF16 ? EPI_APPLY_BF16 : EPI_APPLY; }

static GemmArgs apply_args(const StepCtx& c, const Group& G) {
  GemmArgs g{};
  g.params = c.params;
  g.probs = c.probs + G.first;
  g.m_valid = static_cast<int32_t>(G.m);
  g.n_valid = static_cast<int32_t>(G.n);
  g.decay = c.decay;
  g.lr = c.h->lr;
  g.update_out = c.update_out;
  g.shadow = c.shadow;
  return g;
}

// C = alpha * P Q^T (+ beta D + gamma I) over the problems of a group, symmetric
// (lower tiles, mirrored); both operands K-contiguous.
static void set_sym(GemmArgs& g, const Group& G, const void* P, const void* Q, int64_t K, int64_t ldpq, int64_t pq_ps,
                    void* C) {
  // tiles of G.sym_tile up to m (rounded up): with 128-tiles in a 256-padded
  // buffer, the padding beyond them is never written, and never read into a
  // valid result either (every K loop stops at m rounded to 128, and the full
  // launches' extra rows are output rows that nothing reads)
  const int T = static_cast<int>((G.m + G.sym_tile - 1) / G.sym_tile);
  g.P = P; g.p_ps = pq_ps; g.ldp = static_cast<int32_t>(ldpq);
  g.Q = Q; g.q_ps = pq_ps; g.ldq = static_cast<int32_t>(ldpq);
  g.K = static_cast<int32_t>(K);
  g.tiles_m = T; g.tiles_n = T;
  g.tiles_per_problem = T * (T + 1) / 2;
  g.total_tiles = g.tiles_per_problem * G.count;
  g.C = C; g.c_ps = G.mp * G.mp; g.ldc = static_cast<int32_t>(G.mp);
  g.Ct = C; g.ct_ps = G.mp * G.mp; g.ldct = static_cast<int32_t>(G.mp);
}

// C = alpha * P Q (+ beta D) over the problems of a group: P rows x K
// (K-contiguous), Q K x cols (cols contiguous).
static void set_full(GemmArgs& g, const Group& G, const void* P, int64_t p_ps, int64_t ldp, const void* Q,
                     int64_t q_ps, int64_t ldq, int64_t K, int64_t rows, int64_t cols) {
  g.P = P; g.p_ps = p_ps; g.ldp = static_cast<int32_t>(ldp);
  g.Q = Q; g.q_ps = q_ps; g.ldq = static_cast<int32_t>(ldq);
  g.K = static_cast<int32_t>(K);
  g.tiles_m = static_cast<int32_t>(rows / G.tile);
  g.tiles_n = static_cast<int32_t>(cols / G.tile);
  g.tiles_per_problem = g.tiles_m * g.tiles_n;
  g.total_tiles = g.tiles_per_problem * G.count;
}

static GemmBatch make_batch(const std::vector<GemmArgs>& v) {
  GemmBatch b{};
  b.n = static_cast<int32_t>(v.size());
  b.start[0] = 0;
  for (size_t g = 0; g < v.size(); ++g) {
    b.g[g] = v[g];
    b.start[g + 1] = b.start[g] + v[g].total_tiles;
  }
  return b;
}

// One launch of `kind` over the per-group arguments `v` (at most kBatchGroups).
static int launch_batch(const char* kind, const StepCtx& c, int tile, bool sym, int epi,
                        const std::vector<GemmArgs>& v) {
  const GemmBatch b = make_batch(v);
  MUON_LAUNCH(kind, c.s, launch_ns_gemm(c.h->ns_dtype, tile, sym, epi, b, c.s));
  return MUON_OK;
}

// Groups whose symmetric launches use smaller tiles than their full launches
// leave the padding rows of their m x m results unwritten; the full launches
// read them as operand rows (of results nobody reads), so they are zeroed once
// per call: rows round_up(m, sym_tile) .. mp - 1 of every problem's buffer.
static int zero_sym_padding(const StepCtx& c, const Group& G, size_t off) {
  if (G.sym_tile == G.tile) return MUON_OK;
  const int64_t esz = element_size(c.h->ns_dtype);
  const int64_t r0 = (G.m + G.sym_tile - 1) / G.sym_tile * G.sym_tile;
  if (r0 >= G.mp) return MUON_OK;
  MUON_LAUNCH("zero_padding", c.s,
              launch_zero_regions(c.ws + off + r0 * G.mp * esz, G.mp * G.mp * esz, (G.mp - r0) * G.mp * esz, G.count,
                                  c.s));
  return MUON_OK;
}

// X0 of every problem of the group (canonical m x n, row-major).
static int run_prep(const StepCtx& c, const Group& G) {
  const float* invn = reinterpret_cast<const float*>(c.ws + c.P->L.off_invnorm) + G.first;
  MUON_LAUNCH("prep_x0", c.s,
              launch_prep_x0(c.h->ns_dtype, c.M, c.probs + G.first, invn, G.count, static_cast<int>(G.m),
                             static_cast<int>(G.n), static_cast<int>(G.mp), static_cast<int>(G.np), c.ws + G.x[0],
                             c.s));
  return MUON_OK;
}

// Single-tile-row group in 16-bit: X0 and R = alpha X0 X0^T in one pass.
static int run_prep_gram(const StepCtx& c, const Group& G, void* R, float alpha) {
  PrepGramArgs a{};
  a.M = c.M;
  a.probs = c.probs + G.first;
  a.inv_norm = reinterpret_cast<const float*>(c.ws + c.P->L.off_invnorm) + G.first;
  a.X = c.ws + G.x[0];
  a.R = R;
  a.m = static_cast<int32_t>(G.m); a.n = static_cast<int32_t>(G.n);
  a.mp = static_cast<int32_t>(G.mp); a.np = static_cast<int32_t>(G.np);
  a.n_problems = G.count;
  a.alpha = alpha;
  MUON_LAUNCH("prep_gram", c.s, launch_prep_gram(c.h->ns_dtype, a, c.s));
  return MUON_OK;
}

// Standard quintic (DeepSpeed-Muon article, section 核心算子): per step
//   A = X X^T;  B = a I + b A + c A A;  X <- B X,
// (a X + (b A + c A A) X with the a X term grouped into the stored B, as the
// Gram form groups a I into Q), the last step's epilogue applying
// p <- p * decay - lr * X.
static int run_standard(const StepCtx& c, const GroupSet& set) {
  const int dt = c.h->ns_dtype;
  const int tile = set.front()->tile;
  // single-tile-row groups in 16-bit: X X^T of each new X comes out of the update
  const bool fused = single_row(*set.front()) && dt != MUON_DTYPE_F32;
  char* ws = c.ws;
  int st;
  for (const Group* G : set) {
    if ((st = fused ? run_prep_gram(c, *G, ws + G->a, 1.0f) : run_prep(c, *G)) != MUON_OK) return st;
    if ((st = zero_sym_padding(c, *G, G->b)) != MUON_OK) return st;   // B: the full launches' left operand
  }
  int cur = 0;
  for (int k = 0; k < c.h->ns_steps; ++k) {
    const bool last = (k == c.h->ns_steps - 1);
    std::vector<GemmArgs> v1, v2, v3;
    for (const Group* Gp : set) {
      const Group& G = *Gp;
      void* X[2] = {ws + G.x[0], ws + G.x[1]};
      void* A = ws + G.a;
      void* B = ws + G.b;
      const int64_t xs = G.mp * G.np, ss = G.mp * G.mp;
      GemmArgs g1{};
      set_sym(g1, G, X[cur], X[cur], kext(G.n, dt), G.np, xs, A);
      g1.alpha = 1.0f;
      v1.push_back(g1);

      // B = a I + b A + c A A (the a X term grouped into B)
      GemmArgs g2{};
      set_sym(g2, G, A, A, kext(G.m, dt), G.mp, ss, B);
      g2.alpha = c.h->ns_c;
      g2.beta = c.h->ns_b;
      g2.gamma = c.h->ns_a;
      g2.D = A; g2.d_ps = ss; g2.ldd = static_cast<int32_t>(G.mp);
      v2.push_back(g2);

      // B X with X itself as the K x N operand
      GemmArgs g3 = last ? apply_args(c, G) : GemmArgs{};
      set_full(g3, G, B, ss, G.mp, X[cur], xs, G.np, kext(G.m, dt), G.mp, G.np);
      g3.alpha = 1.0f;
      if (!last) { g3.C = X[cur ^ 1]; g3.c_ps = xs; g3.ldc = static_cast<int32_t>(G.np); }
      if (fused && !last) {
        // one block per problem; the new X X^T goes to A (already consumed by B)
        g3.K = static_cast<int32_t>(G.mp);
        g3.total_tiles = G.count;
        g3.Ct = A; g3.ct_ps = ss; g3.ldct = static_cast<int32_t>(G.mp);
      }
      v3.push_back(g3);
    }
    if (!fused)
      if ((st = launch_batch("ns_gemm_xxt", c, set.front()->sym_tile, true, EPI_STORE, v1)) != MUON_OK) return st;
    if ((st = launch_batch("ns_gemm_poly", c, set.front()->sym_tile, true, EPI_STORE, v2)) != MUON_OK) return st;
    if (!last) {
      if (fused) {
        const GemmBatch b = make_batch(v3);
        MUON_LAUNCH("ns_update_gram", c.s, launch_update_gram(dt, b, c.s));
      } else if ((st = launch_batch("ns_gemm_update", c, tile, false, EPI_STORE, v3)) != MUON_OK) {
        return st;
      }
      cur ^= 1;
    } else {
      if ((st = launch_batch("ns_gemm_apply", c, tile, false, apply_epi(c), v3)) != MUON_OK) return st;
    }
  }
  return MUON_OK;
}

// Gram variant (same section): R0 = s X0 X0^T (s an exact power of two keeping
// R's entries in fp16's normal range; b and c are rescaled to match); per step
//   Q = a I + (b/s) R + (c/s^2) R R;  P <- Q P (P = Q first);  R <- Q (R Q)
// (not after the last step); finally X = P X0 with the apply fused. R, Q and
// R Q are symmetric and computed as such (lower tiles, mirrored); P is computed
// in full.
static int run_gram(const StepCtx& c, const GroupSet& set) {
  const int dt = c.h->ns_dtype;
  const int tile = set.front()->tile;
  const int S = c.h->ns_steps;
  char* ws = c.ws;
  int st;
  auto scale = [&](const Group& G) { return (dt == MUON_DTYPE_F16) ? gram_scale(G.m) : 1.0f; };
  auto R = [&](const Group& G, int i) -> void* { return ws + (i == 0 ? G.a : G.r2); };
  auto Pb = [&](const Group& G, int i) -> void* { return ws + G.p[i]; };
  // single-tile-row groups in 16-bit: X0 and R0 in one pass
  const bool fused = single_row(*set.front()) && dt != MUON_DTYPE_F32;

  std::vector<GemmArgs> v;
  if (fused) {
    // X0 and R0 in one pass; then the whole chain in one launch, with the small
    // matrices in LDS (the same products and roundings as the launches below);
    // then X = P X0 with the apply fused, as below
    GramChainBatch b{};
    b.n = static_cast<int32_t>(set.size());
    for (size_t gi = 0; gi < set.size(); ++gi) {
      const Group& G = *set[gi];
      if ((st = run_prep_gram(c, G, R(G, 0), scale(G))) != MUON_OK) return st;
      const float s = scale(G);
      GramChainArgs& x = b.g[gi];
      x.R0 = R(G, 0);
      x.r_ps = G.mp * G.mp;
      x.P = Pb(G, 0);
      x.p_ps = G.mp * G.mp;
      x.qa = c.h->ns_a;
      x.qb = c.h->ns_b / s;
      x.qc = c.h->ns_c / (s * s);
      x.steps = S;
      x.count = G.count;
      b.start[gi + 1] = b.start[gi] + G.count;
    }
    MUON_LAUNCH("gram_chain", c.s, launch_gram_chain(dt, b, c.s));
    for (const Group* Gp : set) {
      const Group& G = *Gp;
      GemmArgs ga = apply_args(c, G);
      set_full(ga, G, Pb(G, 0), G.mp * G.mp, G.mp, ws + G.x[0], G.mp * G.np, G.np, kext(G.m, dt), G.mp, G.np);
      ga.alpha = 1.0f;
      v.push_back(ga);
    }
    return launch_batch("gram_gemm_apply", c, tile, false, apply_epi(c), v);
  } else {
    for (const Group* G : set) {
      if ((st = run_prep(c, *G)) != MUON_OK) return st;
      // every Q is the left operand of a full launch: the first one is written to P
      if ((st = zero_sym_padding(c, *G, G->p[0])) != MUON_OK) return st;
      if ((st = zero_sym_padding(c, *G, G->b)) != MUON_OK) return st;
    }
    for (const Group* Gp : set) {
      const Group& G = *Gp;
      GemmArgs r0{};
      set_sym(r0, G, ws + G.x[0], ws + G.x[0], kext(G.n, dt), G.np, G.mp * G.np, R(G, 0));
      r0.alpha = scale(G);
      v.push_back(r0);
    }
    if ((st = launch_batch("gram_gemm_sym", c, set.front()->sym_tile, true, EPI_STORE, v)) != MUON_OK) return st;
  }

  int rc = 0, pc = 0;
  for (int k = 0; k < S; ++k) {
    // Q_k (symmetric); on the first step it is also P
    auto Qdst = [&](const Group& G) -> void* { return k == 0 ? Pb(G, 0) : ws + G.b; };
    v.clear();
    for (const Group* Gp : set) {
      const Group& G = *Gp;
      const int64_t ss = G.mp * G.mp;
      const float s = scale(G);
      GemmArgs gq{};
      set_sym(gq, G, R(G, rc), R(G, rc), kext(G.m, dt), G.mp, ss, Qdst(G));
      gq.alpha = c.h->ns_c / (s * s);
      gq.beta = c.h->ns_b / s;
      gq.gamma = c.h->ns_a;
      gq.D = R(G, rc); gq.d_ps = ss; gq.ldd = static_cast<int32_t>(G.mp);
      v.push_back(gq);
    }
    if ((st = launch_batch("gram_gemm_sym", c, set.front()->sym_tile, true, EPI_STORE, v)) != MUON_OK) return st;
    if (k > 0) {
      // P <- Q P, P row-major as the K x N operand
      v.clear();
      for (const Group* Gp : set) {
        const Group& G = *Gp;
        const int64_t ss = G.mp * G.mp;
        GemmArgs gp{};
        set_full(gp, G, Qdst(G), ss, G.mp, Pb(G, pc), ss, G.mp, kext(G.m, dt), G.mp, G.mp);
        gp.alpha = 1.0f;
        gp.C = Pb(G, pc ^ 1); gp.c_ps = ss; gp.ldc = static_cast<int32_t>(G.mp);
        v.push_back(gp);
      }
      if ((st = launch_batch("gram_gemm_full", c, tile, false, EPI_STORE, v)) != MUON_OK) return st;
      pc ^= 1;
    }
    if (k < S - 1) {
      // T = R Q, symmetric (R and Q commute): lower tiles, mirrored; Q is stored
      // symmetric, so R Q = R Q^T
      v.clear();
      for (const Group* Gp : set) {
        const Group& G = *Gp;
        GemmArgs gt{};
        set_sym(gt, G, R(G, rc), Qdst(G), kext(G.m, dt), G.mp, G.mp * G.mp, ws + G.t);
        gt.alpha = 1.0f;
        v.push_back(gt);
      }
      if ((st = launch_batch("gram_gemm_sym", c, set.front()->sym_tile, true, EPI_STORE, v)) != MUON_OK) return st;
      // R <- Q T (symmetric: lower tiles, mirrored)
      v.clear();
      for (const Group* Gp : set) {
        const Group& G = *Gp;
        GemmArgs gr{};
        set_sym(gr, G, Qdst(G), ws + G.t, kext(G.m, dt), G.mp, G.mp * G.mp, R(G, rc ^ 1));
        gr.alpha = 1.0f;
        v.push_back(gr);
      }
      if ((st = launch_batch("gram_gemm_sym", c, set.front()->sym_tile, true, EPI_STORE, v)) != MUON_OK) return st;
      rc ^= 1;
    }
  }
  // X = P X0, X0 row-major as the K x N operand, with the apply fused
  v.clear();
  for (const Group* Gp : set) {
    const Group& G = *Gp;
    GemmArgs ga = apply_args(c, G);
    set_full(ga, G, Pb(G, pc), G.mp * G.mp, G.mp, ws + G.x[0], G.mp * G.np, G.np, kext(G.m, dt), G.mp, G.np);
    ga.alpha = 1.0f;
    v.push_back(ga);
  }
  return launch_batch("gram_gemm_apply", c, tile, false, apply_epi(c), v);
}

}  // namespace muon

using namespace muon;

extern "C" {

const char* muon_version(void) { return "libmuonstep 0.1 (gfx950)"; }

const char* muon_last_error(void) { return g_err.c_str(); }

void muon_default_hyper(muon_hyper_t* h) {
  if (!h) return;
  h->lr = 0.02f;
  h->momentum = 0.95f;
  h->weight_decay = 0.0f;
  h->ns_a = 3.4445f;
  h->ns_b = -4.7750f;
  h->ns_c = 2.0315f;
  h->ns_steps = 5;
  h->ns_eps = 1e-7f;
  h->ns_method = MUON_NS_GRAM;
  h->param_dtype = MUON_DTYPE_F32;
  h->grad_dtype = MUON_DTYPE_BF16;
  h->ns_dtype = MUON_DTYPE_F16;
}

void muon_default_adamw_hyper(muon_adamw_hyper_t* h) {
  if (!h) return;
  h->lr = 3e-4f;
  h->beta1 = 0.9f;
  h->beta2 = 0.95f;
  h->eps = 1e-10f;
  h->weight_decay = 0.0f;
  h->step = 1;
  h->grad_dtype = MUON_DTYPE_BF16;
}

int muon_workspace_size(const muon_matrix_t* table, int32_t n_entries, const muon_hyper_t* h, size_t* bytes_out) {
  g_err.clear();
  if (bytes_out == nullptr) return fail(MUON_ERR_NULL, "bytes_out is NULL");
  std::string err;
  const int st = validate(table, n_entries, h, err);
  if (st != MUON_OK) return fail(st, err);
  *bytes_out = build_layout(table, n_entries, h).ws_bytes;
  return MUON_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// muon_step_noalloc's workspace: a file-scope device array, one copy per GPU
// (held until the process ends). Host code never uses the array's name as an
// address: each device's copy is found once with hipGetSymbolAddress, with that
// device current, and that pointer is what the kernels receive.

namespace muon {

static __device__ __align__(256) char scratch[MUON_NOALLOC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up on the first call on it).
static int scratch_for_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MUON_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return fail(MUON_ERR_HIP, "device index beyond the library's table");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(MUON_ERR_HIP, std::string("hipGetSymbolAddress of the step scratch failed: ") +
                                    hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MUON_OK;
}

}  // namespace muon

extern "C" {

// The shared body of muon_step and muon_step_window. `windows` NULL: params and
// the shadow share the table's layout (params_numel == numel).
static int step_impl(void* params, int64_t params_numel, const void* grads, float* momentum, int64_t numel,
                     const muon_matrix_t* table, const muon_window_t* windows, int32_t n_entries,
                     const muon_hyper_t* h, void* workspace, size_t workspace_bytes, float* update_out,
                     uint16_t* bf16_shadow, void* stream, bool use_scratch = false) {
  g_err.clear();
  std::string err;
  int st = validate(table, n_entries, h, err);
  if (st != MUON_OK) return fail(st, err);
  if (params == nullptr || grads == nullptr || momentum == nullptr)
    return fail(MUON_ERR_NULL, "params, grads and momentum must not be NULL");
  if (numel < 0) return fail(MUON_ERR_RANGE, "numel < 0");
  for (int32_t i = 0; i < n_entries; ++i)
    if (table[i].offset + table[i].rows * table[i].cols > numel)
      return fail(MUON_ERR_RANGE, "entry " + std::to_string(i) + " ends beyond numel");
  if (windows) {
    if (h->param_dtype != MUON_DTYPE_F32)
      return fail(MUON_ERR_UNSUPPORTED, "a partition holder's step takes float32 params only");
    st = validate_windows(table, windows, n_entries, params_numel, err);
    if (st != MUON_OK) return fail(st, err);
  }
  if (bf16_shadow && h->param_dtype == MUON_DTYPE_BF16)
    return fail(MUON_ERR_UNSUPPORTED, "bf16 params are their own bf16 copy: pass no bf16_shadow");
  if (n_entries == 0 || numel == 0) return MUON_OK;
  if (use_scratch) {
    // muon_step_noalloc: the library's device array, once the table is known to fit
    const size_t need = build_layout(table, n_entries, h, windows).ws_bytes;
    if (need > MUON_NOALLOC_WORKSPACE_BYTES)
      return fail(MUON_ERR_WORKSPACE, "the table needs " + std::to_string(need) +
                                          " bytes of workspace; muon_step_noalloc has " +
                                          std::to_string(static_cast<size_t>(MUON_NOALLOC_WORKSPACE_BYTES)));
    if ((st = scratch_for_current_device(&workspace)) != MUON_OK) return st;
    workspace_bytes = MUON_NOALLOC_WORKSPACE_BYTES;
  }
  if (workspace == nullptr) return fail(MUON_ERR_NULL, "workspace is NULL");
  if (misaligned(params, 16) || misaligned(grads, 16) || misaligned(momentum, 16) ||
      (update_out && misaligned(update_out, 16)) || (bf16_shadow && misaligned(bf16_shadow, 16)))
    return fail(MUON_ERR_ALIGN, "a buffer pointer is not 16-byte aligned");
  if (misaligned(workspace, 256)) return fail(MUON_ERR_ALIGN, "workspace is not 256-byte aligned");
  const size_t gsz = static_cast<size_t>(element_size(h->grad_dtype));
  const size_t psz = static_cast<size_t>(element_size(h->param_dtype));
  const size_t ne = static_cast<size_t>(numel), pe = static_cast<size_t>(params_numel);
  const char* pname = windows ? "partition" : "params";
  std::vector<Span> spans = {
      {static_cast<const char*>(params), static_cast<const char*>(params) + pe * psz, pname},
      {static_cast<const char*>(grads), static_cast<const char*>(grads) + ne * gsz, "grads"},
      {reinterpret_cast<const char*>(momentum), reinterpret_cast<const char*>(momentum) + ne * 4, "momentum"},
      {static_cast<const char*>(workspace), static_cast<const char*>(workspace) + workspace_bytes, "workspace"}};
  if (update_out)
    spans.push_back({reinterpret_cast<const char*>(update_out), reinterpret_cast<const char*>(update_out) + ne * 4,
                     "update_out"});
  if (bf16_shadow)
    spans.push_back({reinterpret_cast<const char*>(bf16_shadow), reinterpret_cast<const char*>(bf16_shadow) + pe * 2,
                     "bf16_shadow"});
  std::string which;
  if (overlapping(spans, which)) return fail(MUON_ERR_OVERLAP, "buffers overlap: " + which);

  std::shared_ptr<const Plan> plan;
  st = get_plan(table, windows, n_entries, h, workspace_bytes, plan);
  if (st != MUON_OK) return st;
  const Plan* P = plan.get();

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  ProblemDesc* probs = reinterpret_cast<ProblemDesc*>(ws + P->L.off_desc);
  double* partials = reinterpret_cast<double*>(ws + P->L.off_partials);
  float* invn = reinterpret_cast<float*>(ws + P->L.off_invnorm);
  const float mu = h->momentum;
  MUON_LAUNCH("expand_desc", s,
              launch_expand_desc(P->L.entries.data(), static_cast<int>(P->L.entries.size()), probs, s));
  for (const Group& G : P->L.groups)
    MUON_LAUNCH("momentum_sumsq", s,
                launch_momentum_sumsq(h->grad_dtype, momentum, grads, probs + G.first, G.count, G.m * G.n,
                                      G.chunks, mu, partials + G.partial_first, s));
  for (const Group& G : P->L.groups)
    MUON_LAUNCH("finalize_norm", s,
                launch_finalize_norm(partials + G.partial_first, G.chunks, G.count, h->ns_eps, invn + G.first, s));
  StepCtx c{P, probs, h, ws, momentum, params, update_out, bf16_shadow,
            static_cast<float>(1.0 - static_cast<double>(h->lr) * static_cast<double>(h->weight_decay)), s};
  for (const GroupSet& set : P->sets) {
    st = (h->ns_method == MUON_NS_STANDARD) ? run_standard(c, set) : run_gram(c, set);
    if (st != MUON_OK) return st;
  }
  return MUON_OK;
}

int muon_step(void* params, const void* grads, float* momentum, int64_t numel, const muon_matrix_t* table,
              int32_t n_entries, const muon_hyper_t* h, void* workspace, size_t workspace_bytes, float* update_out,
              uint16_t* bf16_shadow, void* stream) {
  return step_impl(params, numel, grads, momentum, numel, table, nullptr, n_entries, h,
                   workspace, workspace_bytes, update_out, bf16_shadow, stream);
}

int muon_step_noalloc(void* params, const void* grads, float* momentum, int64_t numel, const muon_matrix_t* table,
                      int32_t n_entries, const muon_hyper_t* h, float* update_out, uint16_t* bf16_shadow,
                      void* stream) {
  return step_impl(params, numel, grads, momentum, numel, table, nullptr, n_entries, h, nullptr, 0, update_out,
                   bf16_shadow, stream, /*use_scratch=*/true);
}

int muon_step_window(float* partition, int64_t partition_numel, const void* grads, float* momentum, int64_t numel,
                     const muon_matrix_t* table, const muon_window_t* windows, int32_t n_entries,
                     const muon_hyper_t* h, void* workspace, size_t workspace_bytes, float* update_out,
                     uint16_t* bf16_shadow, void* stream) {
  if (n_entries > 0 && windows == nullptr) {
    g_err.clear();
    return fail(MUON_ERR_NULL, "windows is NULL");
  }
  return step_impl(partition, partition_numel, grads, momentum, numel, table, windows,
                   n_entries, h, workspace, workspace_bytes, update_out, bf16_shadow, stream);
}

int adamw_step(float* params, const void* grads, float* m, float* v, int64_t numel, const muon_adamw_hyper_t* h,
               void* stream) {
  g_err.clear();
  if (h == nullptr) return fail(MUON_ERR_NULL, "hyperparameter pointer is NULL");
  if (numel < 0) return fail(MUON_ERR_RANGE, "numel < 0");
  const float fs[] = {h->lr, h->beta1, h->beta2, h->eps, h->weight_decay};
  for (float f : fs)
    if (!std::isfinite(f)) return fail(MUON_ERR_BAD_HYPER, "a hyperparameter is not finite");
  if (h->step < 1) return fail(MUON_ERR_BAD_HYPER, "step must be >= 1");
  if (h->beta1 < 0.0f || h->beta1 >= 1.0f || h->beta2 < 0.0f || h->beta2 >= 1.0f)
    return fail(MUON_ERR_BAD_HYPER, "betas must lie in [0, 1)");
  const int gsz = element_size(h->grad_dtype);
  if (gsz == 0) return fail(MUON_ERR_UNSUPPORTED, "grad_dtype must be F32, BF16 or F16");
  if (numel == 0) return MUON_OK;
  if (!params || !grads || !m || !v) return fail(MUON_ERR_NULL, "params, grads, m and v must not be NULL");
  if (misaligned(params, 16) || misaligned(grads, 16) || misaligned(m, 16) || misaligned(v, 16))
    return fail(MUON_ERR_ALIGN, "a buffer pointer is not 16-byte aligned");
  const size_t ne = static_cast<size_t>(numel);
  std::vector<Span> spans = {
      {reinterpret_cast<const char*>(params), reinterpret_cast<const char*>(params) + ne * 4, "params"},
      {static_cast<const char*>(grads), static_cast<const char*>(grads) + ne * gsz, "grads"},
      {reinterpret_cast<const char*>(m), reinterpret_cast<const char*>(m) + ne * 4, "m"},
      {reinterpret_cast<const char*>(v), reinterpret_cast<const char*>(v) + ne * 4, "v"}};
  std::string which;
  if (overlapping(spans, which)) return fail(MUON_ERR_OVERLAP, "buffers overlap: " + which);
  const double bc1 = 1.0 - pow(static_cast<double>(h->beta1), h->step);
  const double bc2 = 1.0 - pow(static_cast<double>(h->beta2), h->step);
  const float step_size = static_cast<float>(static_cast<double>(h->lr) / bc1);
  const float inv_bc2 = static_cast<float>(1.0 / bc2);
  const float decay = static_cast<float>(1.0 - static_cast<double>(h->lr) * static_cast<double>(h->weight_decay));
  hipStream_t s = static_cast<hipStream_t>(stream);
  MUON_LAUNCH("adamw", s,
              launch_adamw(h->grad_dtype, params, grads, m, v, numel, h->beta1, h->beta2, step_size, inv_bc2, h->eps,
                           decay, s));
  return MUON_OK;
}

static int check_pack_table(const muon_matrix_t* table, int32_t n, int64_t numel, int32_t dtype) {
  if (element_size(dtype) == 0) return fail(MUON_ERR_UNSUPPORTED, "dtype must be F32, BF16 or F16");
  muon_hyper_t h;
  muon_default_hyper(&h);
  h.ns_method = MUON_NS_STANDARD;
  std::string err;
  const int st = validate(table, n, &h, err);
  if (st != MUON_OK) return fail(st, err);
  for (int32_t i = 0; i < n; ++i)
    if (table[i].offset + table[i].rows * table[i].cols > numel)
      return fail(MUON_ERR_RANGE, "entry " + std::to_string(i) + " ends beyond numel");
  return MUON_OK;
}

static int run_copies(const std::vector<CopyItem>& items, hipStream_t s) {
  for (size_t i = 0; i < items.size(); i += kCopyBatch) {
    const int n = static_cast<int>(std::min<size_t>(kCopyBatch, items.size() - i));
    MUON_LAUNCH("copy_batch", s, launch_copy_batch(items.data() + i, n, s));
  }
  return MUON_OK;
}

int muon_pack(void* packed, int64_t numel, const void* const* srcs, const muon_matrix_t* table, int32_t n_entries,
              int32_t dtype, void* stream) {
  g_err.clear();
  int st = check_pack_table(table, n_entries, numel, dtype);
  if (st != MUON_OK) return st;
  if (n_entries == 0) return MUON_OK;
  if (!packed || !srcs) return fail(MUON_ERR_NULL, "packed and srcs must not be NULL");
  const size_t esz = static_cast<size_t>(element_size(dtype));
  std::vector<CopyItem> items;
  for (int32_t i = 0; i < n_entries; ++i) {
    if (!srcs[i]) return fail(MUON_ERR_NULL, "srcs[" + std::to_string(i) + "] is NULL");
    items.push_back({srcs[i], static_cast<char*>(packed) + table[i].offset * esz,
                     static_cast<int64_t>(table[i].rows * table[i].cols * esz)});
  }
  return run_copies(items, static_cast<hipStream_t>(stream));
}

int muon_unpack(void* const* dsts, const void* packed, int64_t numel, const muon_matrix_t* table, int32_t n_entries,
                int32_t dtype, void* stream) {
  g_err.clear();
  int st = check_pack_table(table, n_entries, numel, dtype);
  if (st != MUON_OK) return st;
  if (n_entries == 0) return MUON_OK;
  if (!packed || !dsts) return fail(MUON_ERR_NULL, "packed and dsts must not be NULL");
  const size_t esz = static_cast<size_t>(element_size(dtype));
  std::vector<CopyItem> items;
  for (int32_t i = 0; i < n_entries; ++i) {
    if (!dsts[i]) return fail(MUON_ERR_NULL, "dsts[" + std::to_string(i) + "] is NULL");
    items.push_back({static_cast<const char*>(packed) + table[i].offset * esz, dsts[i],
                     static_cast<int64_t>(table[i].rows * table[i].cols * esz)});
  }
  return run_copies(items, static_cast<hipStream_t>(stream));
}

int64_t muon_ns_flops(int64_t m, int64_t n, int32_t ns_method, int32_t steps) {
  return ns_flops(m, n, ns_method, steps);
}

int muon_plan_owners(const muon_param_t* params, int32_t n_params, int32_t n_owners, int32_t ns_method,
                     int32_t ns_steps, int64_t align, muon_assign_t* assign, muon_owner_t* owners) {
  g_err.clear();
  std::string err;
  const int st = plan_owners(params, n_params, n_owners, ns_method, ns_steps, align, assign, owners, err);
  return st == MUON_OK ? MUON_OK : fail(st, err);
}

double muon_comm_elements(int64_t p_m, int32_t n_ranks, int32_t zero_stage, int32_t dedicated) {
  return comm_elements(p_m, n_ranks, zero_stage, dedicated);
}

int muon_release_plans(void) {
  g_err.clear();
  std::lock_guard<std::mutex> lk(g_plan_mu);
  g_plans.clear();
  return MUON_OK;
}

int muon_profile_begin(void) {
  g_err.clear();
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& r : g_prof) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_prof.clear();
  g_prof_active.store(true, std::memory_order_release);
  return MUON_OK;
}

int muon_profile_end(muon_kernel_stat_t* out, int32_t max_kinds, int32_t* n_kinds_out) {
  g_err.clear();
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_active.store(false, std::memory_order_release);
  std::vector<muon_kernel_stat_t> stats;
  int status = MUON_OK;
  for (auto& r : g_prof) {
    float ms = 0.0f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
      status = fail(MUON_ERR_HIP, "reading kernel timing events failed");
    }
    muon_kernel_stat_t* k = nullptr;
    for (auto& s : stats)
      if (strncmp(s.name, r.kind, sizeof(s.name)) == 0) k = &s;
    if (!k) {
      muon_kernel_stat_t s{};
      strncpy(s.name, r.kind, sizeof(s.name) - 1);
      stats.push_back(s);
      k = &stats.back();
    }
    k->launches += 1;
    k->total_ms += ms;
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_prof.clear();
  const int32_t n = static_cast<int32_t>(stats.size());
  if (n_kinds_out) *n_kinds_out = n;
  if (out)
    for (int32_t i = 0; i < n && i < max_kinds; ++i) out[i] = stats[i];
  return status;
}

}  // extern "C"
