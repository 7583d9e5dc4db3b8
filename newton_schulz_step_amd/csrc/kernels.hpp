// Launch interfaces of the HIP kernels (internal to libmuonstep).
#pragma once

#include "common.hpp"
#include "plan.hpp"

namespace muon {

// Per-problem descriptors of a step, written into the caller's workspace on the
// stream from the table's entry records, passed by value kDescChunk at a time.
constexpr int kDescChunk = 32;
hipError_t launch_expand_desc(const EntryRec* entries, int n, ProblemDesc* out, hipStream_t s);

// EPI_APPLY: fp32 params; EPI_APPLY_BF16: bf16 params (raw 16-bit words), the
// new value rounded to nearest even
enum { EPI_STORE = 0, EPI_APPLY = 1, EPI_APPLY_BF16 = 2 };

// One batched GEMM launch: for every problem p of a shape group,
//   C_p = epilogue(alpha * P_p op(Q_p) + beta * D_p + gamma * I),
// where P_p is rows x K, K contiguous. Symmetric launches take Q_p as N x K, K
// contiguous (op = transpose, "NT"); full launches take it as K x N, N
// contiguous (op = identity, "NN"). Strides (_ps) are elements between
// consecutive problems; ld* are row pitches in elements. K, and the
// tile-padded extents, are multiples of the tile sizes, so the main loop needs
// no bounds checks (padding holds zeros).
struct GemmArgs {
  const void* P; int64_t p_ps; int32_t ldp;
  const void* Q; int64_t q_ps; int32_t ldq;
  int32_t K;
  int32_t tiles_m, tiles_n, tiles_per_problem, total_tiles;
  float alpha, beta, gamma;                      // gamma: symmetric launches only
  const void* D; int64_t d_ps; int32_t ldd;      // optional beta term: symmetric launches only,
                                                 // and then in every group of the launch
  void* C; int64_t c_ps; int32_t ldc;            // optional row-major store
  void* Ct; int64_t ct_ps; int32_t ldct;         // optional transposed store (SYM: mirror, = C)
  // EPI_APPLY(_BF16): p <- p * decay - lr * v at the problem's stored position
  void* params; const ProblemDesc* probs; int32_t m_valid, n_valid;
  float decay, lr;
  float* update_out; unsigned short* shadow;
};

// Several shape groups in one launch (same element type, tile and kind):
// group g owns blocks [start[g], start[g + 1]); start[0] = 0 and
// start[g + 1] - start[g] = g[g].total_tiles.
constexpr int kBatchGroups = 4;
struct GemmBatch {
  GemmArgs g[kBatchGroups];
  int32_t start[kBatchGroups + 1];
  int32_t n;
};

hipError_t launch_ns_gemm(int dtype, int tile, bool sym, int epi, const GemmBatch& b, hipStream_t s);

// Single-tile-row groups (mp = 128, bf16/fp16): X' = alpha B X and A' = X' X'^T
// (stored symmetric) in one pass, one block per problem. Per group: P = B,
// Q = X, C = X', Ct = A', K = 128, tiles_n = np / 128, total_tiles = number of
// problems; D must be null and beta 0.
hipError_t launch_update_gram(int dtype, const GemmBatch& b, hipStream_t s);

// Single-tile-row groups (mp = 128, fp16), Gram method: the whole chain
//   Q = qa I + qb R + qc R R;  P <- Q P (P = Q first);  T = R Q, R <- Q T
// (stored symmetric, as the symmetric launches store them) for `steps` steps,
// one workgroup per problem with R, Q, T and P held in LDS; the final P is
// written row-major (pitch 128, p_ps elements apart) for the apply launch.
// R0 (r_ps apart, pitch 128) is as the prep pass wrote it. Every product and
// rounding matches the separate launches, so P is bit-identical to theirs.
struct GramChainArgs {
  const void* R0; int64_t r_ps;
  void* P; int64_t p_ps;
  float qa, qb, qc;
  int32_t steps;
  int32_t count;
};
struct GramChainBatch {
  GramChainArgs g[kBatchGroups];
  int32_t start[kBatchGroups + 1];
  int32_t n;
};
hipError_t launch_gram_chain(int dtype, const GramChainBatch& b, hipStream_t s);

// Single-tile-row groups (mp = 128, bf16/fp16): X0 = round(M * inv_norm) as the
// X0 kernel writes it, and R = alpha X0 X0^T (stored symmetric) as the symmetric
// launch computes it, in one pass; one block per problem.
struct PrepGramArgs {
  const float* M; const ProblemDesc* probs; const float* inv_norm;
  void* X;        // n_problems x mp x np
  void* R;        // n_problems x mp x mp
  int32_t m, n, mp, np, n_problems;
  float alpha;
};
hipError_t launch_prep_gram(int dtype, const PrepGramArgs& a, hipStream_t s);

// M <- mu M + G over every problem of a group (each m n contiguous elements at
// its src_off), kMomChunk elements per block; partials[b] = sum of squares of the
// new M in block b (problem b / chunks, block b % chunks of that problem), float64.
hipError_t launch_momentum_sumsq(int grad_dtype, float* M, const void* G, const ProblemDesc* probs, int n_problems,
                                 int64_t per_problem, int64_t chunks, float mu, double* partials, hipStream_t s);

// inv_norm[p] = 1 / (sqrt(sum of the `chunks` partials of p) + eps), summed in a fixed order.
hipError_t launch_finalize_norm(const double* partials, int64_t chunks, int n_problems, float eps, float* inv_norm,
                                hipStream_t s);

// X0 (canonical m x n, padded mp x np, row-major) of every problem of a group,
// X0 = round(M * inv_norm); padding zero.
hipError_t launch_prep_x0(int ns_dtype, const float* M, const ProblemDesc* probs, const float* inv_norm,
                          int n_problems, int m, int n, int mp, int np, void* X, hipStream_t s);

hipError_t launch_adamw(int grad_dtype, float* p, const void* g, float* m, float* v, int64_t n,
                        float beta1, float beta2, float step_size, float inv_bc2, float eps,
                        float decay, hipStream_t s);

// Zeros over `count` regions of `bytes` bytes, `stride` bytes apart (the base,
// stride and bytes multiples of 16).
hipError_t launch_zero_regions(void* base, int64_t stride, int64_t bytes, int64_t count, hipStream_t s);

struct CopyItem { const void* src; void* dst; int64_t bytes; };
constexpr int kCopyBatch = 64;
hipError_t launch_copy_batch(const CopyItem* items, int n, hipStream_t s);

}  // namespace muon
