// Host-side planning of a Muon step: table validation, problem expansion
// (split blocks), canonical shapes, shape groups, momentum chunks and the
// workspace layout. Pure host code, no HIP calls.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "muon_step.h"

namespace muon {

// A problem is a block of a matrix: block element (r, c) is stored at src_off +
// r * ld + c (ld = the matrix's cols), and its local index is r * ld + c.
struct HostProblem {
  int64_t src_off;
  int64_t p_base;      // params index of local index 0
  int64_t lo, hi;      // local indices whose update is applied
  int32_t ld;
  int32_t transposed;
  int32_t entry;
};

// All problems of one canonical shape (m <= n). Buffers are tile-padded
// (mp x np), one slice per problem, consecutive.
struct Group {
  int64_t m = 0, n = 0, mp = 0, np = 0;
  int tile = 0;
  int sym_tile = 0;                  // tile edge of the symmetric (m x m) launches
  int first = 0, count = 0;          // problems [first, first + count) of the plan
  int64_t chunks = 0;                // momentum blocks per problem (ceil(m n / kMomChunk))
  size_t partial_first = 0;          // index of the group's first per-block partial sum
  // workspace byte offsets
  size_t x[2] = {0, 0};                  // X, ping-pong (standard); X0 in [0] (gram)
  size_t a = 0, b = 0;                   // standard: A, B; gram: R, Q
  size_t r2 = 0, p[2] = {0, 0}, t = 0;   // gram: next R, P (ping-pong), R Q
};

// What the descriptor kernel needs to write the problems of one table entry.
// Problem b (b < nblk) of the entry is problem first + b of the layout: block
// (b / ncb, b % ncb) of the matrix, whose element 0 is flat element
// f = (b / ncb) * rstep + (b % ncb) * cstep of the matrix; src_off = offset + f,
// p_base = p0 + f, and [lo, hi) (flat in the matrix) shifted by f and clamped to
// [0, span], span = the block's last local index + 1.
struct EntryRec {
  int64_t offset;   // element offset of the matrix in grads / momentum
  int64_t rstep;    // flat elements between vertically adjacent blocks (block rows x cols)
  int64_t span;     // (block rows - 1) x cols + block cols
  int64_t lo, hi;   // elements of the flattened matrix whose update is applied
  int64_t p0;       // params index of flat element 0 of the matrix
  int32_t cstep;    // block cols
  int32_t ncb;      // blocks per row of blocks
  int32_t ld;       // the matrix's cols
  int32_t w;        // stored block width (block cols)
  int32_t first;    // layout index of the entry's first problem
  int32_t nblk_t;   // problems of the entry << 1 | transposed
};

struct Layout {
  std::vector<HostProblem> problems;   // ordered by group
  std::vector<Group> groups;
  std::vector<EntryRec> entries;       // one per table entry, for the descriptor kernel
  size_t n_partials = 0;               // per-block partial sums of squares, all groups
  size_t off_desc = 0;                 // per-problem descriptors (ProblemDesc, 48 bytes each)
  size_t off_partials = 0, off_invnorm = 0;
  size_t ws_bytes = 0;
};

constexpr size_t kProblemDescBytes = 48;

int element_size(int dtype);

// Checks the hyperparameters and the table (shapes, splits, offsets, alignment,
// overlap). Returns a MUON_* status and fills `err`.
int validate(const muon_matrix_t* table, int32_t n_entries, const muon_hyper_t* h, std::string& err);

// Checks the windows of a windowed step against the table and a partition of
// `partition_numel` elements (bounds, lo <= hi, no two windows sharing a
// partition element).
int validate_windows(const muon_matrix_t* table, const muon_window_t* windows, int32_t n_entries,
                     int64_t partition_numel, std::string& err);

// Builds the layout of a validated table; `windows` may be NULL (every element
// applied in place at its own offset).
Layout build_layout(const muon_matrix_t* table, int32_t n_entries, const muon_hyper_t* h,
                    const muon_window_t* windows = nullptr);

// Tile edge used for a group of `count` problems whose short side is m.
int tile_for(int64_t m, int64_t count);
// Tile edge of the group's symmetric launches: 128 where the last row of
// 256-tiles would be at most half used (the full launches keep 256-tiles).
int sym_tile_for(int64_t m, int tile);

}  // namespace muon
