// Owner planning (host only): the FLOP model, the LPT owner assignment with
// per-owner packed layout, and the per-step communication volume.
#pragma once

#include <cstdint>
#include <string>

#include "muon_step.h"

namespace muon {

// Nominal Newton-Schulz FLOPs of one m x n problem (m <= n); -1 on bad input
// or int64 overflow.
int64_t ns_flops(int64_t m, int64_t n, int method, int steps);

// Fills assign[n_params] and owners[n_owners]; returns a MUON_* status (and
// writes nothing but `err` when it is not MUON_OK).
int plan_owners(const muon_param_t* params, int32_t n_params, int32_t n_owners, int32_t method, int32_t steps,
                int64_t align, muon_assign_t* assign, muon_owner_t* owners, std::string& err);

// Elements sent per step on the shard group; negative on bad input.
double comm_elements(int64_t p_m, int32_t n_ranks, int32_t zero_stage, int32_t dedicated);

}  // namespace muon
