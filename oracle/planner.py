"""Plain-Python reference of the owner planner.

TEST INFRASTRUCTURE ONLY (see the package docstring). It shares no code with the
library's planner.

Sources:
  [DM] "Z2 与 Z3 模式" (DMuon docs): every Muon-target matrix has a single
       owner that alone runs its Newton-Schulz (section on the relation to
       ZeRO-2 / ZeRO-3); an owner's matrices are packed into one contiguous
       buffer (section on the two packed-buffer lifecycles); DMuon-Z3 holds one
       layer's packed buffer at a time, DMuon-Z2 all of them (memory section);
       per-step communication on the shard group (communication section).
Readings (the pages do not say how owners are chosen):
  * owners are balanced by the nominal Newton-Schulz FLOPs of their problems,
    with the largest-first greedy rule: matrices by decreasing FLOPs (ties:
    more elements, then lower index), each to the owner with the least FLOPs
    so far (ties: lower owner index);
  * an owner's packed buffer holds its matrices ordered by (layer, index),
    each at the next multiple of `align` elements.
"""
from typing import Dict, List, Sequence, Tuple


def ns_products(m: int, n: int, method: str = "standard", steps: int = 5
                ) -> List[Tuple[int, int, int]]:
    """(rows, inner, cols) of every matrix product the iteration on an m x n
    problem (m <= n) performs, in order, as the oracle's Newton-Schulz runs it."""
    out = []
    if method == "standard":
        for _ in range(steps):
            out += [(m, n, m),      # A = X X^T
                    (m, m, m),      # A A
                    (m, m, n)]      # B X
        return out
    out.append((m, n, m))           # R0 = X0 X0^T
    for k in range(steps):
        out.append((m, m, m))       # R R inside Q
        if k > 0:
            out.append((m, m, m))   # P <- Q P
        if k < steps - 1:
            out += [(m, m, m), (m, m, m)]   # R Q, then Q (R Q)
    out.append((m, m, n))           # P X0
    return out


def ns_flops(m: int, n: int, method: str = "standard", steps: int = 5) -> int:
    """2 x rows x inner x cols summed over the products (multiply-add = 2 FLOPs)."""
    return sum(2 * r * k * c for r, k, c in ns_products(m, n, method, steps))


def matrix_flops(rows: int, cols: int, split_rows: int, method: str = "standard",
                 steps: int = 5, split_cols: int = 0) -> int:
    """FLOPs of one matrix: its problems (the whole matrix, or each split block)."""
    pr = split_rows if split_rows > 0 else rows
    pc = split_cols if split_cols > 0 else cols
    return (rows // pr) * (cols // pc) * ns_flops(min(pr, pc), max(pr, pc), method, steps)


def lpt(costs: Sequence[int], sizes: Sequence[int], n_owners: int) -> List[int]:
    """Largest-first greedy assignment; returns the owner of each job."""
    order = sorted(range(len(costs)), key=lambda i: (-costs[i], -sizes[i], i))
    load = [0] * n_owners
    owner = [0] * len(costs)
    for i in order:
        best = 0
        for o in range(1, n_owners):
            if load[o] < load[best]:
                best = o
        owner[i] = best
        load[best] += costs[i]
    return owner


def plan_owners(params: Sequence[Tuple[int, int, int, int]], n_owners: int,
                method: str = "standard", steps: int = 5, align: int = 64) -> Dict:
    """params: (rows, cols, split_rows, layer[, split_cols]) per matrix. Returns
    {"assign": [(owner, offset)], "owners": [dict(numel, max_layer_numel,
    ns_flops, n_matrices)]}."""
    costs = [matrix_flops(q[0], q[1], q[2], method, steps, q[4] if len(q) > 4 else 0)
             for q in params]
    sizes = [q[0] * q[1] for q in params]
    owner = lpt(costs, sizes, n_owners)
    offset = [0] * len(params)
    owners = []
    for o in range(n_owners):
        mine = sorted((i for i in range(len(params)) if owner[i] == o),
                      key=lambda i: (params[i][3], i))
        end = 0
        spans: Dict[int, List[int]] = {}
        for i in mine:
            start = -(-end // align) * align
            offset[i] = start
            end = start + sizes[i]
            layer = params[i][3]
            if layer not in spans:
                spans[layer] = [start, end]
            spans[layer][1] = end
        owners.append({"numel": end,
                       "max_layer_numel": max((b - a for a, b in spans.values()), default=0),
                       "ns_flops": sum(costs[i] for i in mine),
                       "n_matrices": len(mine)})
    return {"assign": [(owner[i], offset[i]) for i in range(len(params))], "owners": owners}


# [DM] communication section: multiples of (N-1)/N * P_M per step on the shard group
COMM_FACTORS = {("dmuon", 2): 2, ("dmuon", 3): 3, ("naive", 2): 3, ("naive", 3): 4}


def comm_elements(p_m: int, n_ranks: int, zero_stage: int, dedicated: bool) -> float:
    k = COMM_FACTORS[("dmuon" if dedicated else "naive", zero_stage)]
    return k * (n_ranks - 1) / n_ranks * p_m
