"""Owner planner (host code, no GPU): the library's muon_plan_owners,
muon_ns_flops and muon_comm_elements against the plain-Python reference in
oracle/planner.py, and both against what the pages and textbook scheduling fix.

Pins of the reference:
  * the FLOP model equals the products the oracle's Newton-Schulz performs,
    counted while it runs (standard and gram), and the closed forms
    20 m^2 n + 10 m^3 and 4 m^2 n + 34 m^3 at five steps;
  * largest-first greedy on the textbook instance {3, 3, 2, 2, 2} on two
    machines gives 7 where the optimum is 6, and never exceeds Graham's bound
    (4/3 - 1/(3N)) x optimum (optimum by brute force on tiny instances);
  * the communication factors and the 7B memory example printed by the DMuon
    docs (tests/golden/dmuon_planning.json), and the consistency of its two
    tables (Z3 - Z2 = one more shard broadcast per step).
Library vs reference: identical owners, offsets and per-owner totals (integer
work, bit-exact).
"""
import ctypes
import itertools
import json
import os

import numpy as np
import pytest

import newton_schulz_step_amd as nss
import oracle
from oracle import planner as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "dmuon_planning.json")


# --------------------------------------------------------------------------- FLOP model

class _Counting(np.ndarray):
    """An ndarray that adds 2 m k n to a counter for every matmul it takes part in."""
    count = [0]

    def __array_ufunc__(self, ufunc, method, *inputs, **kw):
        plain = [np.asarray(x) if isinstance(x, _Counting) else x for x in inputs]
        if ufunc is np.matmul:
            a, b = plain
            _Counting.count[0] += 2 * a.shape[0] * a.shape[1] * b.shape[1]
        out = getattr(ufunc, method)(*plain, **kw)
        return out.view(_Counting) if isinstance(out, np.ndarray) else out


def _counted(fn, X0, steps):
    _Counting.count[0] = 0
    fn(X0.view(_Counting), steps)
    return _Counting.count[0]


@pytest.mark.parametrize("m,n", [(1, 1), (3, 7), (8, 8), (5, 40)])
@pytest.mark.parametrize("steps", [1, 2, 5])
def test_flop_model_counts_the_oracle_products(m, n, steps):
    X0 = np.random.default_rng(m * 100 + n).standard_normal((m, n))
    X0 /= np.linalg.norm(X0)
    std = _counted(oracle.newton_schulz_standard, X0, steps)
    gram = _counted(oracle.newton_schulz_gram, X0, steps)
    assert std == ref.ns_flops(m, n, "standard", steps)
    assert gram == ref.ns_flops(m, n, "gram", steps)


def test_flop_model_closed_forms():
    for m, n in [(1, 1), (128, 1024), (4096, 11008), (16384, 1 << 24)]:
        assert ref.ns_flops(m, n, "standard") == 20 * m * m * n + 10 * m ** 3
        assert ref.ns_flops(m, n, "gram") == 4 * m * m * n + 34 * m ** 3


def test_library_flop_model():
    for m, n in [(1, 1), (3, 7), (128, 1024), (4096, 11008), (16384, 1 << 24)]:
        for method in ("standard", "gram"):
            for steps in (1, 5, 64):
                assert nss.ns_flops(m, n, method, steps) == ref.ns_flops(m, n, method, steps)
    lib = nss.load()
    assert lib.muon_ns_flops(0, 5, 0, 5) == -1
    assert lib.muon_ns_flops(5, 5, 2, 5) == -1
    assert lib.muon_ns_flops(5, 5, 0, 0) == -1
    assert lib.muon_ns_flops(1 << 40, 1 << 40, 0, 5) == -1   # int64 overflow


# --------------------------------------------------------------------------- assignment

def _makespan(costs, owner, n):
    load = [0] * n
    for c, o in zip(costs, owner):
        load[o] += c
    return max(load)


def _optimum(costs, n):
    return min(_makespan(costs, a, n) for a in itertools.product(range(n), repeat=len(costs)))


def test_lpt_textbook_instance():
    costs = [3, 3, 2, 2, 2]
    owner = ref.lpt(costs, [1] * 5, 2)
    assert _makespan(costs, owner, 2) == 7 and _optimum(costs, 2) == 6
    assert owner == [0, 1, 0, 1, 0]


def test_lpt_within_graham_bound():
    rng = np.random.default_rng(5)
    for _ in range(60):
        n = int(rng.integers(2, 4))
        costs = [int(c) for c in rng.integers(1, 30, size=int(rng.integers(n + 1, 8)))]
        got = _makespan(costs, ref.lpt(costs, [1] * len(costs), n), n)
        assert got * 3 * n <= (4 * n - 1) * _optimum(costs, n)


# (rows, cols, split_rows, split_cols)
POOL = [(2048, 2048, 0, 0), (5632, 2048, 0, 0), (2048, 5632, 0, 0), (4096, 4096, 0, 0),
        (11008, 4096, 0, 0), (4096, 11008, 0, 0), (1024, 128, 128, 0), (384, 200, 0, 0),
        (8, 8, 0, 0), (1, 1, 0, 0), (257, 33, 0, 0), (512, 64, 64, 0), (64, 4096, 0, 0),
        (4096, 4096, 0, 128), (2048, 640, 0, 64), (512, 768, 256, 384)]


def _random_model(rng, n):
    """(rows, cols, split_rows, layer, split_cols) per matrix."""
    out = []
    for _ in range(n):
        r, c, s, sc = POOL[int(rng.integers(len(POOL)))]
        out.append((r, c, s, int(rng.integers(0, 4)), sc))
    return out


@pytest.mark.parametrize("seed", range(6))
def test_library_plan_matches_reference(seed):
    rng = np.random.default_rng(100 + seed)
    model = _random_model(rng, int(rng.integers(1, 40)))
    for n_owners in (1, 2, 3, 8, 13):
        for method in ("standard", "gram"):
            for align in (8, 64):
                want = ref.plan_owners(model, n_owners, method, 5, align)
                assign, owners = nss.plan_owners(model, n_owners, method, 5, align)
                assert assign == want["assign"]
                for o, w in zip(owners, want["owners"]):
                    assert {k: o[k] for k in w} == w


def test_plan_layout_invariants():
    rng = np.random.default_rng(7)
    model = _random_model(rng, 60)
    assign, owners = nss.plan_owners(model, 5, "standard", 5, 64)
    seen = set()
    for o, info in enumerate(owners):
        spans = sorted((assign[i][1], assign[i][1] + model[i][0] * model[i][1], model[i][3], i)
                       for i in range(len(model)) if assign[i][0] == o)
        assert info["n_matrices"] == len(spans)
        assert [s[3] for s in spans] == info["index"]
        assert info["table"] == [(s[0], model[s[3]][0], model[s[3]][1], model[s[3]][2], model[s[3]][4])
                                 for s in spans]
        for (a0, a1, la, _), (b0, b1, lb, _) in zip(spans, spans[1:]):
            assert a1 <= b0 and la <= lb           # no overlap; layers in order
        assert all(s[0] % 64 == 0 for s in spans)
        assert info["numel"] == (spans[-1][1] if spans else 0)
        per_layer = {}
        for a, b, layer, _ in spans:
            lo, hi = per_layer.get(layer, (a, b))
            per_layer[layer] = (min(lo, a), max(hi, b))
        assert info["max_layer_numel"] == max((b - a for a, b in per_layer.values()), default=0)
        flops = sum(ref.matrix_flops(*model[s[3]][:3], split_cols=model[s[3]][4]) for s in spans)
        assert info["ns_flops"] == flops
        seen.update(s[3] for s in spans)
    assert seen == set(range(len(model)))


def test_more_owners_than_matrices():
    assign, owners = nss.plan_owners([(64, 64, 0, 0), (32, 64, 0, 0)], 4)
    assert assign == [(0, 0), (1, 0)]
    for info in owners[2:]:
        assert (info["numel"], info["max_layer_numel"], info["ns_flops"], info["n_matrices"]) == (0, 0, 0, 0)


def test_plan_rejects_and_writes_nothing():
    lib = nss.load()

    def call(model, n_owners=2, method=0, steps=5, align=64, null_out=False):
        arr = (nss.MuonParam * max(len(model), 1))(*[nss.MuonParam(r, c, s, l, 0) for r, c, s, l in model])
        a = (nss.MuonAssign * max(len(model), 1))()
        o = (nss.MuonOwner * max(n_owners, 1))()
        for x in a:
            x.owner, x.offset = -7, -7
        st = lib.muon_plan_owners(arr, len(model), n_owners, method, steps, align, a,
                                  None if null_out else o)
        if st != nss.OK:
            assert all(x.owner == -7 and x.offset == -7 for x in a)
        return st

    good = [(64, 64, 0, 0)]
    assert call(good) == nss.OK
    assert call(good, n_owners=0) == nss.ERR_BAD_SHAPE
    assert call([(0, 64, 0, 0)]) == nss.ERR_BAD_SHAPE
    assert call([(64, 64, 5, 0)]) == nss.ERR_BAD_SHAPE
    assert call([(64, 64, 0, -1)]) == nss.ERR_BAD_SHAPE
    assert call([(20000, 20000, 0, 0)]) == nss.ERR_BAD_SHAPE
    assert call(good, method=5) == nss.ERR_BAD_METHOD
    assert call(good, steps=0) == nss.ERR_BAD_HYPER
    assert call(good, align=12) == nss.ERR_ALIGN
    assert call(good, align=0) == nss.ERR_ALIGN
    assert call(good, null_out=True) == nss.ERR_NULL
    with pytest.raises(nss.MuonError):
        nss.plan_owners(good, 0)


# --------------------------------------------------------------------------- pages' figures

def test_comm_factors_match_the_pages():
    g = json.load(open(GOLDEN))
    c = g["comm_per_step"]
    cases = {("naive", 2): c["naive_fsdp2_z2"], ("dmuon", 2): c["dmuon_z2"],
             ("naive", 3): c["naive_fsdp2_z3"], ("dmuon", 3): c["dmuon_z3"]}
    for (kind, stage), k in cases.items():
        for n in (1, 2, 8, 64):
            for p_m in (0, 1000, 3_500_000_000):
                want = k * (n - 1) / n * p_m
                assert ref.comm_elements(p_m, n, stage, kind == "dmuon") == want
                assert nss.comm_elements(p_m, n, stage, kind == "dmuon") == pytest.approx(want, rel=1e-15)
    # DMuon saves one gradient all-gather in both modes; Z3 pays one more shard
    # broadcast per step than Z2 (the lifecycle table)
    b = g["shard_broadcasts_per_step"]
    assert c["naive_fsdp2_z2"] - c["dmuon_z2"] == 1 and c["naive_fsdp2_z3"] - c["dmuon_z3"] == 1
    assert c["dmuon_z3"] - c["dmuon_z2"] == b["dmuon_z3"] - b["dmuon_z2"]
    lib = nss.load()
    assert lib.muon_comm_elements(10, 0, 2, 1) < 0 and lib.muon_comm_elements(10, 2, 4, 1) < 0


def test_memory_example_of_the_pages():
    # 3.5B Muon-target elements in identical matrices over 8 owners: each owner
    # keeps P_M / 8 elements resident under DMuon-Z2, 875 MB in bf16
    g = json.load(open(GOLDEN))["memory_example"]
    model = [(1750, 2000, 0, layer) for layer in range(1000)]
    assert sum(r * c for r, c, _s, _l in model) == g["p_m"]
    assert g["p_m"] * 2 == g["bf16_total_bytes"]
    _, owners = nss.plan_owners(model, g["shard_ways"], "standard", 5, 8)
    for info in owners:
        assert info["numel"] * 2 == g["dmuon_z2_extra_bytes_per_rank"]
        assert info["max_layer_numel"] == 1750 * 2000   # DMuon-Z3: one layer at a time
    want = ref.plan_owners(model, g["shard_ways"], "standard", 5, 8)
    assert [o["numel"] for o in want["owners"]] == [o["numel"] for o in owners]
