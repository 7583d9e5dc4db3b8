"""GPU: seeded random shape tables against the oracle.

Each case draws a table of 3-6 entries: random rows and cols (1 to ~900),
some split into row blocks (split_rows a divisor of rows), stored at offsets
with random gaps (multiples of 8 elements). Gradients are Gaussian (the
iteration is well conditioned on them, so the faithful gate measures the
kernels), momentum non-zero. fp32 iterations are gated against the exact
oracle, bf16 / fp16 ones against the storage-faithful oracle; momentum and
the untouched bytes outside the table as in the other parity tests.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import entry_slices, outside_mask, rel, run_step

pytestmark = pytest.mark.gpu

SEEDS = range(8)
CONFIGS = [("standard", "f32", "f32"), ("standard", "bf16", "bf16"), ("gram", "f16", "bf16")]


def _random_table(seed):
    rng = np.random.default_rng(7000 + seed)
    shapes = []
    for _ in range(int(rng.integers(3, 7))):
        kind = rng.integers(4)
        if kind == 0:     # small and ragged
            r, c = int(rng.integers(1, 40)), int(rng.integers(1, 60))
        elif kind == 1:   # around the 128 edge
            r, c = int(rng.integers(100, 160)), int(rng.integers(100, 700))
        else:             # larger, either orientation
            r, c = int(rng.integers(60, 700)), int(rng.integers(60, 900))
        if rng.random() < 0.5:
            r, c = c, r
        split = 0
        if rng.random() < 0.3:
            divs = [d for d in range(1, r) if r % d == 0 and d * c >= 1]
            if divs:
                split = int(rng.choice(divs))
        shapes.append((r, c, split))
    offs, cur = [], 0
    for r, c, _ in shapes:
        cur += 8 * int(rng.integers(0, 3))
        offs.append(cur)
        cur = (cur + r * c + 7) // 8 * 8
    return shapes, offs, cur + 8 * int(rng.integers(0, 3))


@pytest.mark.parametrize("seed", SEEDS)
@pytest.mark.parametrize("method,ns_dtype,grad_dtype", CONFIGS)
def test_random_table(lib, seed, method, ns_dtype, grad_dtype):
    shapes, offs, n = _random_table(seed)
    tab = [(o, r, c, s) for o, (r, c, s) in zip(offs, shapes)]
    print(f"[case] seed {seed} {method} {ns_dtype}: {tab}", flush=True)
    rng = np.random.default_rng(9000 + seed)
    params = rng.standard_normal(n).astype(np.float32)
    g = rng.standard_normal(n).astype(np.float32)
    grads = g if grad_dtype == "f32" else W.f32_to_bf16_bits(g)
    g64 = g.astype(np.float64) if grad_dtype == "f32" else W.bf16_bits_to_f32(grads).astype(np.float64)
    mom = (0.3 * rng.standard_normal(n)).astype(np.float32)
    h = lib.hyper(ns_method=method, ns_dtype=ns_dtype, grad_dtype=grad_dtype, lr=0.02, momentum=0.95,
                  weight_decay=0.1)
    gpu = run_step(lib, params, grads, mom, tab, h)
    kw = dict(lr=0.02, mu=0.95, weight_decay=0.1, method=method)
    exact = oracle.muon_step(params, g64, mom, tab, **kw)
    ref = exact if ns_dtype == "f32" else oracle.muon_step(params, g64, mom, tab, store_fmt=ns_dtype, **kw)
    gate = 1e-4 if ns_dtype == "f32" else 3e-2
    for i, sl in enumerate(entry_slices(tab)):
        eo = rel(gpu["update"][sl], ref["update"][sl])
        dp = rel(gpu["params"][sl] - params[sl], ref["params"][sl] - params[sl])
        em = rel(gpu["momentum"][sl], exact["momentum"][sl])
        assert eo <= gate and dp <= gate and em <= 1e-6, (i, tab[i], eo, dp, em)
    mask = outside_mask(tab, n)
    assert np.array_equal(gpu["params"][mask], params[mask])
    assert np.array_equal(gpu["momentum"][mask], mom[mask])
    assert not np.any(gpu["update"][mask])
