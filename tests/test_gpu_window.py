"""GPU: the step of a holder of one flat parameter partition (muon_step_window).

DeepSpeed-Muon article, ZeRO stage support section, on partition boundaries:
every rank that holds part of a Muon matrix straddling a ZeRO partition boundary
receives the whole reduced gradient before the nonlinear update. Each holder
here keeps the whole momentum of the matrix, runs the whole step and writes its
own window of the parameters.

Gates:
  the holders' partitions, put together       == muon_step's params, bit for bit
  each holder's momentum and update_out       == muon_step's, bit for bit
  the holders' bf16 shadows, put together     == muon_step's shadow, bit for bit
  partition elements outside every window      unchanged (canary values)
  weight change per window vs the oracle's window_step: the parity gates
  (fp32 iteration 1e-4 vs exact; bf16 / fp16 3e-2 vs the storage-faithful oracle)
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import rel, run_step, to_device

pytestmark = pytest.mark.gpu

CANARY = 7.0


@pytest.fixture
def nss(lib):
    return lib


def _inputs(wl, seed):
    params, grads, _ = W.host_inputs(wl)
    tab = wl.table()
    inside = np.zeros(wl.numel, bool)
    for off, r, c, *_ in tab:
        inside[off:off + r * c] = True
    params[~inside] = CANARY
    # a momentum carried over from an earlier step
    rng = np.random.default_rng(seed)
    mom = np.where(inside, 0.5 * W.grad_as_f64(wl, grads) *
                   (1.0 + 0.1 * rng.standard_normal(wl.numel)), 0.0).astype(np.float32)
    return params, grads, mom, tab, inside


def _hyper(nss, wl, method, ns_dtype):
    return nss.hyper(ns_method=method, ns_dtype=ns_dtype, grad_dtype=wl.grad_dtype, lr=wl.lr,
                     momentum=wl.momentum, weight_decay=wl.weight_decay)


def _holders(n, cuts):
    edges = [0] + list(cuts) + [n]
    return list(zip(edges[:-1], edges[1:]))


def _run_holders(nss, wl, params, grads, mom, tab, cuts, h, subset_tables=False):
    """Each holder's step on its own device buffers; host results per holder."""
    import torch
    dev = "cuda:0"
    g = to_device(grads, dev, torch)
    out = []
    for a, b in _holders(wl.numel, cuts):
        wins = oracle.partition_windows(tab, a, b)
        t, w = tab, wins
        if subset_tables:
            keep = [i for i, (lo, hi, _po) in enumerate(wins) if hi > lo]
            t, w = [tab[i] for i in keep], [wins[i] for i in keep]
        print(f"[holder] [{a}, {b}) entries={len(t)} windows={w}", flush=True)
        part = to_device(params[a:b].copy(), dev, torch)
        m = to_device(mom, dev, torch)
        upd = torch.zeros(wl.numel, dtype=torch.float32, device=dev)
        sh = torch.zeros(b - a, dtype=torch.int16, device=dev)
        nss.step_window(part, g, m, t, w, h, update_out=upd, bf16_shadow=sh)
        torch.cuda.synchronize()
        out.append({"range": (a, b), "table": t, "windows": w, "partition": part.cpu().numpy(),
                    "momentum": m.cpu().numpy(), "update": upd.cpu().numpy(),
                    "shadow": sh.cpu().numpy().view(np.uint16)})
    return out


def _check_union(wl, params, mom, tab, inside, whole, holders):
    got = np.empty_like(params)
    shadow = np.empty(wl.numel, np.uint16)
    for hd in holders:
        a, b = hd["range"]
        got[a:b] = hd["partition"]
        shadow[a:b] = hd["shadow"]
        listed = np.zeros(wl.numel, bool)
        for off, r, c, *_ in hd["table"]:
            listed[off:off + r * c] = True
        assert np.array_equal(hd["momentum"][listed], whole["momentum"][listed])
        assert np.array_equal(hd["momentum"][~listed], mom[~listed])
        assert np.array_equal(hd["update"][listed], whole["update"][listed])
        assert np.all(hd["update"][~listed] == 0.0)
    assert np.array_equal(got, whole["params"])
    assert np.all(got[~inside] == CANARY)
    assert np.array_equal(shadow, whole["shadow"])


def _check_oracle(wl, params, grads, mom, holders, method, store_fmt, gate):
    g64 = W.grad_as_f64(wl, grads)
    for hd in holders:
        a, b = hd["range"]
        ref = oracle.window_step(params[a:b], g64, mom, hd["table"], hd["windows"], lr=wl.lr,
                                 weight_decay=wl.weight_decay, mu=wl.momentum, method=method,
                                 store_fmt=store_fmt)
        sel = np.zeros(b - a, bool)
        for lo, hi, po in hd["windows"]:
            sel[po:po + max(hi - lo, 0)] = True
        if not sel.any():
            continue
        d_gpu = hd["partition"][sel] - params[a:b][sel]
        d_ref = ref["partition"][sel] - params[a:b][sel]
        err = rel(d_gpu, d_ref)
        print(f"  holder [{a}, {b}): {int(sel.sum())} window elements, dp {err:.2e}")
        assert err <= gate, (a, b, err)


SHAPES = [(200, 328, 0), (300, 96, 0), (256, 64, 64), (130, 130, 0), (1, 1, 0), (40, 24, 0)]


def _cuts(wl):
    offs = wl.offsets
    return sorted([
        offs[0] + 7 * 328 + 16,        # inside a wide matrix, 8-aligned
        offs[1] + 1000 + 3,            # inside a tall (transposed) matrix, unaligned
        offs[2] + 64 * 64 + 101,       # inside the second split block, unaligned
        offs[3] - 20,                  # in the alignment gap before a matrix
        offs[3] + 5,                   # five elements into a matrix
        offs[5] + 24 * 17,             # a row boundary of the last matrix
    ])


@pytest.mark.parametrize("method,ns_dtype,grad_dtype", [
    ("standard", "bf16", "bf16"), ("standard", "f32", "f32"), ("gram", "f16", "bf16")])
def test_window_union_is_the_whole_step(nss, method, ns_dtype, grad_dtype):
    # Gaussian gradients for fp16 Gram, whose storage-faithful gate holds on
    # well-conditioned inputs only (test_gpu_parity's Gram gates)
    wl = W.custom_workload(SHAPES, grad_dtype=grad_dtype, ns_dtype=ns_dtype, wid=170,
                           grad_kind="gaussian" if method == "gram" else "")
    params, grads, mom, tab, inside = _inputs(wl, 1)
    h = _hyper(nss, wl, method, ns_dtype)
    print(f"[case] window union {method} {ns_dtype} shapes={SHAPES}", flush=True)
    whole = run_step(nss, params, grads, mom, tab, h, shadow=True)
    holders = _run_holders(nss, wl, params, grads, mom, tab, _cuts(wl), h)
    _check_union(wl, params, mom, tab, inside, whole, holders)
    faithful = ns_dtype != "f32"
    _check_oracle(wl, params, grads, mom, holders, method, ns_dtype if faithful else None,
                  3e-2 if faithful else 1e-4)


def test_window_subset_tables(nss):
    # each holder lists only the matrices it holds part of (smaller groups, other
    # tile choices): the union is still the whole step, bit for bit
    wl = W.custom_workload(SHAPES, grad_dtype="bf16", ns_dtype="bf16", wid=171)
    params, grads, mom, tab, inside = _inputs(wl, 2)
    h = _hyper(nss, wl, "standard", "bf16")
    print("[case] window subset tables", flush=True)
    whole = run_step(nss, params, grads, mom, tab, h, shadow=True)
    holders = _run_holders(nss, wl, params, grads, mom, tab, _cuts(wl), h, subset_tables=True)
    _check_union(wl, params, mom, tab, inside, whole, holders)


def test_window_single_holder_and_empty_windows(nss):
    import torch
    wl = W.custom_workload(SHAPES[:3], grad_dtype="bf16", ns_dtype="bf16", wid=172)
    params, grads, mom, tab, inside = _inputs(wl, 3)
    h = _hyper(nss, wl, "standard", "bf16")
    print("[case] window single holder / empty windows", flush=True)
    whole = run_step(nss, params, grads, mom, tab, h, shadow=True)
    # one holder of everything is muon_step
    holders = _run_holders(nss, wl, params, grads, mom, tab, [], h)
    _check_union(wl, params, mom, tab, inside, whole, holders)
    # all windows empty: the partition stays as it was, the momentum still moves
    dev = "cuda:0"
    part = torch.full((37,), 3.0, dtype=torch.float32, device=dev)
    m = to_device(mom, dev, torch)
    nss.step_window(part, to_device(grads, dev, torch), m, tab, [(0, 0, 0)] * len(tab), h)
    torch.cuda.synchronize()
    assert torch.all(part == 3.0).item()
    assert np.array_equal(m.cpu().numpy()[inside], whole["momentum"][inside])


def test_window_full_size_straddle(nss):
    # a 2048 x 5632 and a 5632 x 2048 matrix (the 1B-class MLP shapes) cut by two
    # partition boundaries, one inside each: bit-exact union at full size
    wl = W.custom_workload([(2048, 5632, 0), (5632, 2048, 0)], grad_dtype="bf16",
                           ns_dtype="bf16", wid=173)
    params, grads, mom, tab, inside = _inputs(wl, 4)
    h = _hyper(nss, wl, "standard", "bf16")
    print("[case] window full-size straddle", flush=True)
    whole = run_step(nss, params, grads, mom, tab, h, shadow=True)
    cuts = [wl.offsets[0] + 2048 * 5632 // 3 + 8, wl.offsets[1] + 777 * 2048 + 1]
    holders = _run_holders(nss, wl, params, grads, mom, tab, cuts, h)
    _check_union(wl, params, mom, tab, inside, whole, holders)


COL_SHAPES = [(256, 384, 0, 128), (300, 72, 0, 24), (512, 768, 256, 384), (60, 100, 0, 20)]


@pytest.mark.parametrize("method,ns_dtype", [("standard", "bf16"), ("gram", "f16")])
def test_window_union_with_column_splits(nss, method, ns_dtype):
    # partition boundaries inside column and grid blocks: a window covers part
    # of some rows of a block, whose rows are ld elements apart in the matrix
    wl = W.custom_workload(COL_SHAPES, grad_dtype="bf16", ns_dtype=ns_dtype, wid=174,
                           grad_kind="gaussian" if method == "gram" else "")
    params, grads, mom, tab, inside = _inputs(wl, 5)
    h = _hyper(nss, wl, method, ns_dtype)
    print(f"[case] window union with column splits {method} {ns_dtype}", flush=True)
    offs = wl.offsets
    cuts = sorted([
        offs[0] + 100 * 384 + 200 + 3,    # mid-row, inside column block 1
        offs[1] + 77 * 72 + 30,           # inside column block 1 of a 24-wide split
        offs[2] + 300 * 768 + 500,        # inside grid block (1, 1)
        offs[3] + 7 * 100 + 45,           # inside a 20-wide block, unaligned
    ])
    whole = run_step(nss, params, grads, mom, tab, h, shadow=True)
    holders = _run_holders(nss, wl, params, grads, mom, tab, cuts, h)
    _check_union(wl, params, mom, tab, inside, whole, holders)
    _check_oracle(wl, params, grads, mom, holders, method, ns_dtype, 3e-2)
