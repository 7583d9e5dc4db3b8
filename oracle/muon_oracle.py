"""CPU oracle of the Muon optimizer step, float64 (numpy).

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports or calls this
module; only tests/, the smoke check and the benchmark's CPU-baseline leg do.
It shares no code with the GPU library.

Sources (pages, by title and section):
  [DS]  "DeepSpeed 集成 Muon 优化器实战：从正交化原理到 ZeRO 微调配置"
        (DeepSpeed-Muon article): section "什么是 Muon 优化器？" (momentum first,
        then orthogonalise the momentum matrix, then update the weights);
        section "核心算子：牛顿-舒尔茨正交化内核" (quintic Newton-Schulz with
        a=3.4445, b=-4.7750, c=2.0315, five steps, stable in bf16; a Gram variant
        iterating on R = X X^T in fp16; decoupled weight decay p *= 1 - lr*wd then
        p -= lr * update; the Adam fallback); section "如何用 DeepSpeed 配置启用
        Muon" (defaults: Muon lr 0.02, momentum 0.95, ns_method "gram"; Adam lr
        3e-4, betas (0.9, 0.95), eps 1e-10; the example config's values).
  [DM]  "Z2 与 Z3 模式" (DMuon docs): one owner packs all of its Muon-target
        parameters into one contiguous buffer (section on the two packed-buffer
        lifecycles).

Readings where the pages leave a step open (each also listed in the design notes):
  * Newton-Schulz step form: A = X X^T, B = a I + b A + c A A, X <- B X, i.e.
    the odd quintic p(x) = a x + b x^3 + c x^5 applied to every singular value;
    the article's "maximise the slope at zero" matches p'(0) = a. The article
    fixes the polynomial, its coefficients and the bf16 precision, not how the
    a X term is grouped; B carries a I, the grouping its Gram variant uses for
    Q = a I + b R + c R R. In exact arithmetic this is a X + (b A + c A A) X.
  * X0 = Y / (||Y||_F + eps), eps = 1e-7; Y is transposed first when it has more
    rows than columns, and the result is transposed back.
  * Momentum: heavy ball, M <- mu M + G, no Nesterov term, no dampening.
    Parity unpinned: nothing on the pages tells this form from Nesterov. The
    function is pinned to the reading by the constant-gradient closed form, and
    one-step results do not depend on the choice (normalisation cancels M = G's
    scale).
  * Gram recurrence: R0 = X0 X0^T; per step Q = a I + b R + c R R; P <- Q P
    (P = Q on the first step); R <- Q (R Q) except after the last step; the
    result is P X0. In exact arithmetic this equals the standard iteration,
    because every iterate is an odd polynomial in X0 and Q commutes with R.
  * Update scale: none beyond lr (the article adds the orthogonalised matrix with
    alpha = -lr).
  * Per-head split ("Muon Split" in the article's TL;DR): split_rows = k cuts a
    matrix into rows/k blocks of k rows; each block is its own problem, with its
    own norm. split_cols = k cuts it into cols/k blocks of k columns the same way
    (the heads of a projection whose input side holds them); with both, the
    blocks are the split_rows x split_cols tiles.
  * AdamW: bias-corrected moments, eps added outside the square root, decoupled
    weight decay applied before the moment step (the article's AdamW mode).

Storage-faithful mode: the article runs the standard iteration in bf16 and the
Gram iteration in fp16. `store` rounds (once, to nearest even, from float64) at
each point where such an implementation stores a matrix; the arithmetic between
those points stays float64. Standard: X0, A, B (a I included) and X1..X4 are
stored; X5 is not.
Gram: X0, R0, every Q, P and R, and the intermediate T = R Q are stored; P X0 is
not. The Gram state may carry an exact power-of-two scale s (R is kept as
s X X^T, and b, c become b/s, c/s^2); with s = 1 this is the plain recurrence.
A product is stored as a symmetric matrix (its lower triangle, row index >=
column index, rounded and mirrored) only where its stored operands make it
exactly symmetric under any fixed-order evaluation: A = X X^T and R0 = X0 X0^T
(entry (i, j) and (j, i) add the same products in the same order), and B and
the first Q, polynomials in such a matrix. Everything else is stored as
computed: T = R Q and R <- Q T (after rounding, Q no longer commutes with R, so
neither product is symmetric), every later Q (a polynomial in such an R), and P.
The exact mode evaluates the products as they are.
"""
from __future__ import annotations

from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np

from .rounding import storer

# [DS] 核心算子: quintic coefficients and the number of iterations.
NS_A, NS_B, NS_C = 3.4445, -4.7750, 2.0315
NS_STEPS = 5
NS_EPS = 1e-7
# [DS] 核心算子: the two accepted methods; the default is "gram".
NS_METHODS = ("standard", "gram")
DEFAULT_NS_METHOD = "gram"
# [DS] 如何用 DeepSpeed 配置启用 Muon: group defaults.
MUON_DEFAULTS = {"lr": 0.02, "momentum": 0.95, "ns_method": "gram"}
ADAM_DEFAULTS = {"lr": 3e-4, "betas": (0.9, 0.95), "eps": 1e-10}

Store = Callable[[np.ndarray], np.ndarray]


def _ident(z):
    return z


def _symmetric(store: Store) -> Store:
    """Store a product that any fixed-order evaluation leaves exactly symmetric:
    lower triangle, mirrored (storage-faithful mode only; the exact mode keeps
    the product as computed)."""
    if store is _ident:
        return store
    return lambda z: store(np.tril(z) + np.tril(z, -1).T)


def momentum_update(M: np.ndarray, G: np.ndarray, mu: float) -> np.ndarray:
    """[DS] 什么是 Muon 优化器？: momentum is formed from the gradient first.
    Heavy-ball form (a reading; parity unpinned against the pages)."""
    return mu * M + G


def normalise(Y: np.ndarray, eps: float = NS_EPS) -> np.ndarray:
    """Frobenius normalisation before the iteration (reading; the pages are silent)."""
    return Y / (np.sqrt(np.sum(Y * Y)) + eps)


def newton_schulz_standard(X0: np.ndarray, steps: int = NS_STEPS,
                           coeffs: Tuple[float, float, float] = (NS_A, NS_B, NS_C),
                           store: Store = _ident) -> np.ndarray:
    """[DS] 核心算子, zeropower_via_newtonschulz5: `steps` quintic steps on a
    matrix with no more rows than columns."""
    a, b, c = coeffs
    sym = _symmetric(store)
    X = store(X0)
    eye = np.eye(X0.shape[0])
    for k in range(steps):
        A = sym(X @ X.T)
        B = sym(a * eye + b * A + c * (A @ A))
        X_next = B @ X
        X = X_next if k == steps - 1 else store(X_next)
    return X


def newton_schulz_gram(X0: np.ndarray, steps: int = NS_STEPS,
                       coeffs: Tuple[float, float, float] = (NS_A, NS_B, NS_C),
                       store: Store = _ident, scale: float = 1.0) -> np.ndarray:
    """[DS] 核心算子, zeropower_via_gram_newtonschulz: the iteration carried on the
    small square Gram matrix R = X X^T, applied to X0 once at the end."""
    a, b, c = coeffs
    m = X0.shape[0]
    eye = np.eye(m)
    sym = _symmetric(store)
    X = store(X0)
    R = sym(scale * (X @ X.T))
    bs, cs = b / scale, c / (scale * scale)
    P = None
    for k in range(steps):
        # symmetric only while R is: R0, stored symmetric; later R as computed
        Q = (sym if k == 0 else store)(a * eye + bs * R + cs * (R @ R))
        P = Q if k == 0 else store(Q @ P)
        if k < steps - 1:
            T = store(R @ Q)
            R = store(Q @ T)
    return P @ X


def gram_scale(m: int) -> float:
    """Power-of-two scale of the stored Gram state in fp16 (keeps R's entries of
    size ~1/m in fp16's normal range): 2**ceil(log2 m), at most 2**15."""
    e = 0
    while (1 << e) < m and e < 15:
        e += 1
    return float(1 << e)


def orthogonalise(Y: np.ndarray, method: str = "standard", steps: int = NS_STEPS,
                  coeffs: Tuple[float, float, float] = (NS_A, NS_B, NS_C),
                  eps: float = NS_EPS, store_fmt: Optional[str] = None,
                  scale: Optional[float] = None) -> np.ndarray:
    """Orthogonalised update O for one momentum block Y (same orientation as Y).

    store_fmt None evaluates exactly in float64; "bf16"/"f16"/"f32" stores the
    iterates in that format (see the module notes). For "gram" in fp16 the Gram
    state carries gram_scale(m) unless `scale` is given.
    """
    if method not in NS_METHODS:
        raise ValueError(f"ns_method must be one of {NS_METHODS}, got {method!r}")
    transposed = Y.shape[0] > Y.shape[1]
    X0 = normalise(Y.T if transposed else Y, eps)
    st = storer(store_fmt)
    if method == "standard":
        O = newton_schulz_standard(X0, steps, coeffs, st)
    else:
        if scale is None:
            scale = gram_scale(X0.shape[0]) if store_fmt == "f16" else 1.0
        O = newton_schulz_gram(X0, steps, coeffs, st, scale)
    return O.T if transposed else O


def problem_blocks(rows: int, cols: int, split_rows: int, split_cols: int = 0):
    """(first row, row count, first column, column count) of each independent
    problem of one entry, row of blocks by row of blocks."""
    pr = split_rows if split_rows > 0 else rows
    pc = split_cols if split_cols > 0 else cols
    return [(r, pr, c, pc) for r in range(0, rows, pr) for c in range(0, cols, pc)]


def _entry(e):
    """(offset, rows, cols, split_rows, split_cols) of a 4- or 5-field table entry."""
    off, rows, cols, split_rows = e[:4]
    return off, rows, cols, split_rows, (e[4] if len(e) > 4 else 0)


def muon_step(params: np.ndarray, grads: np.ndarray, momentum: np.ndarray,
              table: Sequence[Sequence[int]], lr: float = 0.02,
              mu: float = 0.95, weight_decay: float = 0.0, method: str = "standard",
              steps: int = NS_STEPS, coeffs: Tuple[float, float, float] = (NS_A, NS_B, NS_C),
              eps: float = NS_EPS, store_fmt: Optional[str] = None,
              entries: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """One Muon step over a packed buffer described by `table`.

    params/grads/momentum: flat arrays of the packed buffer ([DM]: one contiguous
    buffer per owner). table: (offset, rows, cols, split_rows[, split_cols]) per
    entry, each matrix row-major at `offset` ([DS]: grads are recovered by
    reshape(p.shape)).
    Returns float64 copies of the new params, new momentum and the update O
    (zero outside the entries). `entries` restricts the work to those entries.
    [DS] 核心算子: p <- p * (1 - lr * wd), then p <- p - lr * O.
    """
    p = np.asarray(params, dtype=np.float64).copy()
    M = np.asarray(momentum, dtype=np.float64).copy()
    G = np.asarray(grads, dtype=np.float64)
    O_all = np.zeros_like(p)
    idx = range(len(table)) if entries is None else entries
    for i in idx:
        off, rows, cols, split_r, split_c = _entry(table[i])
        span = slice(off, off + rows * cols)
        M[span] = momentum_update(M[span], G[span], mu)
        Mm = M[span].reshape(rows, cols)
        O = np.empty((rows, cols))
        for r0, nr, c0, nc in problem_blocks(rows, cols, split_r, split_c):
            O[r0:r0 + nr, c0:c0 + nc] = orthogonalise(Mm[r0:r0 + nr, c0:c0 + nc], method, steps,
                                                      coeffs, eps, store_fmt)
        O_all[span] = O.ravel()
        p[span] = p[span] * (1.0 - lr * weight_decay)
        p[span] = p[span] - lr * O_all[span]
    return {"params": p, "momentum": M, "update": O_all}


def partition_windows(table: Sequence[Sequence[int]], start: int,
                      stop: int) -> List[Tuple[int, int, int]]:
    """(lo, hi, param_offset) per entry for the holder of the flat partition
    [start, stop) of the full layout: the part of each matrix (flattened in
    stored row-major order) that falls in the partition, and where it sits in
    the partition. (0, 0, 0) for a matrix the partition does not touch."""
    out = []
    for e in table:
        off, rows, cols = e[:3]
        a, b = max(start, off), min(stop, off + rows * cols)
        out.append((a - off, b - off, a - start) if a < b else (0, 0, 0))
    return out


def window_step(partition: np.ndarray, grads: np.ndarray, momentum: np.ndarray,
                table: Sequence[Sequence[int]],
                windows: Sequence[Tuple[int, int, int]], lr: float = 0.02,
                weight_decay: float = 0.0, **kw) -> Dict[str, np.ndarray]:
    """One Muon step for the holder of a flat parameter partition.

    [DS] ZeRO stage support, partition boundaries: when a Muon matrix straddles a
    ZeRO partition boundary, every rank that holds part of it receives the whole
    reduced gradient before the nonlinear update. Reading: the holder keeps the
    whole momentum of the matrix, forms the whole update O as muon_step does,
    and applies p <- p (1 - lr wd) - lr O to the elements of its own window only.
    windows[i] = (lo, hi, param_offset): elements [lo, hi) of entry i, flat in
    stored order, at partition[param_offset:param_offset + hi - lo].
    grads/momentum are in the table's full layout; `kw` goes to muon_step.
    Returns float64 copies of the new partition, the new momentum and O.
    """
    full = muon_step(np.zeros(len(momentum)), grads, momentum, table, lr=0.0, **kw)
    part = np.asarray(partition, dtype=np.float64).copy()
    O = full["update"]
    for e, (lo, hi, po) in zip(table, windows):
        off = e[0]
        if hi <= lo:
            continue
        span = slice(po, po + hi - lo)
        part[span] = part[span] * (1.0 - lr * weight_decay)
        part[span] = part[span] - lr * O[off + lo:off + hi]
    return {"partition": part, "momentum": full["momentum"], "update": O}


def adamw_step(p: np.ndarray, g: np.ndarray, m: np.ndarray, v: np.ndarray, lr: float,
               beta1: float, beta2: float, eps: float, weight_decay: float, t: int):
    """[DS] 核心算子 / 如何用 DeepSpeed 配置启用 Muon: the Adam fallback for non-2D
    parameters, in AdamW mode. Returns float64 (p, m, v) after step t >= 1."""
    p = np.asarray(p, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** t)
    v_hat = v / (1.0 - beta2 ** t)
    p = p * (1.0 - lr * weight_decay)
    p = p - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p, m, v


def pack(arrays: Sequence[np.ndarray], table: Sequence[Sequence[int]],
         numel: int, dtype=np.float32) -> np.ndarray:
    """[DM] packed buffer: each matrix copied row-major to its offset; gaps zero."""
    out = np.zeros(numel, dtype=dtype)
    for arr, e in zip(arrays, table):
        off, rows, cols = e[:3]
        out[off:off + rows * cols] = np.asarray(arr).reshape(rows * cols)
    return out


def unpack(packed: np.ndarray, table: Sequence[Sequence[int]]):
    return [packed[e[0]:e[0] + e[1] * e[2]].reshape(e[1], e[2]).copy() for e in table]
