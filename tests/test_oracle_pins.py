"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each check is independent of the oracle's own formulas: constants printed by the
DeepSpeed-Muon article, the singular-value closed form of an odd matrix
polynomial, special inputs whose iteration reduces to scalar arithmetic,
orthogonal equivariance, library routines (numpy's float16 cast, torch's bf16
cast and AdamW), and brute force on tiny inputs.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import rounding

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "deepspeed_muon_constants.json")


def phi(s, steps=5, a=3.4445, b=-4.7750, c=2.0315):
    """The scalar quintic applied `steps` times (what NS does to a singular value)."""
    s = np.asarray(s, dtype=np.float64)
    for _ in range(steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def svd_closed_form(Y, eps=1e-7, steps=5):
    U, s, Vt = np.linalg.svd(Y, full_matrices=False)
    return (U * phi(s / (np.linalg.norm(Y) + eps), steps)) @ Vt


def rel(x, y):
    return np.linalg.norm(x - y) / np.linalg.norm(y)


def rand_orth(rng, n):
    q, r = np.linalg.qr(rng.standard_normal((n, n)))
    return q * np.sign(np.diag(r))


# --------------------------------------------------------------------------- constants

def test_constants_match_article():
    g = json.load(open(GOLDEN))
    ns = g["newton_schulz"]
    assert (oracle.NS_A, oracle.NS_B, oracle.NS_C) == (ns["a"], ns["b"], ns["c"])
    assert oracle.NS_STEPS == ns["steps"]
    assert tuple(oracle.NS_METHODS) == tuple(g["ns_methods"]["methods"])
    assert oracle.DEFAULT_NS_METHOD == g["ns_methods"]["default"]
    d = g["group_defaults"]
    assert oracle.MUON_DEFAULTS == d["muon"]
    assert oracle.ADAM_DEFAULTS["lr"] == d["adam"]["lr"]
    assert list(oracle.ADAM_DEFAULTS["betas"]) == d["adam"]["betas"]
    assert oracle.ADAM_DEFAULTS["eps"] == d["adam"]["eps"]


def test_slope_at_zero_is_a():
    # the article: coefficients chosen to maximise the slope at zero -> p'(0) = a
    h = 1e-9
    assert abs(phi(h, steps=1) / h - 3.4445) < 1e-6


# --------------------------------------------------------------------------- rounding

def _f16_cases(rng):
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.uniform(-9, 5, 20000),
        [0.0, -0.0, 65504.0, 65519.99, 65520.0, -65520.0, 1e6, 6.1e-5, 5.96e-8,
         2.98e-8, 2.99e-8, -1e-9, np.inf, -np.inf],
    ])
    # exact midpoints between adjacent fp16 values (ties)
    h = rng.standard_normal(5000).astype(np.float16)
    h = h[np.isfinite(h)]
    nxt = np.nextafter(h, np.float16(np.inf), dtype=np.float16)
    mid = (h.astype(np.float64) + nxt.astype(np.float64)) / 2
    return np.concatenate([x, mid[np.isfinite(mid)]])


def test_round_f16_matches_numpy_cast():
    rng = np.random.default_rng(1)
    x = _f16_cases(rng)
    ours = rounding.round_to(x, "f16")
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).astype(np.float64)
    assert np.array_equal(ours, ref)
    assert np.array_equal(np.signbit(ours), np.signbit(ref))


def test_round_f32_matches_cast():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(20000) * 10.0 ** rng.uniform(-44, 38, 20000)
    x = np.concatenate([x, [3.5e38, -3.5e38, 1e-46, 7e-46]])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float32).astype(np.float64)
    assert np.array_equal(rounding.round_to(x, "f32"), ref)


def test_round_bf16_matches_torch_on_f32_inputs():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(50000) * 10.0 ** rng.uniform(-40, 38, 50000)).astype(np.float32)
    bits = rng.integers(0, 2 ** 16, 2000, dtype=np.uint32)
    ties = ((bits << 16) | 0x8000).astype(np.uint32).view(np.float32)  # exact bf16 midpoints
    x = np.concatenate([x, ties[np.isfinite(ties)]])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(rounding.round_to(x.astype(np.float64), "bf16"), ref)


def _bf16_neighbours(r):
    """Adjacent bf16 values below/above a finite bf16 value r (brute force on bits)."""
    u = np.array([r], dtype=np.float32).view(np.uint32)[0] >> 16
    up = np.array([(u + 1) << 16], dtype=np.uint32).view(np.float32)[0]
    dn = np.array([(u - 1) << 16], dtype=np.uint32).view(np.float32)[0] if (u & 0x7FFF) else -r
    return float(min(up, dn)), float(max(up, dn)), int(u)


def test_round_bf16_nearest_by_brute_force():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(3000) * 10.0 ** rng.uniform(-30, 30, 3000)
    r = rounding.round_to(x, "bf16")
    for xi, ri in zip(x, r):
        f = np.float32(ri)
        assert float(f) == ri and (np.array([f]).view(np.uint32)[0] & 0xFFFF) == 0
        lo, hi, u = _bf16_neighbours(ri)
        for nb in (lo, hi):
            d_r, d_n = abs(xi - ri), abs(xi - nb)
            assert d_r < d_n or (d_r == d_n and (u & 1) == 0)


def test_round_special_values():
    for fmt in ("bf16", "f16", "f32"):
        out = rounding.round_to(np.array([np.nan, np.inf, -np.inf, -0.0]), fmt)
        assert np.isnan(out[0]) and out[1] == np.inf and out[2] == -np.inf
        assert out[3] == 0 and np.signbit(out[3])
    assert rounding.round_to(3.4e38, "bf16") == np.inf          # beyond bf16's largest finite
    assert rounding.round_to(1.0 + 2 ** -8, "bf16") == 1.0       # tie -> even


# --------------------------------------------------------------------------- Newton-Schulz

@pytest.mark.parametrize("shape", [(1, 1), (4, 4), (5, 3), (3, 5), (17, 33), (64, 96), (96, 64)])
@pytest.mark.parametrize("method", ["standard", "gram"])
def test_ns_matches_svd_closed_form(shape, method):
    rng = np.random.default_rng(sum(shape))
    Y = rng.standard_normal(shape)
    O = oracle.orthogonalise(Y, method)
    assert O.shape == Y.shape
    assert rel(O, svd_closed_form(Y)) < 1e-11


def test_ns_one_by_one_is_the_scalar_sequence():
    # 1x1: X0 = y/(|y| + eps); five quintic steps; known value near s = 1
    for y in (0.37, 5.0, 1e3):
        O = oracle.orthogonalise(np.array([[y]]), "standard")
        assert abs(O[0, 0] - phi(y / (y + 1e-7))) < 1e-13
    assert abs(phi(1.0) - 0.6964364) < 1e-6
    assert abs(oracle.orthogonalise(np.array([[-2.0]]), "gram")[0, 0] + phi(2 / (2 + 1e-7))) < 1e-13


@pytest.mark.parametrize("m,n", [(8, 8), (16, 40), (128, 256)])
def test_ns_orthonormal_rows(m, n):
    rng = np.random.default_rng(m * n)
    Qm = np.linalg.qr(rng.standard_normal((n, m)))[0].T     # m x n, orthonormal rows
    for method in ("standard", "gram"):
        O = oracle.orthogonalise(Qm, method)
        assert rel(O, phi(1.0 / (np.sqrt(m) + 1e-7)) * Qm) < 1e-12
    if m == 128:
        assert abs(phi(1 / np.sqrt(128)) - 0.722762160445) < 1e-11


def test_ns_equivariance_and_transpose():
    rng = np.random.default_rng(7)
    Y = rng.standard_normal((12, 20))
    U, V = rand_orth(rng, 12), rand_orth(rng, 20)
    for method in ("standard", "gram"):
        O = oracle.orthogonalise(Y, method)
        assert rel(oracle.orthogonalise(U @ Y @ V.T, method), U @ O @ V.T) < 1e-12
        assert rel(oracle.orthogonalise(Y.T, method), O.T) < 1e-13


def test_ns_scale_invariance_and_zero():
    rng = np.random.default_rng(8)
    Y = rng.standard_normal((10, 14))
    # exact without eps; with eps = 1e-7 only up to eps / ||Y||
    assert rel(oracle.orthogonalise(1e3 * Y, eps=0.0), oracle.orthogonalise(Y, eps=0.0)) < 1e-13
    assert rel(oracle.orthogonalise(1e3 * Y), oracle.orthogonalise(Y)) < 1e-7
    assert np.all(oracle.orthogonalise(np.zeros((6, 9))) == 0)


def test_gram_equals_standard_in_float64():
    rng = np.random.default_rng(9)
    for shape in ((32, 32), (24, 80), (80, 24)):
        Y = rng.standard_normal(shape) @ np.diag(np.logspace(0, -3, shape[1]))
        assert rel(oracle.orthogonalise(Y, "gram"), oracle.orthogonalise(Y, "standard")) < 1e-11


def test_ns_output_singular_values_in_band():
    rng = np.random.default_rng(10)
    m, n = 20, 30
    s = np.linspace(1.0, 0.25, m)            # normalised values all >= 0.05 after scaling
    U, V = rand_orth(rng, m), rand_orth(rng, n)[:m]
    Y = (U * s) @ V
    so = np.linalg.svd(oracle.orthogonalise(Y), compute_uv=False)
    assert so.min() > 0.6818 and so.max() < 1.2024


def _hadamard(n):
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_faithful_standard_on_hadamard_reduces_to_scalars(fmt):
    """Rows of a Hadamard matrix: X_k = t_k H, A_k = n t_k^2 I, B_k = beta_k I, so the
    stored iteration is a scalar one. Pins the storage points (X0, A, B = a I +
    b A + c A A, X1..X4 stored; X5 not) of the faithful mode."""
    m, n = 16, 64
    H = _hadamard(n)[:m]
    rnd = lambda z: float(rounding.round_to(z, fmt))
    a, b, c = 3.4445, -4.7750, 2.0315
    t = rnd(1.0 / np.sqrt(m * n))      # eps = 0: X0 = H / ||H||_F, entries exact
    for k in range(5):
        alpha = rnd(n * t * t)
        beta = rnd(a + b * alpha + c * alpha * alpha)
        t_next = beta * t
        t = t_next if k == 4 else rnd(t_next)
    O = oracle.orthogonalise(H, "standard", eps=0.0, store_fmt=fmt)
    assert np.array_equal(O, t * H)


def test_faithful_gram_on_hadamard_reduces_to_scalars():
    m, n = 16, 64
    H = _hadamard(n)[:m]
    rnd = lambda z: float(rounding.round_to(z, "f16"))
    a, b, c = 3.4445, -4.7750, 2.0315
    s = 16.0                           # 2**ceil(log2 16)
    x0 = rnd(1.0 / np.sqrt(m * n))
    r = rnd(s * n * x0 * x0)
    p = None
    for k in range(5):
        q = rnd(a + (b / s) * r + (c / s ** 2) * r * r)
        p = q if k == 0 else rnd(q * p)
        if k < 4:
            rq = rnd(r * q)
            r = rnd(q * rq)
    O = oracle.orthogonalise(H, "gram", eps=0.0, store_fmt="f16")
    assert oracle.gram_scale(m) == s
    assert np.array_equal(O, (p * x0) * H)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_faithful_row_scaled_hadamard_is_per_row_scalars(fmt):
    """Y = D H with D diagonal and H rows of a Hadamard matrix (H H^T = n I): every
    stored iterate is diagonal, so each row follows its own scalar recurrence,
    rounded at every storage point. Distinct row scales catch transposed or
    misordered products (B X vs X B, Q P vs P Q, P X0) that a single scale hides."""
    m, n = 8, 32
    H = _hadamard(n)[:m]
    d = np.array([1.0, 0.5, 2.0, 0.125, 3.0, 0.75, 1.5, 0.3])
    nu = np.sqrt(n * np.sum(d * d))
    rnd = lambda z: float(rounding.round_to(z, fmt))
    a, b, c = 3.4445, -4.7750, 2.0315
    # standard
    t = np.array([rnd(di / nu) for di in d])
    for k in range(5):
        al = np.array([rnd(n * ti * ti) for ti in t])
        be = np.array([rnd(a + b * x + c * x * x) for x in al])
        nxt = be * t
        t = nxt if k == 4 else np.array([rnd(x) for x in nxt])
    O = oracle.orthogonalise(d[:, None] * H, "standard", eps=0.0, store_fmt=fmt)
    assert np.array_equal(O, t[:, None] * H)
    if fmt != "f16":
        return
    # gram, with the fp16 scale of the Gram state
    s = oracle.gram_scale(m)
    x0 = np.array([rnd(di / nu) for di in d])
    r = np.array([rnd(s * n * x * x) for x in x0])
    p = None
    for k in range(5):
        q = np.array([rnd(a + (b / s) * ri + (c / s ** 2) * ri * ri) for ri in r])
        p = q if k == 0 else np.array([rnd(qi * pi) for qi, pi in zip(q, p)])
        if k < 4:
            rq = np.array([rnd(ri * qi) for ri, qi in zip(r, q)])
            r = np.array([rnd(qi * x) for qi, x in zip(q, rq)])
    O = oracle.orthogonalise(d[:, None] * H, "gram", eps=0.0, store_fmt="f16")
    assert np.array_equal(O, (p * x0)[:, None] * H)


def _fixed_order_matmul(A, B):
    """A B with every entry summed over k = 0, 1, ... in that order (one rounding
    per product and per addition). Entry (i, j) of X X^T and entry (j, i) then add
    the same products in the same order, so the result is exactly symmetric."""
    C = np.zeros((A.shape[0], B.shape[1]))
    for k in range(A.shape[1]):
        C = C + np.outer(A[:, k], B[k, :])
    return C


def _recording_storer(fmt, seen):
    def rec(z):
        z = rounding.round_to(z, fmt)
        seen.append(z)
        return z
    return rec


def test_faithful_symmetric_storage_is_a_fixed_order_evaluation():
    """The faithful mode stores A, B (standard) and R0 and the first Q (gram) as
    mirrored lower triangles. That is no approximation: a fixed-order evaluation
    of each, from the stored operands, gives the same bits (and is symmetric)."""
    rng = np.random.default_rng(21)
    X0 = rng.standard_normal((6, 10)) / 8
    a, b, c = 3.4445, -4.7750, 2.0315
    rnd = lambda z: rounding.round_to(z, "f16")
    # standard: X0, then A, B, X1, A, B, ...
    seen = []
    oracle.newton_schulz_standard(X0, 5, store=_recording_storer("f16", seen))
    X = seen[0]
    for k in range(5):
        A, B = seen[1 + 3 * k], seen[2 + 3 * k]
        A_fo = _fixed_order_matmul(X, X.T)
        assert np.array_equal(A_fo, A_fo.T)
        assert np.array_equal(A, rnd(A_fo)), k
        B_fo = a * np.eye(6) + b * A + c * _fixed_order_matmul(A, A)
        assert np.array_equal(B_fo, B_fo.T)
        assert np.array_equal(B, rnd(B_fo)), k
        if k < 4:
            X = seen[3 + 3 * k]
    # gram: X0, R0, Q0, then T0, R1, Q1, P1, ...
    seen = []
    s = 8.0
    oracle.newton_schulz_gram(X0, 5, store=_recording_storer("f16", seen), scale=s)
    X, R0, Q0 = seen[0], seen[1], seen[2]
    R0_fo = s * _fixed_order_matmul(X, X.T)
    assert np.array_equal(R0, rnd(R0_fo)) and np.array_equal(R0_fo, R0_fo.T)
    Q0_fo = a * np.eye(6) + (b / s) * R0 + (c / s ** 2) * _fixed_order_matmul(R0, R0)
    assert np.array_equal(Q0, rnd(Q0_fo)) and np.array_equal(Q0_fo, Q0_fo.T)


def test_faithful_gram_stores_later_iterates_as_computed():
    """Once Q is rounded it no longer commutes with R, so T = R Q and R <- Q T are
    not symmetric; the faithful mode stores them (and every later Q, a
    polynomial in such an R) as computed, like P."""
    rng = np.random.default_rng(22)
    X0 = rng.standard_normal((6, 10)) / 8
    seen = []
    oracle.newton_schulz_gram(X0, 5, store=_recording_storer("f16", seen), scale=8.0)
    sq = [z for z in seen if z.shape == (6, 6)]
    # R0, Q0; step 0: T, R; steps 1-3: Q, P, T, R; step 4: Q, P
    assert len(sq) == 2 + 2 + 3 * 4 + 2
    R0, Q0, T0, R1, Q1, P1 = sq[:6]
    assert np.array_equal(R0, R0.T) and np.array_equal(Q0, Q0.T)
    for z in (T0, R1, Q1, P1):
        assert not np.array_equal(z, z.T)
    rnd = lambda z: rounding.round_to(z, "f16")
    assert np.array_equal(T0, rnd(R0 @ Q0))
    assert np.array_equal(R1, rnd(Q0 @ T0))
    assert np.array_equal(P1, rnd(Q1 @ Q0))            # P starts as Q0


def test_gram_scale_at_the_workload_shapes():
    """2^ceil(log2 m), capped at 2^15: values worked out by hand for the short
    sides of the workloads (head blocks 128, experts 1408, layers 2048 / 4096,
    the long MLP side 5632 and 11008), the size limit and beyond the cap."""
    table = {1: 1, 2: 2, 3: 4, 5: 8, 100: 128, 128: 128, 129: 256, 1000: 1024, 1408: 2048,
             2047: 2048, 2048: 2048, 2049: 4096, 4096: 4096, 5632: 8192, 11008: 16384,
             16384: 16384, 16385: 32768, 32768: 32768, 40000: 32768, 1 << 20: 32768}
    for m, s in table.items():
        assert oracle.gram_scale(m) == float(s), m


def test_faithful_first_storage_point_is_x0():
    rng = np.random.default_rng(11)
    Y = rng.standard_normal((8, 12))
    X0 = Y / (np.linalg.norm(Y) + 1e-7)
    assert np.array_equal(oracle.orthogonalise(Y, "standard", steps=0, store_fmt="bf16"),
                          rounding.round_to(X0, "bf16"))


def test_faithful_modes_stay_near_exact_on_gaussian():
    rng = np.random.default_rng(12)
    Y = rng.standard_normal((64, 160))
    ex = oracle.orthogonalise(Y)
    assert rel(oracle.orthogonalise(Y, "standard", store_fmt="bf16"), ex) < 3e-2
    assert rel(oracle.orthogonalise(Y, "gram", store_fmt="f16"), ex) < 1e-2
    assert rel(oracle.orthogonalise(Y, "standard", store_fmt="f32"), ex) < 1e-5


# --------------------------------------------------------------------------- full step

def _table(shapes, align=8):
    """shapes: (rows, cols, split_rows[, split_cols])."""
    offs, cur, tab = [], 0, []
    for sh in shapes:
        r, c = sh[0], sh[1]
        cur = (cur + align - 1) // align * align
        tab.append((cur,) + tuple(sh))
        cur += r * c
    return tab, cur


def test_step_rule_against_closed_form():
    rng = np.random.default_rng(13)
    tab, n = _table([(6, 10, 0), (12, 4, 0), (8, 8, 4)])
    p0, g, m0 = rng.standard_normal(n), rng.standard_normal(n), rng.standard_normal(n)
    lr, mu, wd = 0.02, 0.95, 0.1
    out = oracle.muon_step(p0, g, m0, tab, lr=lr, mu=mu, weight_decay=wd)
    for off, r, c, s in tab:
        sl = slice(off, off + r * c)
        M = mu * m0[sl] + g[sl]
        assert np.allclose(out["momentum"][sl], M, rtol=0, atol=1e-15)
        Mm = M.reshape(r, c)
        blocks = [(0, r)] if s == 0 else [(i, s) for i in range(0, r, s)]
        O = np.vstack([svd_closed_form(Mm[i:i + k]) for i, k in blocks])
        assert rel(out["update"][sl].reshape(r, c), O) < 1e-11
        expect = p0[sl] * (1 - lr * wd) - lr * O.ravel()
        assert np.max(np.abs(out["params"][sl] - expect)) < 1e-12
    # bytes outside the entries are untouched
    mask = np.ones(n, bool)
    for off, r, c, _ in tab:
        mask[off:off + r * c] = False
    assert np.array_equal(out["params"][mask], p0[mask])
    assert np.array_equal(out["momentum"][mask], m0[mask])


def test_step_special_cases():
    rng = np.random.default_rng(14)
    tab, n = _table([(5, 7, 0), (9, 3, 0)])
    p0, g = rng.standard_normal(n), rng.standard_normal(n)
    zero = np.zeros(n)
    # lr = 0: params unchanged bit-for-bit
    assert np.array_equal(oracle.muon_step(p0, g, zero, tab, lr=0.0, weight_decay=0.1)["params"], p0)
    # mu = 0: momentum equals the gradient exactly
    M1 = oracle.muon_step(p0, g, zero + 3.0, tab, mu=0.0)["momentum"]
    for off, r, c, _ in tab:
        assert np.array_equal(M1[off:off + r * c], g[off:off + r * c])
    # zero gradient and momentum: pure decay
    out = oracle.muon_step(p0, zero, zero, tab, lr=0.5, weight_decay=0.2)
    for off, r, c, _ in tab:
        sl = slice(off, off + r * c)
        assert np.array_equal(out["params"][sl], p0[sl] * (1 - 0.5 * 0.2))
    # constant gradient, three steps: M = (1 + mu + mu^2) G
    M = zero
    for _ in range(3):
        M = oracle.muon_step(p0, g, M, tab, mu=0.95)["momentum"]
    for off, r, c, _ in tab:
        sl = slice(off, off + r * c)
        assert np.allclose(M[sl], (1 + 0.95 + 0.95 ** 2) * g[sl], rtol=1e-15, atol=1e-15)


def test_split_equals_separate_entries():
    rng = np.random.default_rng(15)
    rows, cols, k = 12, 10, 4
    tab_split = [(0, rows, cols, k)]
    tab_sep = [(i * k * cols, k, cols, 0) for i in range(rows // k)]
    n = rows * cols
    p0, g = rng.standard_normal(n), rng.standard_normal(n)
    a = oracle.muon_step(p0, g, np.zeros(n), tab_split)
    b = oracle.muon_step(p0, g, np.zeros(n), tab_sep)
    for key in ("params", "momentum", "update"):
        assert np.array_equal(a[key], b[key])
    # each block has its own norm: scaling one block's gradient leaves its update unchanged
    g2 = g.copy()
    g2[:k * cols] *= 100.0
    c2 = oracle.muon_step(p0, g2, np.zeros(n), tab_split)
    assert rel(c2["update"][:k * cols], a["update"][:k * cols]) < 1e-7


def _blocks_as_entries(rows, cols, pr, pc):
    """Table of the pr x pc blocks of a rows x cols matrix stored as separate
    contiguous matrices, and the index map taking those packed elements to
    the matrix's flat positions."""
    idx = np.arange(rows * cols).reshape(rows, cols)
    tab, order, cur = [], [], 0
    for r0 in range(0, rows, pr):
        for c0 in range(0, cols, pc):
            tab.append((cur, pr, pc, 0))
            order.append(idx[r0:r0 + pr, c0:c0 + pc].ravel())
            cur += pr * pc
    return tab, np.concatenate(order)


@pytest.mark.parametrize("method", ["standard", "gram"])
@pytest.mark.parametrize("shape", [(10, 12, 0, 4), (12, 10, 0, 5), (8, 12, 4, 6)])
def test_column_and_grid_split_equal_separate_entries(method, shape):
    # a column block (or a split_rows x split_cols tile) is its own problem: its
    # values, copied out as a matrix of their own, give the same update, and the
    # blocks' momenta and weights move as the copies' do
    rng = np.random.default_rng(18)
    rows, cols, sr, sc = shape
    n = rows * cols
    p0, g, m0 = rng.standard_normal(n), rng.standard_normal(n), rng.standard_normal(n)
    kw = dict(lr=0.03, weight_decay=0.1, mu=0.9, method=method)
    a = oracle.muon_step(p0, g, m0, [(0, rows, cols, sr, sc)], **kw)
    tab, order = _blocks_as_entries(rows, cols, sr or rows, sc or cols)
    b = oracle.muon_step(p0[order], g[order], m0[order], tab, **kw)
    for key in ("params", "momentum", "update"):
        assert np.allclose(a[key][order], b[key], rtol=0, atol=1e-13), key
    # every block has its own norm: scaling one block's gradient and momentum
    # leaves the update of every block unchanged
    s = np.ones((rows, cols))
    s[:sr or rows, :sc or cols] = 100.0
    c = oracle.muon_step(p0, g * s.ravel(), m0 * s.ravel(), [(0, rows, cols, sr, sc)], **kw)
    assert rel(c["update"], a["update"]) < 1e-7


@pytest.mark.parametrize("method", ["standard", "gram"])
def test_column_split_is_the_row_split_of_the_transpose(method):
    # polar(B^T) = polar(B)^T, and the iteration runs on the short side either
    # way: splitting W by columns gives the transpose of splitting W^T by rows
    rng = np.random.default_rng(19)
    rows, cols, k = 9, 24, 6
    W = rng.standard_normal((rows, cols))
    Wt = np.ascontiguousarray(W.T)
    a = oracle.muon_step(np.zeros(W.size), W.ravel(), np.zeros(W.size), [(0, rows, cols, 0, k)],
                         mu=0.0, method=method)
    b = oracle.muon_step(np.zeros(W.size), Wt.ravel(), np.zeros(W.size), [(0, cols, rows, k)],
                         mu=0.0, method=method)
    Oa = a["update"].reshape(rows, cols)
    Ob = b["update"].reshape(cols, rows)
    assert np.allclose(Oa, Ob.T, rtol=0, atol=1e-13)
    # each 9 x 6 block is close to a matrix with orthonormal columns after five
    # quintic steps (singular values in the coefficients' band, not all 1)
    for c0 in range(0, cols, k):
        sv = np.linalg.svd(Oa[:, c0:c0 + k], compute_uv=False)
        assert sv.min() > 0.6 and sv.max() < 1.25


def test_column_split_flops_and_windows():
    from oracle import planner
    # a column-split o_proj costs what its row-split transpose costs; a grid
    # costs one problem per tile
    assert planner.matrix_flops(4096, 4096, 0, split_cols=128) == planner.matrix_flops(4096, 4096, 128)
    assert planner.matrix_flops(512, 768, 256, split_cols=384) == 4 * planner.ns_flops(256, 384)
    # windows are flat in the matrix whatever the split: every element of a
    # column-split matrix falls in exactly one holder's window
    tab, n = _table([(6, 10, 0, 5), (12, 4, 0, 2), (8, 8, 4, 4)])
    seen = np.zeros(n, int)
    for a, b in _holders(n, [7, 33, 61, 100]):
        for (off, r, c, *_), (lo, hi, po) in zip(tab, oracle.partition_windows(tab, a, b)):
            if hi > lo:
                assert a + po == off + lo
                seen[off + lo:off + hi] += 1
    for off, r, c, *_ in tab:
        assert np.all(seen[off:off + r * c] == 1)
    # and the holders' windows together carry the whole step's update
    rng = np.random.default_rng(20)
    p0, g, m0 = rng.standard_normal(n), rng.standard_normal(n), rng.standard_normal(n)
    kw = dict(lr=0.03, weight_decay=0.1, mu=0.9, method="standard")
    whole = oracle.muon_step(p0, g, m0, tab, **kw)
    got = p0.copy()
    for a, b in _holders(n, [7, 33, 61, 100]):
        got[a:b] = oracle.window_step(p0[a:b], g, m0, tab, oracle.partition_windows(tab, a, b),
                                      **kw)["partition"]
    assert np.array_equal(got, whole["params"])


def test_pack_unpack_roundtrip():
    rng = np.random.default_rng(16)
    tab, n = _table([(3, 5, 0), (4, 4, 0), (1, 7, 0)])
    mats = [rng.standard_normal((r, c)).astype(np.float32) for _, r, c, _ in tab]
    packed = oracle.pack(mats, tab, n + 5)
    for a, b in zip(oracle.unpack(packed, tab), mats):
        assert np.array_equal(a, b)
    used = sum(r * c for _, r, c, _ in tab)
    assert np.count_nonzero(packed) <= used


# --------------------------------------------------------------------------- partitions

def _holders(n, cuts):
    edges = [0] + list(cuts) + [n]
    return list(zip(edges[:-1], edges[1:]))


def test_partition_windows_tile_the_layout():
    # every element of every matrix falls in exactly one holder's window, at the
    # partition index that the flat layout gives it
    tab, n = _table([(6, 10, 0), (12, 4, 0), (8, 8, 4)])
    for cuts in ([], [30], [7, 61, 100], [60, 108], [1, 2, 3]):
        seen = np.zeros(n, int)
        for a, b in _holders(n, cuts):
            for (off, r, c, _s), (lo, hi, po) in zip(tab, oracle.partition_windows(tab, a, b)):
                assert 0 <= lo <= hi <= r * c
                if hi > lo:
                    assert a + po == off + lo and a + po + (hi - lo) <= b
                    seen[off + lo:off + hi] += 1
        for off, r, c, _s in tab:
            assert np.all(seen[off:off + r * c] == 1)


def test_window_union_equals_whole_step():
    # [DS] partition boundaries: each holder gets the whole reduced gradient, so the
    # holders' windows together carry exactly the update of the unpartitioned step
    rng = np.random.default_rng(17)
    tab, n = _table([(6, 10, 0), (12, 4, 0), (8, 8, 4), (5, 5, 0)])
    p0, g, m0 = rng.standard_normal(n), rng.standard_normal(n), rng.standard_normal(n)
    kw = dict(lr=0.03, weight_decay=0.1, mu=0.9, method="standard")
    whole = oracle.muon_step(p0, g, m0, tab, **kw)
    for cuts in ([33], [7, 61, 100], [60, 108, 120, 150]):
        got = p0.copy()
        for a, b in _holders(n, cuts):
            out = oracle.window_step(p0[a:b], g, m0, tab, oracle.partition_windows(tab, a, b), **kw)
            got[a:b] = out["partition"]
            assert np.array_equal(out["momentum"], whole["momentum"])
            assert np.array_equal(out["update"], whole["update"])
        assert np.array_equal(got, whole["params"])


def test_window_step_needs_the_whole_gradient():
    # the rule matters: orthogonalising only the rows a holder owns gives another
    # update, because the map from momentum to O is not elementwise
    rng = np.random.default_rng(18)
    rows, cols = 8, 12
    M = rng.standard_normal((rows, cols))
    O = oracle.orthogonalise(M, "standard")
    O_top = oracle.orthogonalise(M[:4], "standard")
    assert rel(O_top, O[:4]) > 0.1


def test_window_step_special_cases():
    rng = np.random.default_rng(19)
    tab, n = _table([(6, 10, 0), (12, 4, 0)])
    p0, g, m0 = rng.standard_normal(n), rng.standard_normal(n), rng.standard_normal(n)
    whole = oracle.muon_step(p0, g, m0, tab, lr=0.02, weight_decay=0.1)
    # one holder of everything: windows cover each matrix at its own offset
    wins = [(0, r * c, off) for off, r, c, _s in tab]
    out = oracle.window_step(p0, g, m0, tab, wins, lr=0.02, weight_decay=0.1)
    assert np.array_equal(out["partition"], whole["params"])
    # empty windows: the partition is untouched, the momentum still moves
    part = rng.standard_normal(17)
    out = oracle.window_step(part, g, m0, tab, [(0, 0, 0), (5, 5, 3)], lr=0.02)
    assert np.array_equal(out["partition"], part)
    assert np.array_equal(out["momentum"], whole["momentum"])
    # lr = 0 leaves the window as it was
    out = oracle.window_step(part, g, m0, tab, [(3, 10, 2), (0, 0, 0)], lr=0.0, weight_decay=0.3)
    assert np.array_equal(out["partition"], part)


# --------------------------------------------------------------------------- AdamW

def test_adamw_first_step_closed_form():
    rng = np.random.default_rng(17)
    p, g = rng.standard_normal(1000), rng.standard_normal(1000)
    g[:10] = 0.0
    lr, wd, eps = 3e-4, 0.1, 1e-8
    p1, m1, v1 = oracle.adamw_step(p, g, np.zeros(1000), np.zeros(1000), lr, 0.9, 0.95, eps, wd, 1)
    expect = p * (1 - lr * wd) - lr * g / (np.abs(g) + eps)
    assert np.max(np.abs(p1 - expect)) < 1e-15
    assert np.array_equal(p1[:10], p[:10] * (1 - lr * wd))


def test_adamw_matches_torch_adamw():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(18)
    n = 257
    p0 = rng.standard_normal(n)
    grads = [rng.standard_normal(n) for _ in range(4)]
    lr, b1, b2, eps, wd = 3e-4, 0.9, 0.95, 1e-8, 0.1
    tp = torch.nn.Parameter(torch.tensor(p0, dtype=torch.float64))
    opt = torch.optim.AdamW([tp], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd)
    p, m, v = p0, np.zeros(n), np.zeros(n)
    for t, g in enumerate(grads, start=1):
        tp.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        p, m, v = oracle.adamw_step(p, g, m, v, lr, b1, b2, eps, wd, t)
    assert np.max(np.abs(p - tp.detach().numpy())) < 1e-14
