"""GPU: the symmetric products are stored as exactly symmetric matrices.

The symmetric launches compute the lower tiles of A = X X^T, B = aI + bA + cA^2
(standard) or R, Q and T = R Q (Gram) and store each tile together with its
mirror; the diagonal tiles store their lower part and its mirror element by
element. A wrong or missing mirror element changes a step's result by far less
than the parity gates can see, so these tests read the workspace after a step
instead: it was filled with a sentinel first, and it must then hold the expected
number of m x m regions (at the padded row pitch the library uses) that are
bit-for-bit symmetric, free of the sentinel and with a non-zero diagonal.

The workspace is scanned at every 256-byte boundary, where its buffers start,
so the test depends on no other detail of its layout.
"""
import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu

# (method, iteration type, rows, cols, symmetric buffers at least). With a
# short side above 128 every product runs through the tiled launches; the sizes
# cover symmetric 128-tiles (m mod 256 <= 128) and 256-tiles, ragged diagonal
# tiles and a matrix stored transposed (rows > cols). With a short side of at
# most 128 the 16-bit paths are fused: standard keeps A' (from the update + Gram
# pass) and B; Gram keeps R0 (from the X0 + R0 pass) in the workspace, its chain
# runs in LDS.
CASES = [
    ("standard", "bf16", 300, 520, 2),
    ("standard", "bf16", 700, 900, 2),
    ("standard", "bf16", 1000, 460, 2),
    ("standard", "f32", 300, 520, 2),
    ("gram", "f16", 300, 700, 3),
    ("gram", "f16", 700, 1000, 3),
    ("standard", "bf16", 100, 700, 2),
    ("gram", "f16", 700, 100, 1),
]


def _symmetric_regions(ws, m, esz):
    """Offsets (bytes) and pitches of the m x m regions of `ws` (raw bytes) that
    are exactly symmetric, sentinel-free and have no zero on the diagonal."""
    words = ws.view(np.uint16 if esz == 2 else np.uint32)
    sentinel = np.iinfo(words.dtype).max
    found = []
    rng = np.random.default_rng(0)
    pi, pj = rng.integers(0, m, 16), rng.integers(0, m, 16)
    for pitch in sorted({-(-m // 128) * 128, -(-m // 256) * 256}):
        span = (m - 1) * pitch + m
        starts = np.arange(0, words.size - span + 1, 256 // esz)
        if starts.size == 0:
            continue
        # quick filter: 16 random pairs (i, j) against (j, i)
        a = words[starts[:, None] + pi * pitch + pj]
        b = words[starts[:, None] + pj * pitch + pi]
        for s in starts[np.all(a == b, axis=1)]:
            R = words[s:s + span + (pitch - m)].reshape(m, pitch)[:, :m] if span + (pitch - m) <= words.size - s \
                else np.stack([words[s + i * pitch:s + i * pitch + m] for i in range(m)])
            # every diagonal entry of these products is non-zero (R and A have
            # squared row norms there), while a principal submatrix that starts
            # inside a buffer runs into its zero padding rows
            if np.any(R == sentinel) or np.any((np.diagonal(R) & (sentinel >> 1)) == 0):
                continue
            if np.array_equal(R, R.T):
                found.append((int(s) * esz, pitch))
    # a principal submatrix of a symmetric buffer is symmetric too: keep only
    # regions that do not overlap one found earlier, one per buffer
    kept, end = [], -1
    for off, pitch in sorted(found):
        if off >= end:
            kept.append((off, pitch))
            end = off + m * pitch * esz
    return kept


@pytest.mark.parametrize("method,ns_dtype,rows,cols,expect", CASES)
def test_symmetric_products_stored_symmetric(lib, method, ns_dtype, rows, cols, expect):
    import torch
    print(f"[case] {method} {ns_dtype} {rows}x{cols}", flush=True)
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(rows * 7 + cols)
    n = rows * cols
    tab = [(0, rows, cols, 0)]
    h = lib.hyper(ns_method=method, ns_dtype=ns_dtype, grad_dtype="bf16", lr=0.02, momentum=0.95,
                  weight_decay=0.1)
    nbytes = lib.workspace_size(tab, h)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=dev)
    p = torch.from_numpy(rng.standard_normal(n).astype(np.float32)).to(dev)
    g = torch.from_numpy(W.f32_to_bf16_bits(rng.standard_normal(n).astype(np.float32)).view(np.int16)).to(dev)
    g = g.view(torch.bfloat16)
    m = torch.from_numpy((0.3 * rng.standard_normal(n)).astype(np.float32)).to(dev)
    lib.step(p, g, m, tab, h, ws=ws)
    torch.cuda.synchronize()
    esz = 4 if ns_dtype == "f32" else 2
    found = _symmetric_regions(ws.cpu().numpy(), min(rows, cols), esz)
    print(f"[symmetric regions] (byte offset, row pitch): {found}", flush=True)
    assert len(found) >= expect, found
