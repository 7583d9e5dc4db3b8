"""GPU: the largest problems the C ABI accepts, checked where the oracle can.

- Short side at MUON_MAX_SHORT_SIDE (16384 x 16384): too large for the float64
  oracle as a matrix, so the input is diagonal. Every product of the iteration
  then maps diagonal matrices to diagonal matrices entry by entry, so the
  storage-faithful iteration is one scalar recurrence per diagonal entry (the
  oracle's Newton-Schulz on 1 x 1 matrices, with the whole matrix's norm and
  Gram scale). Gates: the update is exactly zero off the diagonal, and its
  diagonal is within 3e-2 of the recurrences.
- Long side at MUON_MAX_LONG_SIDE (2 x 2^24, stored as is and transposed): the
  oracle runs the whole step; the usual gates (faithful 3e-2, momentum 1e-6).
"""
import numpy as np
import pytest

import oracle
from oracle.muon_oracle import gram_scale, newton_schulz_gram, newton_schulz_standard
from oracle.rounding import storer
import workloads as W
from gpu_helpers import rel

pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(900)]

MAX_SHORT = 16384
MAX_LONG = 1 << 24
LP_GATE = 3e-2


@pytest.mark.parametrize("method,ns_dtype", [("standard", "bf16"), ("gram", "f16")])
def test_max_short_side_diagonal(lib, method, ns_dtype):
    import torch
    nss = lib
    n = MAX_SHORT
    dev = "cuda:0"
    d_bits = W.f32_to_bf16_bits((1.0 + np.arange(n) / n).astype(np.float32))
    d = W.bf16_bits_to_f32(d_bits).astype(np.float64)
    print(f"[case] {n}x{n} diagonal, {method} {ns_dtype}", flush=True)
    p = torch.zeros(n * n, device=dev)
    g = torch.zeros(n * n, dtype=torch.bfloat16, device=dev)
    g.view(n, n).diagonal().copy_(torch.from_numpy(d.astype(np.float32)).to(dev).to(torch.bfloat16))
    m = torch.zeros(n * n, device=dev)
    u = torch.zeros(n * n, device=dev)
    h = nss.hyper(ns_method=method, ns_dtype=ns_dtype, grad_dtype="bf16", lr=0.02, momentum=0.95,
                  weight_decay=0.1)
    nss.step(p, g, m, [(0, n, n, 0)], h, update_out=u)
    torch.cuda.synchronize()
    U = u.view(n, n)
    diag = U.diagonal().clone()
    U.diagonal().zero_()
    off_nonzero = int(torch.count_nonzero(U).item())
    diag = diag.cpu().numpy().astype(np.float64)
    del p, g, m, u, U
    torch.cuda.empty_cache()
    assert off_nonzero == 0

    x0 = d / (np.linalg.norm(d) + 1e-7)          # M = G (zero momentum), then the whole matrix's norm
    st = storer(ns_dtype)
    if method == "standard":
        want = np.array([newton_schulz_standard(np.array([[x]]), store=st)[0, 0] for x in x0])
    else:
        s = gram_scale(n)
        want = np.array([newton_schulz_gram(np.array([[x]]), store=st, scale=s)[0, 0] for x in x0])
    err = rel(diag, want)
    print(f"  diagonal vs scalar recurrences: {err:.2e}", flush=True)
    assert err <= LP_GATE


def test_max_long_side(lib):
    import torch
    nss = lib
    shapes = [(2, MAX_LONG, 0), (MAX_LONG, 2, 0)]
    wl = W.custom_workload(shapes, grad_dtype="bf16", wid=116, grad_kind="gaussian")
    params, grads, mom = W.host_inputs(wl)
    tab = wl.table()
    print(f"[case] {shapes}", flush=True)
    from gpu_helpers import run_step
    h = nss.hyper(ns_method="standard", ns_dtype="bf16", grad_dtype="bf16", lr=wl.lr,
                  momentum=wl.momentum, weight_decay=wl.weight_decay)
    gpu = run_step(nss, params, grads, mom, tab, h)
    torch.cuda.empty_cache()
    g64 = W.grad_as_f64(wl, grads)
    ref = oracle.muon_step(params, g64, mom, tab, lr=wl.lr, mu=wl.momentum, weight_decay=wl.weight_decay,
                           method="standard", store_fmt="bf16")
    for i, (o, r, c, _) in enumerate(tab):
        sl = slice(o, o + r * c)
        eo = rel(gpu["update"][sl], ref["update"][sl])
        em = rel(gpu["momentum"][sl], ref["momentum"][sl])
        print(f"  entry {i} {r}x{c}: O {eo:.2e} M {em:.2e}", flush=True)
        assert eo <= LP_GATE and em <= 1e-6
