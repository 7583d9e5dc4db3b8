"""GPU: a model planned onto several owners (muon_plan_owners), each owner's
packed buffer built with muon_pack and stepped with muon_step, gives every
matrix exactly the step it gets when the whole model is one owner.

DMuon ("Z2 与 Z3 模式"): each Muon-target matrix has a single owner, which packs
its matrices into one contiguous buffer and alone runs their Newton-Schulz. One
GPU plays each owner in turn. Gates: new params, new momentum and update of
every matrix bit-equal to the single-owner step; every owner's table covers its
matrices once, inside its packed length.
"""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import run_step, to_device

pytestmark = pytest.mark.gpu

# two layers of a 1B-class decoder: q, k, v, o, gate, up, down
LAYER = [(2048, 2048, 0), (2048, 2048, 0), (2048, 2048, 0), (2048, 2048, 0),
         (5632, 2048, 0), (5632, 2048, 0), (2048, 5632, 0)]
# a few small and split matrices to fill odd corners
EXTRA = [(1024, 128, 128), (384, 200, 0), (1, 1, 0), (257, 33, 0)]


@pytest.mark.parametrize("method,ns_dtype,n_owners", [("standard", "bf16", 4), ("gram", "f16", 3)])
def test_owner_plan_equals_single_owner(lib, method, ns_dtype, n_owners):
    import torch
    nss = lib
    dev = "cuda:0"
    shapes = LAYER + LAYER + EXTRA
    layers = [0] * len(LAYER) + [1] * len(LAYER) + [2] * len(EXTRA)
    wl = W.custom_workload(shapes, grad_dtype="bf16", ns_dtype=ns_dtype, wid=180)
    params, grads, _ = W.host_inputs(wl)
    tab = wl.table()
    rng = np.random.default_rng(11)
    mom = (0.5 * W.grad_as_f64(wl, grads) * (1 + 0.1 * rng.standard_normal(wl.numel))).astype(np.float32)
    h = nss.hyper(ns_method=method, ns_dtype=ns_dtype, grad_dtype="bf16", lr=wl.lr,
                  momentum=wl.momentum, weight_decay=wl.weight_decay)
    print(f"[case] owner plan {method} {ns_dtype} owners={n_owners} matrices={len(shapes)}", flush=True)
    whole = run_step(nss, params, grads, mom, tab, h)

    assign, owners = nss.plan_owners([(r, c, s, l) for (r, c, s), l in zip(shapes, layers)],
                                     n_owners, method)
    covered = []
    for o, info in enumerate(owners):
        if info["n_matrices"] == 0:
            continue
        idx, otab = info["index"], info["table"]
        assert all(off + r * c <= info["numel"] for off, r, c, *_ in otab)
        covered += idx
        print(f"[owner {o}] {len(idx)} matrices, {info['numel']} elements, "
              f"{info['ns_flops'] / 1e12:.2f} TFLOP", flush=True)
        sl = [slice(tab[i][0], tab[i][0] + tab[i][1] * tab[i][2]) for i in idx]
        # per-matrix device tensors, packed into the owner's buffers
        p_src = [to_device(params[s].copy(), dev, torch) for s in sl]
        g_src = [to_device(grads[s].copy(), dev, torch) for s in sl]
        m_src = [to_device(mom[s].copy(), dev, torch) for s in sl]
        P = torch.zeros(info["numel"], dtype=torch.float32, device=dev)
        G = torch.zeros(info["numel"], dtype=torch.bfloat16, device=dev)
        M = torch.zeros(info["numel"], dtype=torch.float32, device=dev)
        U = torch.zeros(info["numel"], dtype=torch.float32, device=dev)
        nss.pack(P, p_src, otab)
        nss.pack(G, g_src, otab)
        nss.pack(M, m_src, otab)
        nss.step(P, G, M, otab, h, update_out=U)
        u_out = [torch.empty_like(t) for t in p_src]
        nss.unpack(p_src, P, otab)
        nss.unpack(m_src, M, otab)
        nss.unpack(u_out, U, otab)
        torch.cuda.synchronize()
        for k, s in enumerate(sl):
            assert np.array_equal(p_src[k].cpu().numpy(), whole["params"][s]), (o, idx[k])
            assert np.array_equal(m_src[k].cpu().numpy(), whole["momentum"][s]), (o, idx[k])
            assert np.array_equal(u_out[k].cpu().numpy(), whole["update"][s]), (o, idx[k])
    assert sorted(covered) == list(range(len(shapes)))
