"""Shared helpers of the GPU parity tests (they run the C ABI through the binding)."""
import numpy as np

import oracle
import workloads as W


def rel(x, y):
    d = np.linalg.norm(y)
    return float(np.linalg.norm(x - y) / (d if d > 0 else 1.0))


def to_device(arr, dev, torch):
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(dev)


def run_step(nss, params, grads, mom, tab, h, shadow=False, dev="cuda:0", steps=1):
    """`steps` muon_step calls on device copies of the host buffers; numpy results."""
    import torch
    p = to_device(params, dev, torch)
    g = to_device(grads, dev, torch)
    m = to_device(mom, dev, torch)
    upd = torch.zeros_like(p)
    sh = torch.zeros(p.numel(), dtype=torch.int16, device=dev) if shadow else None
    for _ in range(steps):
        nss.step(p, g, m, tab, h, update_out=upd, bf16_shadow=sh)
    torch.cuda.synchronize()
    out = {"params": p.cpu().numpy(), "momentum": m.cpu().numpy(), "update": upd.cpu().numpy()}
    if shadow:
        out["shadow"] = sh.cpu().numpy().view(np.uint16)
    return out


def block_grid(e):
    """(first row, rows, first column, cols) of each independent block of a
    workload entry: split_rows x split_cols tiles (0 = the whole side)."""
    pr = e.split_rows or e.rows
    pc = e.split_cols or e.cols
    return [(r, pr, c, pc) for r in range(0, e.rows, pr) for c in range(0, e.cols, pc)]


def entry_slices(tab):
    return [slice(o, o + r * c) for o, r, c, *_ in tab]


def outside_mask(tab, n):
    mask = np.ones(n, bool)
    for s in entry_slices(tab):
        mask[s] = False
    return mask


def grads_f64(wl, grads):
    return W.grad_as_f64(wl, grads)


def top_left_singular_vectors(M, k=16):
    if min(M.shape) <= 512:
        return np.linalg.svd(M, full_matrices=False)[0][:, :k]
    from scipy.sparse.linalg import svds
    U, s, _ = svds(M, k=k, v0=np.ones(min(M.shape)))
    return U[:, np.argsort(s)[::-1]]


def top_subspace_err(O, O_ref, M, k=16):
    """||U_k^T (O - O_ref)|| / ||U_k^T O_ref||, U_k = top-k left singular vectors of M."""
    U = top_left_singular_vectors(M, k)
    return rel(U.T @ O, U.T @ O_ref)


def oracle_entry(wl, i, g, p, method, store_fmt, steps=1):
    """Oracle step(s) of one entry alone (float64 results, shaped rows x cols)."""
    e = wl.entries[i]
    n = e.rows * e.cols
    tab = [(0, e.rows, e.cols, e.split_rows)]
    gg = W.grad_as_f64(wl, np.asarray(g).ravel())
    P = np.asarray(p, np.float64).ravel()
    M = np.zeros(n)
    for _ in range(steps):
        out = oracle.muon_step(P, gg, M, tab, lr=wl.lr, mu=wl.momentum,
                               weight_decay=wl.weight_decay, method=method, store_fmt=store_fmt)
        P, M = out["params"], out["momentum"]
    shp = (e.rows, e.cols)
    return {k: v.reshape(shp) for k, v in out.items()}
