"""GPU: muon_step_noalloc, the entry point that allocates nothing, against muon_step.

Both run the same kernels; the allocation-free one takes its workspace from the
library's per-GPU device array instead of the caller's buffer. On two calls in
a row, the second with a smaller table (the array then holds the first call's
leftovers), every output (params, momentum, update, bf16 shadow) must equal
muon_step's bit for bit, for the three iteration types. A table needing more
workspace than the array holds is refused before any device work.
"""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import to_device

pytestmark = pytest.mark.gpu

CALLS = [
    [(300, 200, 0), (130, 700, 0), (64, 2000, 0), (256, 96, 64), (9, 13, 0)],   # first call
    [(128, 512, 0), (40, 24, 0)],                                               # smaller second call
]


def _run(nss, fn, params, grads, mom, tab, h, **kw):
    import torch
    dev = "cuda:0"
    p, g, m = (to_device(a.copy(), dev, torch) for a in (params, grads, mom))
    u = torch.zeros_like(p)
    sh = torch.zeros(p.numel(), dtype=torch.int16, device=dev)
    fn(p, g, m, tab, h, update_out=u, bf16_shadow=sh, **kw)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (p, m, u, sh)]


@pytest.mark.parametrize("method,ns_dtype,gdt", [("standard", "bf16", "bf16"), ("gram", "f16", "bf16"),
                                                 ("standard", "f32", "f32")])
def test_noalloc_equals_muon_step(lib, method, ns_dtype, gdt):
    nss = lib
    for call, shapes in enumerate(CALLS):
        wl = W.custom_workload(shapes, grad_dtype=gdt, wid=190 + call)
        params, grads, mom = W.host_inputs(wl)
        tab = wl.table()
        h = nss.hyper(ns_method=method, ns_dtype=ns_dtype, grad_dtype=gdt, lr=wl.lr,
                      momentum=wl.momentum, weight_decay=wl.weight_decay)
        assert nss.workspace_size(tab, h) <= nss.NOALLOC_WORKSPACE_BYTES
        print(f"[case] noalloc call {call} {method} {ns_dtype}: {tab}", flush=True)
        want = _run(nss, nss.step, params, grads, mom, tab, h)
        got = _run(nss, nss.step_noalloc, params, grads, mom, tab, h)
        for name, x, y in zip(("params", "momentum", "update", "shadow"), got, want):
            assert np.array_equal(x, y), (call, name)
        assert not np.array_equal(got[0], params)          # the step did update the params


def test_noalloc_refuses_a_table_beyond_its_array(lib):
    import torch
    nss = lib
    dev = "cuda:0"
    tab = [(0, 4096, 4096, 0)]
    h = nss.hyper(ns_method="standard", ns_dtype="bf16", grad_dtype="bf16")
    assert nss.workspace_size(tab, h) > nss.NOALLOC_WORKSPACE_BYTES
    n = 4096 * 4096
    p = torch.randn(n, device=dev)
    g = torch.randn(n, device=dev).to(torch.bfloat16)
    m = torch.zeros(n, device=dev)
    p0 = p.clone()
    with pytest.raises(nss.MuonError) as ei:
        nss.step_noalloc(p, g, m, tab, h)
    assert ei.value.status == nss.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.equal(p, p0) and not torch.any(m)
