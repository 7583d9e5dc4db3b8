"""GPU: the library's runtime services, through the C ABI.

- Plan cache (host layouts): a step after muon_release_plans() rebuilds the
  table's layout and gives the same bits; many distinct tables each get their
  own.
- Profiling hooks: between muon_profile_begin() and muon_profile_end() every
  launch is counted under its kind; the counts are the launch sequence of the
  method (which bench.py's per-kernel times rely on).
- Threads: two host threads stepping different tables on their own streams
  give the same bits as the same steps run one after the other.
- No synchronisation: the first call ever made with a table returns while a
  long step queued earlier on another stream is still running.
- Graphs: every call is kernel launches only, so even the first call with a
  table can be captured into a HIP graph; every replay (with eager work and
  synchronisation between replays, and after the host cache has been
  overflowed and dropped) equals an eager step from the same state.
"""
import threading

import numpy as np
import pytest

import workloads as W
from gpu_helpers import to_device

pytestmark = pytest.mark.gpu


def _inputs(shapes, wid, grad_dtype="bf16"):
    wl = W.custom_workload(shapes, grad_dtype=grad_dtype, wid=wid)
    params, grads, mom = W.host_inputs(wl)
    return wl, params, grads, mom


def _step(nss, wl, params, grads, mom, h, stream=None):
    import torch
    p, g, m = (to_device(a.copy(), "cuda:0", torch) for a in (params, grads, mom))
    nss.step(p, g, m, wl.table(), h, stream=stream)
    return p, m


def _hyper(nss, wl, method="standard", ns_dtype="bf16"):
    return nss.hyper(ns_method=method, ns_dtype=ns_dtype, grad_dtype=wl.grad_dtype, lr=wl.lr,
                     momentum=wl.momentum, weight_decay=wl.weight_decay)


def test_release_plans_and_many_tables(lib):
    import torch
    nss = lib
    wl, params, grads, mom = _inputs([(256, 384, 0), (384, 256, 0), (128, 640, 0)], wid=130)
    h = _hyper(nss, wl)
    p1, m1 = _step(nss, wl, params, grads, mom, h)
    torch.cuda.synchronize()
    nss.release_plans()
    p2, m2 = _step(nss, wl, params, grads, mom, h)
    torch.cuda.synchronize()
    assert torch.equal(p1, p2) and torch.equal(m1, m2)
    # 40 distinct tables (different shapes), then the first again
    for k in range(40):
        wk, pk, gk, mk = _inputs([(64 + 8 * k, 96, 0), (32, 40 + 8 * k, 0)], wid=131 + k)
        _step(nss, wk, pk, gk, mk, _hyper(nss, wk))
    p3, m3 = _step(nss, wl, params, grads, mom, h)
    torch.cuda.synchronize()
    assert torch.equal(p1, p3) and torch.equal(m1, m3)


@pytest.mark.parametrize("method,ns_dtype,shapes,want", [
    # one 128-tile group (m >= 129): the separate launches
    ("standard", "bf16", [(256, 384, 0)],
     {"expand_desc": 1, "momentum_sumsq": 1, "finalize_norm": 1, "prep_x0": 1, "ns_gemm_xxt": 5, "ns_gemm_poly": 5,
      "ns_gemm_update": 4, "ns_gemm_apply": 1}),
    # one single-row group (m <= 128, 16-bit): X0 + Gram and update + Gram in one pass each
    ("standard", "bf16", [(128, 640, 0)],
     {"expand_desc": 1, "momentum_sumsq": 1, "finalize_norm": 1, "prep_gram": 1, "ns_gemm_poly": 5,
      "ns_update_gram": 4, "ns_gemm_apply": 1}),
    ("gram", "f16", [(256, 384, 0)],
     {"expand_desc": 1, "momentum_sumsq": 1, "finalize_norm": 1, "prep_x0": 1, "gram_gemm_sym": 14, "gram_gemm_full": 4,
      "gram_gemm_apply": 1}),
    ("gram", "f16", [(128, 640, 0)],
     {"expand_desc": 1, "momentum_sumsq": 1, "finalize_norm": 1, "prep_gram": 1, "gram_chain": 1,
      "gram_gemm_apply": 1}),
])
def test_profile_counts_the_launch_sequence(lib, method, ns_dtype, shapes, want):
    import torch
    nss = lib
    wl, params, grads, mom = _inputs(shapes, wid=175)
    h = _hyper(nss, wl, method, ns_dtype)
    _step(nss, wl, params, grads, mom, h)          # plan built outside the profile
    torch.cuda.synchronize()
    nss.profile_begin()
    _step(nss, wl, params, grads, mom, h)
    got = nss.profile_end()
    assert {k: v[0] for k, v in got.items()} == want
    assert all(ms > 0 for _, ms in got.values())


def test_two_threads_two_streams(lib):
    import torch
    nss = lib
    cases = [_inputs([(512, 768, 0), (96, 700, 32)], wid=176), _inputs([(384, 1024, 0), (128, 128, 0)], wid=177)]
    hs = [_hyper(nss, c[0]) for c in cases]
    want = []
    for c, h in zip(cases, hs):
        p, m = _step(nss, *c, h)
        torch.cuda.synchronize()
        want.append((p.cpu(), m.cpu()))
    for _ in range(3):
        got = [None, None]
        errors = []

        def run(k):
            try:
                s = torch.cuda.Stream()
                with torch.cuda.stream(s):
                    p, m = _step(nss, *cases[k], hs[k], stream=s)
                s.synchronize()
                got[k] = (p.cpu(), m.cpu())
            except Exception as e:          # surfaced in the main thread
                errors.append(e)

        threads = [threading.Thread(target=run, args=(k,)) for k in range(2)]
        for t in threads:
            t.start()
        for t in threads:
            t.join()
        assert not errors, errors
        for k in range(2):
            assert torch.equal(got[k][0], want[k][0]) and torch.equal(got[k][1], want[k][1]), k


def _overflow_plan_cache(nss, n=1030):
    """More distinct tables than the host cache holds (1024), each stepped once on
    a tiny buffer; then the cache is dropped."""
    import torch
    dev = "cuda:0"
    p = torch.zeros(4096, device=dev)
    g = torch.zeros(4096, dtype=torch.bfloat16, device=dev)
    m = torch.zeros(4096, device=dev)
    h = nss.hyper(ns_method="standard", ns_dtype="bf16", grad_dtype="bf16")
    tables = [[(8 * (k % 64), 1 + k // 64, 8 + 8 * (k % 7), 0)] for k in range(n)]
    assert len({tuple(t[0]) for t in tables}) == n and all(o + r * c <= 4096 for (o, r, c, _), in tables)
    ws = torch.empty(max(nss.workspace_size(t, h) for t in tables), dtype=torch.uint8, device=dev)
    for t in tables:
        nss.step(p, g, m, t, h, ws=ws)
    nss.release_plans()


@pytest.mark.parametrize("method,ns_dtype", [("standard", "bf16"), ("gram", "f16"), ("standard", "f32")])
def test_graph_capture_and_replay(lib, method, ns_dtype):
    # every call is kernel launches only (the descriptors are written into the
    # workspace on the stream), so the first call ever made with a table can be
    # captured into a HIP graph; each replay is one more step and must equal an
    # eager step from the same state, also after the host cache was overflowed
    import torch
    nss = lib
    gdt = "f32" if ns_dtype == "f32" else "bf16"
    # a shape set no other test uses, so the captured call is this table's first
    wl, params, grads, mom = _inputs([(264, 392, 0), (128, 648, 0), (304, 136, 0)], wid=178, grad_dtype=gdt)
    h = nss.hyper(ns_method=method, ns_dtype=ns_dtype, grad_dtype=gdt, lr=wl.lr, momentum=wl.momentum,
                  weight_decay=wl.weight_decay)
    tab = wl.table()
    dev = "cuda:0"
    nss.release_plans()
    p, g, m = (to_device(a.copy(), dev, torch) for a in (params, grads, mom))
    pe, ge, me = (to_device(a.copy(), dev, torch) for a in (params, grads, mom))
    ws = torch.empty(nss.workspace_size(tab, h), dtype=torch.uint8, device=dev)
    ws_e = torch.empty_like(ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=s):
        nss.step(p, g, m, tab, h, ws=ws, stream=s)
    torch.cuda.synchronize()
    for r in range(5):
        graph.replay()
        torch.cuda.synchronize()
        nss.step(pe, ge, me, tab, h, ws=ws_e)     # the same step, eager
        torch.cuda.synchronize()
        assert torch.equal(p, pe) and torch.equal(m, me), r
        # eager work on the graph's own buffers between replays
        g.mul_(1.0)
        torch.cuda.synchronize()
        if r == 2:
            _overflow_plan_cache(nss)
            torch.cuda.synchronize()


def test_first_call_does_not_synchronise(lib):
    # a long step queued on stream A; then the first call ever with a new table,
    # on stream B, must return while A's work is still running (no device or
    # host synchronisation inside the call), and its result must be right
    import torch
    nss = lib
    dev = "cuda:0"
    n_long = 8 * 4096 * 4096
    long_tab = [(k * 4096 * 4096, 4096, 4096, 0) for k in range(8)]
    hl = nss.hyper(ns_method="standard", ns_dtype="bf16", grad_dtype="bf16")
    pl = torch.randn(n_long, device=dev)
    gl = (torch.randn(n_long, device=dev) * 1e-3).to(torch.bfloat16)
    ml = torch.zeros(n_long, device=dev)
    wsl = torch.empty(nss.workspace_size(long_tab, hl), dtype=torch.uint8, device=dev)
    wl, params, grads, mom = _inputs([(200, 328, 0), (96, 520, 24)], wid=179)
    h = _hyper(nss, wl)
    tab = wl.table()
    p, g, m = (to_device(a.copy(), dev, torch) for a in (params, grads, mom))
    ws = torch.empty(nss.workspace_size(tab, h), dtype=torch.uint8, device=dev)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    done = torch.cuda.Event()
    torch.cuda.synchronize()
    nss.release_plans()
    for _ in range(4):                               # about 50 ms of work on A
        nss.step(pl, gl, ml, long_tab, hl, ws=wsl, stream=sa)
    done.record(sa)
    nss.step(p, g, m, tab, h, ws=ws, stream=sb)      # first call with this table
    still_running = not done.query()
    torch.cuda.synchronize()
    assert still_running, "the call waited for work queued on another stream"
    pr, gr, mr = (to_device(a.copy(), dev, torch) for a in (params, grads, mom))
    nss.step(pr, gr, mr, tab, h, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(p, pr) and torch.equal(m, mr)
