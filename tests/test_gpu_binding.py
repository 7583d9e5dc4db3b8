"""GPU: the Python binding's own duties (argument checks, device and stream
handling), through the C ABI.

- Steps enqueued on two streams at once, each with the binding's cached
  workspace, give the same bits as the same steps run one after the other:
  the cache keeps one workspace per (device, stream).
- pack / unpack refuse tensors whose dtype or size does not match the packed
  buffer and their table entry (the copy is sized from the table), before any
  device work.
- Tensors on different devices (here: GPU and host) are refused.
"""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import to_device

pytestmark = pytest.mark.gpu


def test_two_streams_with_cached_workspaces(lib):
    import torch
    nss = lib
    dev = "cuda:0"
    shapes = [(512, 768, 0), (768, 512, 0), (1024, 256, 128), (300, 140, 0)]
    wl = W.custom_workload(shapes, grad_dtype="bf16", wid=120)
    params, grads, mom = W.host_inputs(wl)
    tab = wl.table()
    h = nss.hyper(ns_method="standard", ns_dtype="bf16", grad_dtype="bf16", lr=wl.lr,
                  momentum=wl.momentum, weight_decay=wl.weight_decay)
    g2 = (0.5 * W.grad_as_f64(wl, grads)).astype(np.float32)
    inputs = [grads, W.f32_to_bf16_bits(g2)]     # two gradient sets, bf16 bits

    def fresh(k):
        return (to_device(params.copy(), dev, torch), to_device(inputs[k].copy(), dev, torch),
                to_device(mom.copy(), dev, torch))

    # one after the other, on the current stream
    want = []
    for k in range(2):
        p, g, m = fresh(k)
        nss.step(p, g, m, tab, h)
        torch.cuda.synchronize()
        want.append((p.cpu().numpy(), m.cpu().numpy()))
    # both at once, two streams, no explicit workspace; a few rounds
    for _ in range(3):
        bufs = [fresh(k) for k in range(2)]
        torch.cuda.synchronize()
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        for k in range(2):
            p, g, m = bufs[k]
            nss.step(p, g, m, tab, h, stream=streams[k])
        torch.cuda.synchronize()
        for k in range(2):
            p, _, m = bufs[k]
            assert np.array_equal(p.cpu().numpy(), want[k][0]), k
            assert np.array_equal(m.cpu().numpy(), want[k][1]), k


def test_pack_refuses_mismatched_tensors(lib):
    import torch
    nss = lib
    dev = "cuda:0"
    tab = [(0, 4, 8, 0), (40, 2, 8, 0)]            # gap [32, 40), tail [56, 64)
    packed = torch.zeros(64, dtype=torch.float32, device=dev)
    good = [torch.ones(4, 8, device=dev), torch.ones(2, 8, device=dev)]
    with pytest.raises(ValueError):       # 16-bit tensor into an fp32 buffer
        nss.pack(packed, [good[0].to(torch.bfloat16), good[1]], tab)
    with pytest.raises(ValueError):       # too few elements for its entry
        nss.pack(packed, [good[0][:3], good[1]], tab)
    with pytest.raises(ValueError):       # one tensor for two entries
        nss.unpack([good[0]], packed, tab)
    torch.cuda.synchronize()
    assert not torch.any(packed)          # nothing was copied
    nss.pack(packed, good, tab)
    torch.cuda.synchronize()
    assert torch.equal(packed[:32], torch.ones(32, device=dev))
    assert torch.equal(packed[40:56], torch.ones(16, device=dev))
    assert not torch.any(packed[32:40]) and not torch.any(packed[56:])


def test_tensors_on_different_devices_are_refused(lib):
    import torch
    nss = lib
    p = torch.zeros(64, device="cuda:0")
    m = torch.zeros(64, device="cuda:0")
    g = torch.zeros(64, dtype=torch.bfloat16)      # host
    h = nss.hyper(ns_method="standard", ns_dtype="bf16", grad_dtype="bf16")
    with pytest.raises(ValueError):
        nss.step(p, g, m, [(0, 8, 8, 0)], h)
