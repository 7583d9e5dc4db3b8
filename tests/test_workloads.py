"""The seeded synthetic inputs: shapes, packing and value recipe."""
import numpy as np

import workloads as W


def test_element_counts():
    expect = {1: 294_912, 2: 51_380_224, 3: 809_500_672, 4: 553_648_128, 5: 2_147_483_648}
    for wid, n in expect.items():
        wl = W.workload(wid)
        assert wl.muon_elements == n
        offs = wl.offsets
        assert all(o % W.PACK_ALIGN == 0 for o in offs)
        ends = [o + e.rows * e.cols for o, e in zip(offs, wl.entries)]
        assert all(ends[i] <= offs[i + 1] for i in range(len(offs) - 1))
    assert sum(W.workload(5).adamw_sizes) == 131_338_240


def test_split_entries_divide():
    for e in W.workload(5).entries:
        assert e.split_rows == 128 and e.rows % e.split_rows == 0


def test_values_deterministic_and_seeded_per_entry():
    wl = W.workload(1)
    g0, p0 = W.entry_values(wl, 2)
    g1, p1 = W.entry_values(wl, 2)
    assert np.array_equal(g0, g1) and np.array_equal(p0, p1)
    g2, _ = W.entry_values(wl, 3)
    assert not np.array_equal(g0, g2)


def test_bf16_encoding_roundtrip():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(10000).astype(np.float32)
    b = W.f32_to_bf16_bits(x)
    y = W.bf16_bits_to_f32(b)
    assert np.all(np.abs(y - x) <= np.abs(x) * 2.0 ** -8)
    assert np.array_equal(W.f32_to_bf16_bits(y), b)


def test_low_rank_gradient_is_ill_conditioned():
    wl = W.custom_workload([(256, 512, 0)])
    g, _ = W.entry_values(wl, 0)
    s = np.linalg.svd(W.grad_as_f64(wl, g), compute_uv=False)
    s = s / np.sqrt(np.sum(s ** 2))
    assert s[0] > 0.1 and s[16] < 3e-2 and s[0] / s[16] > 20
