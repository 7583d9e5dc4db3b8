"""The C ABI without a GPU: the library loads, exports what include/muon_step.h
declares, and rejects bad arguments before it touches the device.

Every check in muon_step, adamw_step, muon_pack and muon_unpack runs before
the first HIP call, so these tests pass fake (never dereferenced) device
addresses and only look at the returned status and message.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import newton_schulz_step_amd as nss

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon_step.h")

FAKE = 0x7f0000000000          # a 256-byte aligned address that is never dereferenced


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return nss.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert "muon_step" in names and "adamw_step" in names and "muon_pack" in names
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(nss.EXPORTED)


def test_defaults_match_article(lib):
    h = nss.hyper()
    assert abs(h.lr - 0.02) < 1e-9 and abs(h.momentum - 0.95) < 1e-7
    assert (round(h.ns_a, 4), round(h.ns_b, 4), round(h.ns_c, 4)) == (3.4445, -4.775, 2.0315)
    assert h.ns_steps == 5 and h.ns_method == nss.NS_METHODS["gram"]
    assert abs(h.ns_eps - 1e-7) < 1e-12
    # muon_lr overrides lr, as in the DeepSpeed config
    assert abs(nss.hyper(lr=0.5, muon_lr=0.1).lr - 0.1) < 1e-7
    with pytest.raises(TypeError):
        nss.hyper(no_such_key=1)


def _status(fn):
    try:
        fn()
    except nss.MuonError as e:
        return e.status, e.message
    return nss.OK, ""


def _ws(entries, **kw):
    return _status(lambda: nss.workspace_size(entries, nss.hyper(**kw)))


def test_workspace_size_validation(lib):
    assert _ws([(0, 4, 4, 0)], ns_method="standard")[0] == nss.OK
    assert _ws([(0, 4, 4, 0)], ns_method=7)[0] == nss.ERR_BAD_METHOD
    assert _ws([(0, 4, 4, 0)], ns_method="newton")[0] == nss.ERR_BAD_METHOD
    assert _ws([(0, 0, 4, 0)])[0] == nss.ERR_BAD_SHAPE
    assert _ws([(0, 4, -1, 0)])[0] == nss.ERR_BAD_SHAPE
    assert _ws([(0, 12, 4, 5)])[0] == nss.ERR_BAD_SHAPE          # split does not divide rows
    assert _ws([(0, 12, 4, -2)])[0] == nss.ERR_BAD_SHAPE
    assert _ws([(0, 4, 12, 0, 5)])[0] == nss.ERR_BAD_SHAPE       # split_cols does not divide cols
    assert _ws([(0, 4, 12, 0, -3)])[0] == nss.ERR_BAD_SHAPE
    assert _ws([(0, 4, 12, 0, 13)])[0] == nss.ERR_BAD_SHAPE
    assert _ws([(0, 8, 12, 4, 6)])[0] == nss.OK                  # a grid of 4 x 6 tiles
    assert _ws([(0, 2, (1 << 24) + 8, 0, 8)])[0] == nss.ERR_BAD_SHAPE   # row pitch beyond the long side
    assert _ws([(0, 20000, 20000, 0)])[0] == nss.ERR_BAD_SHAPE   # short side beyond the limit
    assert _ws([(-8, 4, 4, 0)])[0] == nss.ERR_RANGE
    assert _ws([(4, 4, 4, 0)])[0] == nss.ERR_ALIGN
    assert _ws([(0, 4, 4, 0), (8, 4, 4, 0)])[0] == nss.ERR_OVERLAP
    assert _ws([(0, 4, 4, 0)], ns_method="gram", ns_dtype="bf16")[0] == nss.ERR_UNSUPPORTED
    assert _ws([(0, 4, 4, 0)], param_dtype=1)[0] == nss.OK            # bf16 params
    assert _ws([(0, 4, 4, 0)], param_dtype=2)[0] == nss.ERR_UNSUPPORTED
    assert _ws([(0, 4, 4, 0)], ns_steps=0)[0] == nss.ERR_BAD_HYPER
    assert _ws([(0, 4, 4, 0)], lr=float("nan"))[0] == nss.ERR_BAD_HYPER
    st, msg = _ws([(0, 4, 4, 0)], ns_method=7)
    assert "standard" in msg and "gram" in msg


def test_column_split_layout(lib):
    # a 4096 x 4096 matrix split into 32 column blocks has the same problems
    # (32 of canonical shape 128 x 4096) as the same matrix split by rows, so
    # the same workspace; a grid has one problem per tile
    for method, dt in (("standard", "bf16"), ("gram", "f16")):
        kw = dict(ns_method=method, ns_dtype=dt)
        by_rows = nss.workspace_size([(0, 4096, 4096, 128)], nss.hyper(**kw))
        by_cols = nss.workspace_size([(0, 4096, 4096, 0, 128)], nss.hyper(**kw))
        assert by_rows == by_cols
        grid = nss.workspace_size([(0, 512, 768, 256, 384)], nss.hyper(**kw))
        tiles = nss.workspace_size([(i * 256 * 384, 256, 384, 0) for i in range(4)], nss.hyper(**kw))
        assert grid == tiles
    # the problem limit counts column blocks too
    st, msg = _ws([(0, 1 << 13, 1 << 12, 1, 1)])
    assert st == nss.ERR_BAD_SHAPE and "MUON_MAX_PROBLEMS" in msg


def test_table_wide_limits(lib):
    # MUON_MAX_TABLE_ELEMENTS (2^36) over the whole table, MUON_MAX_PROBLEMS
    # (2^24) expanded problems, and offsets that cannot overflow offset + size
    lim = 1 << 36
    assert _ws([(0, 1 << 12, 1 << 24, 1 << 8)])[0] == nss.OK                 # exactly 2^36
    assert _ws([(0, 1 << 12, 1 << 24, 1 << 8), (1 << 36, 1, 8, 0)])[0] == nss.ERR_BAD_SHAPE
    assert _ws([(0, (1 << 40) + 8, 1 << 24, 8)])[0] == nss.ERR_BAD_SHAPE     # product would overflow
    st, msg = _ws([(0, (1 << 24) + 1, 1, 1)])                                # one problem too many
    assert st == nss.ERR_BAD_SHAPE and "MUON_MAX_PROBLEMS" in msg
    assert _ws([((1 << 63) - 8, 1, 8, 0)])[0] == nss.ERR_RANGE
    assert _ws([(lim, 1, 8, 0)])[0] == nss.OK


def test_workspace_grows_with_the_table(lib):
    h = nss.hyper(ns_method="standard", ns_dtype="bf16")
    small = nss.workspace_size([(0, 128, 128, 0)], h)
    big = nss.workspace_size([(0, 128, 128, 0), (16384, 512, 128, 0)], h)
    assert 0 < small < big
    assert nss.workspace_size([], h) > 0


def _raw_step(lib, entries, numel, h, params=FAKE, grads=FAKE + (1 << 36), mom=FAKE + (2 << 36),
              ws=FAKE + (3 << 36), ws_bytes=1 << 40, upd=None, shadow=None):
    arr, n = nss.table(entries)
    st = lib.muon_step(params, grads, mom, numel, arr, n, ctypes.byref(h), ws, ws_bytes,
                       upd, shadow, None)
    return st, lib.muon_last_error().decode()


def test_step_rejects_before_any_device_work(lib):
    h = nss.hyper(ns_method="standard", ns_dtype="bf16")
    ent = [(0, 64, 64, 0)]
    assert _raw_step(lib, ent, 4096, h, params=None)[0] == nss.ERR_NULL
    assert _raw_step(lib, ent, 4095, h)[0] == nss.ERR_RANGE
    assert _raw_step(lib, ent, 4096, h, params=FAKE + 8)[0] == nss.ERR_ALIGN
    assert _raw_step(lib, ent, 4096, h, ws=FAKE + (3 << 36) + 16)[0] == nss.ERR_ALIGN
    assert _raw_step(lib, ent, 4096, h, mom=FAKE + 1024)[0] == nss.ERR_OVERLAP
    assert _raw_step(lib, ent, 4096, h, upd=FAKE + (1 << 36))[0] == nss.ERR_OVERLAP
    assert _raw_step(lib, ent, 4096, h, ws=None)[0] == nss.ERR_NULL
    bad = nss.hyper(ns_method=3)
    assert _raw_step(lib, ent, 4096, bad)[0] == nss.ERR_BAD_METHOD
    # an empty table is a no-op that succeeds without touching the device
    assert _raw_step(lib, [], 4096, h)[0] == nss.OK
    st, msg = _raw_step(lib, [(0, 64, 64, 0), (64 * 64, 8, 8, 0)], 4096, h)
    assert st == nss.ERR_RANGE and "entry 1" in msg


def test_bf16_params_checks(lib):
    # bf16 params take 2 bytes per element; they are their own bf16 copy, so a
    # shadow is refused, and partition holders take float32 partitions only
    h = nss.hyper(ns_method="standard", ns_dtype="bf16", param_dtype="bf16")
    ent = [(0, 64, 64, 0)]
    assert _raw_step(lib, ent, 4096, h, shadow=FAKE + (5 << 36))[0] == nss.ERR_UNSUPPORTED
    assert _raw_step(lib, ent, 4096, h, mom=FAKE + 4096 * 2 - 16)[0] == nss.ERR_OVERLAP
    assert _raw_step(lib, ent, 4096, h, mom=FAKE + 4096 * 2, ws=None)[0] == nss.ERR_NULL
    arr, n = nss.table(ent)
    warr = nss.windows([(0, 16, 0)], n)
    st = lib.muon_step_window(FAKE, 16, FAKE + (1 << 36), FAKE + (2 << 36), 4096, arr, warr, n,
                              ctypes.byref(h), FAKE + (3 << 36), 1 << 40, None, None, None)
    assert st == nss.ERR_UNSUPPORTED


def test_noalloc_refuses_before_any_device_work(lib):
    # a table whose workspace exceeds the library's array is refused on the host
    h = nss.hyper(ns_method="standard", ns_dtype="bf16")
    ent = [(0, 4096, 4096, 0)]
    assert nss.workspace_size(ent, h) > nss.NOALLOC_WORKSPACE_BYTES
    arr, n = nss.table(ent)
    st = lib.muon_step_noalloc(FAKE, FAKE + (1 << 36), FAKE + (2 << 36), 4096 * 4096, arr, n,
                               ctypes.byref(h), None, None, None)
    assert st == nss.ERR_WORKSPACE and "muon_step_noalloc" in lib.muon_last_error().decode()
    arr, n = nss.table([(0, 64, 64, 0)])
    st = lib.muon_step_noalloc(FAKE, FAKE + (1 << 36), FAKE + (2 << 36), 4095, arr, n,
                               ctypes.byref(h), None, None, None)
    assert st == nss.ERR_RANGE


def _raw_window(lib, entries, wins, numel, pnumel, h, part=FAKE + (4 << 36), grads=FAKE + (1 << 36),
                mom=FAKE + (2 << 36), ws=FAKE + (3 << 36), upd=None, shadow=None, null_windows=False):
    arr, n = nss.table(entries)
    warr = None if null_windows else nss.windows(wins, n)
    st = lib.muon_step_window(part, pnumel, grads, mom, numel, arr, warr, n, ctypes.byref(h), ws,
                              1 << 40, upd, shadow, None)
    return st, lib.muon_last_error().decode()


def test_step_window_rejects_before_any_device_work(lib):
    h = nss.hyper(ns_method="standard", ns_dtype="bf16")
    ent = [(0, 64, 64, 0), (4096, 32, 64, 0)]
    ok_w = [(1000, 4096, 0), (0, 100, 3096)]
    # a matrix straddling both ends of the partition, another starting inside it
    assert _raw_window(lib, ent, ok_w, 6144, 4096, h, null_windows=True)[0] == nss.ERR_NULL
    assert _raw_window(lib, ent, ok_w, 6144, 4096, h, part=None)[0] == nss.ERR_NULL
    assert _raw_window(lib, ent, [(10, 5, 0), (0, 0, 0)], 6144, 4096, h)[0] == nss.ERR_RANGE
    assert _raw_window(lib, ent, [(-1, 5, 0), (0, 0, 0)], 6144, 4096, h)[0] == nss.ERR_RANGE
    assert _raw_window(lib, ent, [(0, 4097, 0), (0, 0, 0)], 6144, 8192, h)[0] == nss.ERR_RANGE
    st, msg = _raw_window(lib, ent, [(0, 4096, 1), (0, 0, 0)], 6144, 4096, h)
    assert st == nss.ERR_RANGE and "window 0" in msg
    assert _raw_window(lib, ent, [(0, 4096, -8), (0, 0, 0)], 6144, 8192, h)[0] == nss.ERR_RANGE
    st, msg = _raw_window(lib, ent, [(0, 64, 0), (0, 64, 63)], 6144, 4096, h)
    assert st == nss.ERR_OVERLAP and "windows overlap" in msg
    # adjacent windows and empty windows anywhere are fine as far as validation goes
    assert _raw_window(lib, ent, [(0, 64, 0), (0, 64, 64)], 6144, 128, h, ws=None)[0] == nss.ERR_NULL
    assert _raw_window(lib, ent, [(7, 7, 0), (0, 0, 99)], 6144, 0, h, ws=None)[0] == nss.ERR_NULL
    # the partition and the shadow are sized by partition_numel
    assert _raw_window(lib, ent, ok_w, 6144, 4096, h, part=FAKE + (2 << 36) - 4096)[0] == nss.ERR_OVERLAP
    st = _raw_window(lib, ent, ok_w, 6144, 4096, h, shadow=FAKE + (4 << 36) + 4096 * 4 - 16)[0]
    assert st == nss.ERR_OVERLAP
    assert _raw_window(lib, ent, ok_w, 6144, 4096, h, upd=FAKE + (4 << 36) - 6144 * 4 + 16)[0] == nss.ERR_OVERLAP
    assert _raw_window(lib, ent, ok_w, 6143, 4096, h)[0] == nss.ERR_RANGE
    assert _raw_window(lib, [(0, 64, 64, 0)], [(0, 1, 0)], 4096, 4096, h, part=FAKE + (4 << 36) + 8)[0] == nss.ERR_ALIGN


def test_adamw_rejects_before_any_device_work(lib):
    h = nss.AdamWHyper()
    lib.muon_default_adamw_hyper(ctypes.byref(h))
    assert abs(h.lr - 3e-4) < 1e-10 and abs(h.beta1 - 0.9) < 1e-7 and abs(h.beta2 - 0.95) < 1e-7
    a, b, c, d = FAKE, FAKE + (1 << 36), FAKE + (2 << 36), FAKE + (3 << 36)
    assert lib.adamw_step(a, b, c, d, 1000, None, None) == nss.ERR_NULL
    h.step = 0
    assert lib.adamw_step(a, b, c, d, 1000, ctypes.byref(h), None) == nss.ERR_BAD_HYPER
    h.step = 1
    h.beta1 = 1.0
    assert lib.adamw_step(a, b, c, d, 1000, ctypes.byref(h), None) == nss.ERR_BAD_HYPER
    h.beta1 = 0.9
    assert lib.adamw_step(a, b, c + 4, d, 1000, ctypes.byref(h), None) == nss.ERR_ALIGN
    assert lib.adamw_step(a, b, a + 64, d, 1000, ctypes.byref(h), None) == nss.ERR_OVERLAP
    assert lib.adamw_step(a, b, c, d, 0, ctypes.byref(h), None) == nss.OK
    h.grad_dtype = 9
    assert lib.adamw_step(a, b, c, d, 1000, ctypes.byref(h), None) == nss.ERR_UNSUPPORTED


def test_pack_rejects_before_any_device_work(lib):
    arr, n = nss.table([(0, 4, 4, 0), (16, 4, 4, 0)])
    srcs = (ctypes.c_void_p * 2)(FAKE, FAKE + 4096)
    assert lib.muon_pack(FAKE + (1 << 36), 31, srcs, arr, n, 0, None) == nss.ERR_RANGE
    assert lib.muon_pack(FAKE + (1 << 36), 32, srcs, arr, n, 5, None) == nss.ERR_UNSUPPORTED
    srcs_null = (ctypes.c_void_p * 2)(FAKE, None)
    assert lib.muon_pack(FAKE + (1 << 36), 32, srcs_null, arr, n, 0, None) == nss.ERR_NULL
    arr2, n2 = nss.table([(0, 4, 4, 0), (8, 4, 4, 0)])
    assert lib.muon_unpack(srcs, FAKE + (1 << 36), 32, arr2, n2, 1, None) == nss.ERR_OVERLAP


def test_product_path_fails_loudly_without_the_library(monkeypatch, tmp_path):
    from newton_schulz_step_amd import _binding
    monkeypatch.setattr(_binding, "_lib", None)
    monkeypatch.setattr(_binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        _binding.load()


def test_random_tables_get_the_status_of_their_one_violation(lib):
    # Seeded random tables: 1-6 entries of random shapes (some split into row
    # blocks), at 8-aligned offsets with gaps of at least 8 elements. Each table
    # gets at most one violation, and the returned status must be exactly that
    # violation's code; an untouched table must pass. Only rejected tables reach
    # muon_step (with fake pointers: every check runs before the first device
    # call); valid ones go through the host-only muon_workspace_size.
    rng = np.random.default_rng(77)
    h = nss.hyper(ns_method="standard", ns_dtype="bf16")
    kinds = ["none", "zero_rows", "bad_split", "misaligned", "duplicate", "short", "negative",
             "bad_col_split"]
    want = {"none": nss.OK, "zero_rows": nss.ERR_BAD_SHAPE, "bad_split": nss.ERR_BAD_SHAPE,
            "misaligned": nss.ERR_ALIGN, "duplicate": nss.ERR_OVERLAP, "short": nss.ERR_RANGE,
            "negative": nss.ERR_RANGE, "bad_col_split": nss.ERR_BAD_SHAPE}
    for case in range(640):
        ents, cur = [], 0
        for _ in range(int(rng.integers(1, 7))):
            r, c = int(rng.integers(1, 300)), int(rng.integers(1, 300))
            divs = [d for d in range(1, r + 1) if r % d == 0]
            cdivs = [d for d in range(1, c + 1) if c % d == 0]
            split = int(rng.choice(divs)) if rng.random() < 0.3 else 0
            csplit = int(rng.choice(cdivs)) if rng.random() < 0.3 else 0
            cur += 8 * int(rng.integers(1, 4))
            ents.append([cur, r, c, split, csplit])
            cur = (cur + r * c + 7) // 8 * 8
        numel = cur + 8 * int(rng.integers(1, 4))
        kind = kinds[case % len(kinds)]
        k = int(rng.integers(len(ents)))
        if kind == "zero_rows":
            ents[k][1], ents[k][3] = 0, 0
        elif kind == "bad_col_split":
            ents[k][4] = ents[k][2] + 1 if rng.random() < 0.5 else -1
        elif kind == "bad_split":
            ents[k][3] = ents[k][1] + 1
        elif kind == "misaligned":
            ents[k][0] += 4
        elif kind == "duplicate":
            ents.append(list(ents[k]))
        elif kind == "short":
            numel = ents[-1][0] + ents[-1][1] * ents[-1][2] - 1
        elif kind == "negative":
            ents[0][0] = -8
        table = [tuple(e) for e in ents]
        if kind != "short":          # the table alone decides
            st, msg = _status(lambda: nss.workspace_size(table, h))
            assert st == want[kind], (case, kind, ents, st, msg)
        if kind != "none":           # never a valid table with fake pointers
            st, msg = _raw_step(lib, table, numel, h)
            assert st == want[kind], (case, kind, ents, numel, st, msg)
