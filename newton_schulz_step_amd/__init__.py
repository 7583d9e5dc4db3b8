"""Muon optimizer step on one AMD Instinct MI355X (gfx950).

libmuonstep (C ABI, include/muon_step.h) runs one Muon step over an owner's
packed buffer of 2D matrices: momentum, Frobenius-normalised Newton-Schulz
orthogonalisation ("standard" quintic or "gram"), decoupled weight decay and
the lr-scaled update, plus the AdamW fallback. This package is its thin Python
binding; torch supplies device memory and streams.
"""
from ._binding import (  # noqa: F401
    DTYPES, EXPORTED, LIB_PATH, NS_METHODS, STATUS_NAMES, AdamWHyper, KernelStat, MuonError,
    MuonAssign, MuonHyper, MuonMatrix, MuonOwner, MuonParam, MuonWindow, adamw, comm_elements,
    hyper, load, ns_flops, pack, plan_owners, profile_begin, profile_end, release_plans, step,
    step_noalloc, step_window, table, unpack, version, windows, workspace, workspace_size)
from ._binding import NOALLOC_WORKSPACE_BYTES  # noqa: F401
from ._binding import (  # noqa: F401
    ERR_ALIGN, ERR_BAD_HYPER, ERR_BAD_METHOD, ERR_BAD_SHAPE, ERR_HIP, ERR_NULL, ERR_OVERLAP,
    ERR_RANGE, ERR_UNSUPPORTED, ERR_WORKSPACE, OK)
