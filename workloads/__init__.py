"""Seeded synthetic inputs for the Muon step: shapes, packing offsets and values.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It holds no arithmetic of the method itself (no momentum, no
normalisation, no Newton-Schulz, no update rule): only the workload shapes,
the packed layout the caller hands to the step, and seeded random values.

Workloads (sizes as the configurations name them):
  1  tiny fp32 step: 2x128x128, 2x128x512, 2x512x128; params and grads N(0,1)
  2  one transformer layer, bf16 grads: q,k,v,o 2048x2048, gate/up 5632x2048,
     down 2048x5632
  3  an owner's packed buffer at 1/8 of a 7B-class model, bf16 grads:
     16x4096x4096, 8x11008x4096, 4x4096x11008
  4  MoE expert batch, bf16 grads: 64 x (gate 1408x2048, up 1408x2048,
     down 2048x1408)
  5  per-head split: 32 layers of q,k,v,o 4096x4096, each split into 32 row
     blocks of 128x4096; AdamW on a 32000x4096 embedding and 65 vectors of 4096

Gradient recipe for workloads 2-5 (a low-rank signal plus noise, matching the
high condition number that the DeepSpeed-Muon article ascribes to transformer
weight gradients, section on why orthogonalisation matters):
  G = (sigma / sqrt(r)) * U @ V.T + tau * E,  r = 16, sigma = 1e-3, tau = 1e-5,
  U (rows x r), V (cols x r), E (rows x cols) all iid N(0,1), drawn in that
  order, in float64, then stored as bf16 (float64 -> float32 -> bf16, each
  round-to-nearest-even). Params are N(0,1) float32, drawn after E. Momentum
  starts at zero. Workload 1 draws G then P, both N(0,1), stored float32.

Every entry has its own stream: numpy Generator(PCG64(SeedSequence([wid, i]))).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np

PACK_ALIGN = 64  # packed offsets are rounded up to a multiple of 64 elements


@dataclasses.dataclass(frozen=True)
class Entry:
    name: str
    rows: int
    cols: int
    split_rows: int = 0  # 0: whole matrix; k > 0: rows/k independent k-row blocks
    split_cols: int = 0  # k > 0: cols/k independent k-column blocks (with split_rows: tiles)


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    title: str
    entries: Tuple[Entry, ...]
    grad_dtype: str            # "f32" or "bf16"
    ns_dtype: str              # "f32" or "bf16" (standard); gram runs in "f16"
    lr: float = 0.02
    momentum: float = 0.95
    weight_decay: float = 0.1
    adamw_sizes: Tuple[int, ...] = ()   # element counts of the non-2D / AdamW tensors
    grad_kind: str = ""        # "gaussian" | "lowrank"; "" = gaussian for f32, lowrank otherwise

    @property
    def kind(self) -> str:
        if self.grad_kind:
            return self.grad_kind
        return "gaussian" if self.grad_dtype == "f32" else "lowrank"

    @property
    def offsets(self) -> List[int]:
        return packed_offsets(self.entries)

    @property
    def numel(self) -> int:
        offs = self.offsets
        if not self.entries:
            return 0
        last = self.entries[-1]
        return offs[-1] + last.rows * last.cols

    @property
    def muon_elements(self) -> int:
        return sum(e.rows * e.cols for e in self.entries)

    def table(self) -> List[Tuple[int, ...]]:
        """(offset, rows, cols, split_rows) per entry, in packing order, with
        split_cols as a fifth field for entries split by columns."""
        return [(o, e.rows, e.cols, e.split_rows) + ((e.split_cols,) if e.split_cols else ())
                for o, e in zip(self.offsets, self.entries)]


def packed_offsets(entries: Sequence[Entry], align: int = PACK_ALIGN) -> List[int]:
    offs, cur = [], 0
    for e in entries:
        cur = (cur + align - 1) // align * align
        offs.append(cur)
        cur += e.rows * e.cols
    return offs


def _w1() -> Workload:
    ents = (Entry("sq0", 128, 128), Entry("sq1", 128, 128),
            Entry("wide0", 128, 512), Entry("wide1", 128, 512),
            Entry("tall0", 512, 128), Entry("tall1", 512, 128))
    return Workload(1, "tiny fp32 Muon step", ents, "f32", "f32")


def _w2() -> Workload:
    ents = (Entry("q", 2048, 2048), Entry("k", 2048, 2048), Entry("v", 2048, 2048),
            Entry("o", 2048, 2048), Entry("gate", 5632, 2048), Entry("up", 5632, 2048),
            Entry("down", 2048, 5632))
    return Workload(2, "one transformer layer's Muon targets", ents, "bf16", "bf16")


def _w3() -> Workload:
    ents = tuple([Entry(f"attn{i}", 4096, 4096) for i in range(16)]
                 + [Entry(f"gateup{i}", 11008, 4096) for i in range(8)]
                 + [Entry(f"down{i}", 4096, 11008) for i in range(4)])
    return Workload(3, "owner packed buffer at 1/8 share of a 7B-class model", ents,
                    "bf16", "bf16")


def _w4() -> Workload:
    ents = []
    for e in range(64):
        ents += [Entry(f"e{e}.gate", 1408, 2048), Entry(f"e{e}.up", 1408, 2048),
                 Entry(f"e{e}.down", 2048, 1408)]
    return Workload(4, "MoE expert batch", tuple(ents), "bf16", "bf16")


def _w5() -> Workload:
    ents = []
    for layer in range(32):
        for nm in ("q", "k", "v", "o"):
            ents.append(Entry(f"l{layer}.{nm}", 4096, 4096, split_rows=128))
    return Workload(5, "per-head split plus AdamW", tuple(ents), "bf16", "bf16",
                    adamw_sizes=(32000 * 4096,) + (4096,) * 65)


WORKLOADS = {1: _w1, 2: _w2, 3: _w3, 4: _w4, 5: _w5}


def workload(wid: int) -> Workload:
    return WORKLOADS[wid]()


def custom_workload(shapes: Sequence[Tuple[int, ...]], grad_dtype: str = "bf16",
                    ns_dtype: str = "bf16", wid: int = 100, lr: float = 0.02,
                    momentum: float = 0.95, weight_decay: float = 0.1,
                    grad_kind: str = "") -> Workload:
    """A workload from explicit (rows, cols, split_rows[, split_cols]) shapes (used
    for ragged cases)."""
    ents = tuple(Entry(f"m{i}", *sh) for i, sh in enumerate(shapes))
    return Workload(wid, "custom", ents, grad_dtype, ns_dtype, lr, momentum, weight_decay,
                    grad_kind=grad_kind)


# ----------------------------------------------------------------------------
# value encodings (storage formats of the inputs; no method arithmetic)

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (NaN kept quiet)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def entry_rng(wid: int, index: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([wid, index])))


def entry_values(wl: Workload, index: int) -> Tuple[np.ndarray, np.ndarray]:
    """(grad, param) of one entry: grad as stored (float32 values, or bf16 bits as
    uint16), param float32; both shaped (rows, cols)."""
    e = wl.entries[index]
    rng = entry_rng(wl.wid, index)
    if wl.kind == "gaussian":
        g = rng.standard_normal((e.rows, e.cols)).astype(np.float32)
        p = rng.standard_normal((e.rows, e.cols)).astype(np.float32)
        return (g if wl.grad_dtype == "f32" else f32_to_bf16_bits(g)), p
    r = 16
    u = rng.standard_normal((e.rows, r))
    v = rng.standard_normal((e.cols, r))
    noise = rng.standard_normal((e.rows, e.cols))
    g64 = (1e-3 / np.sqrt(r)) * (u @ v.T) + 1e-5 * noise
    p = rng.standard_normal((e.rows, e.cols)).astype(np.float32)
    g32 = g64.astype(np.float32)
    return (g32 if wl.grad_dtype == "f32" else f32_to_bf16_bits(g32)), p


def grad_as_f64(wl: Workload, g: np.ndarray) -> np.ndarray:
    if wl.grad_dtype == "f32":
        return np.asarray(g, dtype=np.float64)
    return bf16_bits_to_f32(g).astype(np.float64)


def host_inputs(wl: Workload, only: Optional[Sequence[int]] = None):
    """Packed host buffers (params float32, grads float32 or bf16 bits, momentum
    zeros float32) for the entries in `only` (all by default). Entries left out
    and the alignment gaps hold zeros."""
    n = wl.numel
    params = np.zeros(n, np.float32)
    grads = np.zeros(n, np.float32 if wl.grad_dtype == "f32" else np.uint16)
    idx = range(len(wl.entries)) if only is None else only
    for i in idx:
        e, off = wl.entries[i], wl.offsets[i]
        g, p = entry_values(wl, i)
        params[off:off + e.rows * e.cols] = p.ravel()
        grads[off:off + e.rows * e.cols] = g.ravel()
    return params, grads, np.zeros(n, np.float32)


def adamw_inputs(n: int, seed: int = 0):
    """AdamW tensors: params and grads N(0,1) (grads stored bf16), zero moments."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([500, seed])))
    p = rng.standard_normal(n).astype(np.float32)
    g = f32_to_bf16_bits(rng.standard_normal(n).astype(np.float32))
    return p, g, np.zeros(n, np.float32), np.zeros(n, np.float32)
