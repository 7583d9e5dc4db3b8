"""ctypes binding of libmuonstep (argument marshalling only).

Every step of the Muon step runs in the library's HIP kernels; this module only
turns torch tensors into device pointers and the current HIP stream, and turns
status codes into MuonError. It never computes a result itself, and it raises
if the library is missing.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmuonstep.so")

# status codes (include/muon_step.h)
OK, ERR_NULL, ERR_BAD_METHOD, ERR_BAD_SHAPE, ERR_RANGE, ERR_OVERLAP, ERR_ALIGN, \
    ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_BAD_HYPER = range(11)
STATUS_NAMES = {
    0: "MUON_OK", 1: "MUON_ERR_NULL", 2: "MUON_ERR_BAD_METHOD", 3: "MUON_ERR_BAD_SHAPE",
    4: "MUON_ERR_RANGE", 5: "MUON_ERR_OVERLAP", 6: "MUON_ERR_ALIGN", 7: "MUON_ERR_UNSUPPORTED",
    8: "MUON_ERR_WORKSPACE", 9: "MUON_ERR_HIP", 10: "MUON_ERR_BAD_HYPER",
}
DTYPES = {"f32": 0, "bf16": 1, "f16": 2}
NS_METHODS = {"standard": 0, "gram": 1}

EXPORTED = (
    "muon_default_hyper", "muon_default_adamw_hyper", "muon_workspace_size", "muon_step",
    "muon_step_window", "adamw_step", "muon_pack", "muon_unpack", "muon_last_error", "muon_release_plans",
    "muon_profile_begin", "muon_profile_end", "muon_version", "muon_ns_flops",
    "muon_plan_owners", "muon_comm_elements", "muon_step_noalloc",
)
NOALLOC_WORKSPACE_BYTES = 64 << 20     # MUON_NOALLOC_WORKSPACE_BYTES


class MuonError(RuntimeError):
    """A non-zero status from libmuonstep."""

    def __init__(self, status: int, message: str):
        self.status = status
        self.message = message
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")


class MuonMatrix(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_int64), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("split_rows", ctypes.c_int64),
                ("split_cols", ctypes.c_int64)]


class MuonHyper(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("momentum", ctypes.c_float),
                ("weight_decay", ctypes.c_float), ("ns_a", ctypes.c_float),
                ("ns_b", ctypes.c_float), ("ns_c", ctypes.c_float),
                ("ns_steps", ctypes.c_int32), ("ns_eps", ctypes.c_float),
                ("ns_method", ctypes.c_int32), ("param_dtype", ctypes.c_int32),
                ("grad_dtype", ctypes.c_int32), ("ns_dtype", ctypes.c_int32)]


class MuonWindow(ctypes.Structure):
    _fields_ = [("lo", ctypes.c_int64), ("hi", ctypes.c_int64), ("param_offset", ctypes.c_int64)]


class MuonParam(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("split_rows", ctypes.c_int64),
                ("layer", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("split_cols", ctypes.c_int64)]


class MuonAssign(ctypes.Structure):
    _fields_ = [("owner", ctypes.c_int32), ("reserved", ctypes.c_int32), ("offset", ctypes.c_int64)]


class MuonOwner(ctypes.Structure):
    _fields_ = [("numel", ctypes.c_int64), ("max_layer_numel", ctypes.c_int64),
                ("ns_flops", ctypes.c_int64), ("n_matrices", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class AdamWHyper(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("step", ctypes.c_int32), ("grad_dtype", ctypes.c_int32)]


class KernelStat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int32),
                ("total_ms", ctypes.c_double)]


_lib = None
_lock = threading.Lock()


def load() -> ctypes.CDLL:
    """Load the built library (raises if it has not been built).

    torch is imported first: torch ships its own HIP runtime under the same
    soname (libamdhip64.so.7) as the system one the library links against, and
    the first one loaded serves the whole process. Loaded in this order the
    library shares torch's runtime (and torch's tensors and streams); loaded
    the other way round, torch ran on the system runtime and the library's
    first HIP call failed."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it with "
                              "`python -m newton_schulz_step_amd.build`")
        import torch  # noqa: F401  (see above)
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        pm = ctypes.POINTER(MuonMatrix)
        lib.muon_default_hyper.argtypes = [ctypes.POINTER(MuonHyper)]
        lib.muon_default_hyper.restype = None
        lib.muon_default_adamw_hyper.argtypes = [ctypes.POINTER(AdamWHyper)]
        lib.muon_default_adamw_hyper.restype = None
        lib.muon_workspace_size.argtypes = [pm, i32, ctypes.POINTER(MuonHyper), ctypes.POINTER(sz)]
        lib.muon_step.argtypes = [vp, vp, vp, i64, pm, i32, ctypes.POINTER(MuonHyper), vp, sz,
                                  vp, vp, vp]
        lib.muon_step_noalloc.argtypes = [vp, vp, vp, i64, pm, i32, ctypes.POINTER(MuonHyper), vp, vp, vp]
        lib.muon_step_window.argtypes = [vp, i64, vp, vp, i64, pm, ctypes.POINTER(MuonWindow), i32,
                                         ctypes.POINTER(MuonHyper), vp, sz, vp, vp, vp]
        lib.adamw_step.argtypes = [vp, vp, vp, vp, i64, ctypes.POINTER(AdamWHyper), vp]
        lib.muon_pack.argtypes = [vp, i64, ctypes.POINTER(vp), pm, i32, i32, vp]
        lib.muon_unpack.argtypes = [ctypes.POINTER(vp), vp, i64, pm, i32, i32, vp]
        lib.muon_ns_flops.argtypes = [i64, i64, i32, i32]
        lib.muon_ns_flops.restype = i64
        lib.muon_plan_owners.argtypes = [ctypes.POINTER(MuonParam), i32, i32, i32, i32, i64,
                                         ctypes.POINTER(MuonAssign), ctypes.POINTER(MuonOwner)]
        lib.muon_comm_elements.argtypes = [i64, i32, i32, i32]
        lib.muon_comm_elements.restype = ctypes.c_double
        lib.muon_last_error.restype = ctypes.c_char_p
        lib.muon_version.restype = ctypes.c_char_p
        lib.muon_profile_end.argtypes = [ctypes.POINTER(KernelStat), i32, ctypes.POINTER(i32)]
        for name in ("muon_workspace_size", "muon_step", "muon_step_noalloc", "muon_step_window", "muon_plan_owners",
                     "adamw_step", "muon_pack", "muon_unpack",
                     "muon_release_plans", "muon_profile_begin", "muon_profile_end"):
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
        return lib


def _check(status: int) -> None:
    if status != OK:
        raise MuonError(status, load().muon_last_error().decode(errors="replace"))


def version() -> str:
    return load().muon_version().decode()


# ----------------------------------------------------------------------------- hyperparameters

def hyper(**kw) -> MuonHyper:
    """Muon-group hyperparameters: the library defaults, then keyword overrides.

    Accepts lr / muon_lr (muon_lr wins, as in the DeepSpeed config), momentum,
    weight_decay, ns_method ("standard" | "gram"), ns_steps, ns_eps, ns_a/b/c,
    grad_dtype and ns_dtype ("f32" | "bf16" | "f16"), param_dtype ("f32" | "bf16")."""
    h = MuonHyper()
    load().muon_default_hyper(ctypes.byref(h))
    kw = dict(kw)
    if "muon_lr" in kw:
        kw["lr"] = kw.pop("muon_lr")
    for k, v in kw.items():
        if k == "ns_method":
            v = NS_METHODS.get(v, v) if isinstance(v, str) else v
            if isinstance(v, str):
                v = -1
        elif k in ("grad_dtype", "ns_dtype", "param_dtype") and isinstance(v, str):
            v = DTYPES[v]
        if not hasattr(h, k):
            raise TypeError(f"unknown Muon hyperparameter {k!r}")
        setattr(h, k, v)
    return h


def table(entries: Iterable[Sequence[int]]):
    """ctypes array of muon_matrix_t from (offset, rows, cols[, split_rows[,
    split_cols]]) tuples."""
    rows = [tuple(e) + (0,) * (5 - len(e)) for e in entries]
    arr = (MuonMatrix * max(len(rows), 1))()
    for i, (o, r, c, s, sc) in enumerate(rows):
        arr[i] = MuonMatrix(o, r, c, s, sc)
    return arr, len(rows)


def workspace_size(entries, h: MuonHyper) -> int:
    arr, n = table(entries)
    out = ctypes.c_size_t(0)
    _check(load().muon_workspace_size(arr, n, ctypes.byref(h), ctypes.byref(out)))
    return out.value


# ----------------------------------------------------------------------------- torch plumbing

_TORCH_DT = None


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}
    if t.dtype not in m:
        raise TypeError(f"unsupported tensor dtype {t.dtype}")
    return m[t.dtype]


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to libmuonstep must be on a GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmuonstep must be contiguous")
    return t.data_ptr()


def _stream(t, stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _device(*tensors):
    """The one GPU all given tensors (None skipped) live on; every call runs with
    it as the current device."""
    devs = {t.device for t in tensors if t is not None}
    if len(devs) != 1:
        raise ValueError(f"tensors passed to libmuonstep must share one GPU, got {sorted(map(str, devs))}")
    dev = devs.pop()
    if dev.type != "cuda":
        raise ValueError("tensors passed to libmuonstep must be on a GPU")
    return dev


_ws_cache: Dict[Tuple[int, int], object] = {}
_ws_lock = threading.Lock()
_WS_CACHE_MAX = 16      # (device, stream) pairs kept; the oldest is dropped first


def workspace(nbytes: int, device, stream=None) -> "torch.Tensor":
    """A device workspace of at least `nbytes` bytes, cached per (device, stream).

    Steps enqueued on one stream reuse it in stream order; steps on different
    streams get different buffers, so they may run concurrently. A torch stream's
    buffer is allocated on that stream, so when a larger one replaces it the old
    memory is recycled in that stream's order. With a raw stream handle the
    caller orders the stream against torch's current stream. At most
    _WS_CACHE_MAX buffers are kept (a dropped one was allocated on its own
    stream, so torch reuses its memory in that stream's order)."""
    torch = _torch()
    dev = torch.device(device)
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    s = stream if stream is not None else torch.cuda.current_stream(idx)
    key = (idx, s.cuda_stream if hasattr(s, "cuda_stream") else int(s))
    with _ws_lock:
        buf = _ws_cache.get(key)
        if buf is None or buf.numel() < nbytes:
            _ws_cache.pop(key, None)
            size = max(nbytes, 256)
            if isinstance(s, torch.cuda.Stream):
                with torch.cuda.stream(s):
                    buf = torch.empty(size, dtype=torch.uint8, device=torch.device("cuda", idx))
            else:
                buf = torch.empty(size, dtype=torch.uint8, device=torch.device("cuda", idx))
            _ws_cache[key] = buf
            while len(_ws_cache) > _WS_CACHE_MAX:
                _ws_cache.pop(next(iter(_ws_cache)))
    return buf


def step(params, grads, momentum, entries, h: MuonHyper, ws=None, update_out=None,
         bf16_shadow=None, stream=None) -> None:
    """One Muon step (muon_step) on packed torch tensors; updates params and momentum."""
    torch = _torch()
    if momentum.dtype != torch.float32:
        raise TypeError("momentum must be float32")
    if params.dtype not in (torch.float32, torch.bfloat16) or _dtype_code(params) != h.param_dtype:
        raise TypeError("params must be float32 or bfloat16, matching hyper.param_dtype")
    if _dtype_code(grads) != h.grad_dtype:
        raise TypeError("grads dtype does not match hyper.grad_dtype")
    numel = params.numel()
    if grads.numel() != numel or momentum.numel() != numel:
        raise ValueError("params, grads and momentum must have the same numel")
    dev = _device(params, grads, momentum, ws, update_out, bf16_shadow)
    arr, n = table(entries)
    need = ctypes.c_size_t(0)
    _check(load().muon_workspace_size(arr, n, ctypes.byref(h), ctypes.byref(need)))
    if ws is None:
        ws = workspace(need.value, dev, stream)
    if update_out is not None and (update_out.dtype != torch.float32 or update_out.numel() != numel):
        raise ValueError("update_out must be float32 with params' numel")
    if bf16_shadow is not None and (bf16_shadow.element_size() != 2 or bf16_shadow.numel() != numel):
        raise ValueError("bf16_shadow must be a 16-bit tensor with params' numel")
    with torch.cuda.device(dev):
        _check(load().muon_step(_ptr(params), _ptr(grads), _ptr(momentum), numel, arr, n,
                                ctypes.byref(h), _ptr(ws), ws.numel() * ws.element_size(),
                                _ptr(update_out), _ptr(bf16_shadow), _stream(params, stream)))


def step_noalloc(params, grads, momentum, entries, h: MuonHyper, update_out=None,
                 bf16_shadow=None, stream=None) -> None:
    """One Muon step through muon_step_noalloc: no workspace argument, nothing
    allocated (the library's per-GPU device array serves as the workspace)."""
    torch = _torch()
    if momentum.dtype != torch.float32:
        raise TypeError("momentum must be float32")
    if params.dtype not in (torch.float32, torch.bfloat16) or _dtype_code(params) != h.param_dtype:
        raise TypeError("params must be float32 or bfloat16, matching hyper.param_dtype")
    if _dtype_code(grads) != h.grad_dtype:
        raise TypeError("grads dtype does not match hyper.grad_dtype")
    numel = params.numel()
    if grads.numel() != numel or momentum.numel() != numel:
        raise ValueError("params, grads and momentum must have the same numel")
    if update_out is not None and (update_out.dtype != torch.float32 or update_out.numel() != numel):
        raise ValueError("update_out must be float32 with params' numel")
    if bf16_shadow is not None and (bf16_shadow.element_size() != 2 or bf16_shadow.numel() != numel):
        raise ValueError("bf16_shadow must be a 16-bit tensor with params' numel")
    dev = _device(params, grads, momentum, update_out, bf16_shadow)
    arr, n = table(entries)
    with torch.cuda.device(dev):
        _check(load().muon_step_noalloc(_ptr(params), _ptr(grads), _ptr(momentum), numel, arr, n,
                                        ctypes.byref(h), _ptr(update_out), _ptr(bf16_shadow),
                                        _stream(params, stream)))


def windows(ws: Iterable[Sequence[int]], n: int):
    """ctypes array of muon_window_t from (lo, hi, param_offset) tuples, one per entry."""
    rows = [tuple(w) for w in ws]
    if len(rows) != n:
        raise ValueError("one window per table entry")
    arr = (MuonWindow * max(n, 1))()
    for i, (lo, hi, po) in enumerate(rows):
        arr[i] = MuonWindow(lo, hi, po)
    return arr


def step_window(partition, grads, momentum, entries, wins, h: MuonHyper, ws=None,
                update_out=None, bf16_shadow=None, stream=None) -> None:
    """One Muon step for the holder of a parameter partition (muon_step_window):
    momentum and Newton-Schulz on every listed matrix in full, the update
    applied to the window (lo, hi, param_offset) of each entry in `partition`."""
    torch = _torch()
    if partition.dtype != torch.float32 or momentum.dtype != torch.float32:
        raise TypeError("partition and momentum must be float32")
    if _dtype_code(grads) != h.grad_dtype:
        raise TypeError("grads dtype does not match hyper.grad_dtype")
    numel = momentum.numel()
    if grads.numel() != numel:
        raise ValueError("grads and momentum must have the same numel")
    dev = _device(partition, grads, momentum, ws, update_out, bf16_shadow)
    arr, n = table(entries)
    warr = windows(wins, n)
    need = ctypes.c_size_t(0)
    _check(load().muon_workspace_size(arr, n, ctypes.byref(h), ctypes.byref(need)))
    if ws is None:
        ws = workspace(need.value, dev, stream)
    if update_out is not None and (update_out.dtype != torch.float32 or update_out.numel() != numel):
        raise ValueError("update_out must be float32 with momentum's numel")
    if bf16_shadow is not None and (bf16_shadow.element_size() != 2 or
                                    bf16_shadow.numel() != partition.numel()):
        raise ValueError("bf16_shadow must be a 16-bit tensor with the partition's numel")
    with torch.cuda.device(dev):
        _check(load().muon_step_window(_ptr(partition), partition.numel(), _ptr(grads), _ptr(momentum),
                                       numel, arr, warr, n, ctypes.byref(h), _ptr(ws),
                                       ws.numel() * ws.element_size(), _ptr(update_out),
                                       _ptr(bf16_shadow), _stream(momentum, stream)))


def _method_code(method) -> int:
    return NS_METHODS[method] if isinstance(method, str) else int(method)


def ns_flops(m: int, n: int, method="standard", steps: int = 5) -> int:
    """Nominal Newton-Schulz FLOPs of one problem with short side m, long side n."""
    f = load().muon_ns_flops(m, n, _method_code(method), steps)
    if f < 0:
        raise ValueError("invalid problem for the FLOP model")
    return int(f)


def plan_owners(params: Sequence[Sequence[int]], n_owners: int, method="standard",
                steps: int = 5, align: int = 64):
    """Owner plan (muon_plan_owners) for matrices given as (rows, cols, split_rows,
    layer[, split_cols]). Returns (assign, owners): assign[i] = (owner, offset);
    owners[o] = dict(numel, max_layer_numel, ns_flops, n_matrices, table), where
    `table` is the owner's muon_step table [(offset, rows, cols, split_rows,
    split_cols), ...] in packed order, and `index` the matching input indices."""
    rows = [tuple(p) + (0,) * (5 - len(p)) for p in params]
    n = len(rows)
    arr = (MuonParam * max(n, 1))()
    for i, (r, c, s, layer, sc) in enumerate(rows):
        arr[i] = MuonParam(r, c, s, layer, 0, sc)
    out_a = (MuonAssign * max(n, 1))()
    out_o = (MuonOwner * max(n_owners, 1))()
    _check(load().muon_plan_owners(arr, n, n_owners, _method_code(method), steps, align, out_a,
                                   out_o))
    assign = [(out_a[i].owner, out_a[i].offset) for i in range(n)]
    owners = []
    for o in range(n_owners):
        idx = sorted((i for i in range(n) if assign[i][0] == o), key=lambda i: assign[i][1])
        owners.append({"numel": out_o[o].numel, "max_layer_numel": out_o[o].max_layer_numel,
                       "ns_flops": out_o[o].ns_flops, "n_matrices": out_o[o].n_matrices,
                       "index": idx,
                       "table": [(assign[i][1], rows[i][0], rows[i][1], rows[i][2], rows[i][4])
                                 for i in idx]})
    return assign, owners


def comm_elements(p_m: int, n_ranks: int, zero_stage: int = 2, dedicated: bool = True) -> float:
    """Elements sent per step on the shard group (muon_comm_elements)."""
    v = load().muon_comm_elements(p_m, n_ranks, zero_stage, int(bool(dedicated)))
    if v < 0:
        raise ValueError("invalid arguments for the communication model")
    return v


def adamw(params, grads, m, v, lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-10, weight_decay=0.0,
          step: int = 1, stream=None) -> None:
    """AdamW step (adamw_step) on flat torch tensors; updates params, m and v."""
    torch = _torch()
    for t in (params, m, v):
        if t.dtype != torch.float32:
            raise TypeError("params, m and v must be float32")
    numel = params.numel()
    if any(t.numel() != numel for t in (grads, m, v)):
        raise ValueError("params, grads, m and v must have the same numel")
    h = AdamWHyper()
    load().muon_default_adamw_hyper(ctypes.byref(h))
    h.lr, h.beta1, h.beta2, h.eps, h.weight_decay = lr, beta1, beta2, eps, weight_decay
    h.step = step
    h.grad_dtype = _dtype_code(grads)
    dev = _device(params, grads, m, v)
    with torch.cuda.device(dev):
        _check(load().adamw_step(_ptr(params), _ptr(grads), _ptr(m), _ptr(v), numel, ctypes.byref(h),
                                 _stream(params, stream)))


def _copy_args(packed, tensors: Sequence, entries):
    """Table and pointer array for pack / unpack; each tensor must hold exactly its
    entry's rows * cols elements of the packed buffer's dtype (the copy is sized
    from the table and that dtype)."""
    tensors = list(tensors)
    arr, n = table(entries)
    if len(tensors) != n:
        raise ValueError(f"{len(tensors)} tensors for {n} table entries")
    for i, t in enumerate(tensors):
        if t.dtype != packed.dtype or t.numel() != arr[i].rows * arr[i].cols:
            raise ValueError(f"tensor {i} must be {packed.dtype} with {arr[i].rows * arr[i].cols} elements, "
                             f"got {t.dtype} with {t.numel()}")
    ptrs = (ctypes.c_void_p * max(n, 1))(*[_ptr(t) for t in tensors])
    return arr, n, ptrs, _device(packed, *tensors)


def pack(packed, tensors: Sequence, entries, stream=None) -> None:
    """Copy each tensor bit for bit into `packed` at its table offset."""
    torch = _torch()
    arr, n, ptrs, dev = _copy_args(packed, tensors, entries)
    with torch.cuda.device(dev):
        _check(load().muon_pack(_ptr(packed), packed.numel(), ptrs, arr, n, _dtype_code(packed),
                                _stream(packed, stream)))


def unpack(tensors: Sequence, packed, entries, stream=None) -> None:
    """Copy each table entry of `packed` bit for bit into its tensor."""
    torch = _torch()
    arr, n, ptrs, dev = _copy_args(packed, tensors, entries)
    with torch.cuda.device(dev):
        _check(load().muon_unpack(ptrs, _ptr(packed), packed.numel(), arr, n, _dtype_code(packed),
                                  _stream(packed, stream)))


def release_plans() -> None:
    _check(load().muon_release_plans())


def profile_begin() -> None:
    _check(load().muon_profile_begin())


def profile_end() -> Dict[str, Tuple[int, float]]:
    """{kernel kind: (launches, summed milliseconds)} since profile_begin()."""
    out = (KernelStat * 64)()
    n = ctypes.c_int32(0)
    _check(load().muon_profile_end(out, 64, ctypes.byref(n)))
    return {out[i].name.decode(): (out[i].launches, out[i].total_ms) for i in range(min(n.value, 64))}
