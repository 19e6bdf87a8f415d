"""Python binding of the gfx950 block-sparse attention library (libbsa.so).

Argument marshalling only: every step of the forward pass runs in the
library's host planner and HIP kernels. PyTorch tensors are accepted for the
device buffers (only their data pointers and the stream handle are used); the
logical mask is host memory (numpy arrays).

The names follow the C ABI in ``include/bsa.h``:
``plan`` (bsa_plan), ``forward`` (bsa_forward), ``Plan.info``
(bsa_plan_info), ``Plan.coverage`` (bsa_plan_coverage).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsa.so")

# enums of bsa.h
OK, ERR_INVALID_ARGUMENT, ERR_INVALID_MASK, ERR_UNSUPPORTED, ERR_OUT_OF_MEMORY, ERR_HIP, ERR_INTERNAL = range(7)
MASK_BLOCK_U8, MASK_BLOCK_BITS, MASK_SLICE_CSR, MASK_VIDEO = 1, 2, 3, 4
PAT_DENSE, PAT_SPATIAL, PAT_TEMPORAL = 0, 1, 2
LAYOUT_FRAME_MAJOR, LAYOUT_TEMPORAL_MAJOR = 0, 1
DTYPE_BF16, DTYPE_F32 = 0, 1
TILE_FULL, TILE_PARTIAL = 0, 1
PRED_NONE, PRED_SUBBLOCK, PRED_VIDEO, PRED_LIST = 0, 1, 2, 3
ORDER_XCD_GROUPED, ORDER_LONGEST_FIRST = 0, 1
ABI_VERSION = 7  # the structures below mirror this version of bsa.h

EXPORTED = ["bsa_abi_version", "bsa_plan_opts_default", "bsa_plan", "bsa_plan_device", "bsa_forward", "bsa_forward_stamped",
            "bsa_plan_destroy",
            "bsa_request_create", "bsa_request_submit", "bsa_request_finish", "bsa_request_stats",
            "bsa_request_destroy", "bsa_route_heads", "bsa_route_heads_noalloc",
            "bsa_plan_info", "bsa_plan_coverage", "bsa_regime_count", "bsa_regime_info", "bsa_status_str",
            "bsa_last_error"]


class MaskDesc(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("data", ctypes.c_void_p), ("row_ptr", ctypes.c_void_p),
                ("col_idx", ctypes.c_void_p), ("head_pattern", ctypes.c_void_p), ("anchor_frame", ctypes.c_int32),
                ("radius", ctypes.c_int32), ("nnz", ctypes.c_int64)]


class PlanOpts(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("T", ctypes.c_int32), ("Hg", ctypes.c_int32), ("Wg", ctypes.c_int32),
                ("head_layout", ctypes.c_void_p), ("force_regime", ctypes.c_int32), ("lut_path", ctypes.c_char_p),
                ("device", ctypes.c_int32), ("task_order", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("regime", ctypes.c_int32), ("tile_q", ctypes.c_int32), ("tile_k", ctypes.c_int32),
                ("gather", ctypes.c_int32), ("tasks", ctypes.c_int64), ("workgroups", ctypes.c_int64),
                ("tiles_full", ctypes.c_int64),
                ("tiles_partial", ctypes.c_int64), ("tiles_empty", ctypes.c_int64), ("gather_rows", ctypes.c_int64),
                ("executed_pairs", ctypes.c_double), ("device_bytes", ctypes.c_int64), ("plan_ns", ctypes.c_int64),
                ("phase_ns", ctypes.c_int64 * 5), ("task_order", ctypes.c_int32), ("mask_density", ctypes.c_double),
                ("mask_fill", ctypes.c_double), ("mask_fill2", ctypes.c_double)]

    def as_dict(self):
        d = {k: getattr(self, k) for k, _ in self._fields_}
        d["phase_ns"] = dict(zip(("ingest", "regime", "mapping", "tasks", "upload"), list(self.phase_ns)))
        return d


class RequestDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("L", ctypes.c_int64), ("d", ctypes.c_int32),
                ("opts", PlanOpts), ("stream", ctypes.c_void_p), ("plan_stream", ctypes.c_void_p),
                ("depth", ctypes.c_int32)]


class RequestStats(ctypes.Structure):
    _fields_ = [("submitted", ctypes.c_int64), ("plan_ns", ctypes.c_int64), ("wait_ns", ctypes.c_int64)]


class RouteDesc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("Hg", ctypes.c_int32), ("Wg", ctypes.c_int32),
                ("anchor_frame", ctypes.c_int32), ("radius", ctypes.c_int32), ("rows", ctypes.c_void_p),
                ("n_rows", ctypes.c_int32), ("device", ctypes.c_int32)]


class RegimeDesc(ctypes.Structure):
    _fields_ = [("family", ctypes.c_int32), ("tile_q", ctypes.c_int32), ("tile_k", ctypes.c_int32),
                ("waves", ctypes.c_int32), ("rows_per_wave", ctypes.c_int32)]


class TileRecord(ctypes.Structure):
    _fields_ = [("q0", ctypes.c_int64), ("q1", ctypes.c_int64), ("kind", ctypes.c_int32),
                ("predicate", ctypes.c_int32), ("k0", ctypes.c_int64), ("k1", ctypes.c_int64),
                ("keys", ctypes.POINTER(ctypes.c_int32)), ("nkeys", ctypes.c_int64), ("sub_bits", ctypes.c_uint32),
                ("sub_q", ctypes.c_int32), ("sub_k", ctypes.c_int32), ("task", ctypes.c_int64)]


SINK = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(TileRecord))

_lib = None


def lib(path: str = LIB_PATH):
    """Load libbsa.so; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() (no CPU fallback exists)")
    # PyTorch ships its own HIP runtime under the same soname. Loading torch
    # first makes the library bind to that runtime, so that device pointers
    # and streams from torch are valid in the library (two HIP runtimes in one
    # process do not share devices, memory or streams).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(path)
    L.bsa_abi_version.restype = ctypes.c_int32
    if L.bsa_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{path}: ABI version {L.bsa_abi_version()}, the binding expects {ABI_VERSION}")
    L.bsa_plan_opts_default.argtypes = [ctypes.POINTER(PlanOpts)]
    L.bsa_plan.restype = ctypes.c_int32
    L.bsa_plan.argtypes = [ctypes.POINTER(MaskDesc), ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                           ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(PlanOpts), ctypes.POINTER(ctypes.c_void_p)]
    L.bsa_plan_device.restype = ctypes.c_int32
    L.bsa_plan_device.argtypes = [ctypes.POINTER(MaskDesc), ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                  ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(PlanOpts),
                                  ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)]
    L.bsa_request_create.restype = ctypes.c_int32
    L.bsa_request_create.argtypes = [ctypes.POINTER(RequestDesc), ctypes.POINTER(ctypes.c_void_p)]
    L.bsa_request_submit.restype = ctypes.c_int32
    L.bsa_request_submit.argtypes = [ctypes.c_void_p, ctypes.POINTER(MaskDesc), ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p]
    L.bsa_request_finish.restype = ctypes.c_int32
    L.bsa_request_finish.argtypes = [ctypes.c_void_p]
    L.bsa_request_stats.restype = ctypes.c_int32
    L.bsa_request_stats.argtypes = [ctypes.c_void_p, ctypes.POINTER(RequestStats)]
    L.bsa_request_destroy.restype = None
    L.bsa_request_destroy.argtypes = [ctypes.c_void_p]
    for fn in (L.bsa_route_heads, L.bsa_route_heads_noalloc):
        fn.restype = ctypes.c_int32
        fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                       ctypes.c_int64, ctypes.c_int32, ctypes.POINTER(RouteDesc), ctypes.c_void_p,
                       ctypes.c_void_p, ctypes.c_void_p]
    L.bsa_forward.restype = ctypes.c_int32
    L.bsa_forward.argtypes = [ctypes.c_void_p] * 6
    L.bsa_forward_stamped.restype = ctypes.c_int32
    L.bsa_forward_stamped.argtypes = [ctypes.c_void_p] * 7
    L.bsa_plan_destroy.argtypes = [ctypes.c_void_p]
    L.bsa_plan_info.restype = ctypes.c_int32
    L.bsa_plan_info.argtypes = [ctypes.c_void_p, ctypes.POINTER(PlanInfo)]
    L.bsa_plan_coverage.restype = ctypes.c_int32
    L.bsa_plan_coverage.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, SINK, ctypes.c_void_p]
    L.bsa_regime_count.restype = ctypes.c_int32
    L.bsa_regime_info.restype = ctypes.c_int32
    L.bsa_regime_info.argtypes = [ctypes.c_int32, ctypes.POINTER(RegimeDesc)]
    L.bsa_status_str.restype = ctypes.c_char_p
    L.bsa_status_str.argtypes = [ctypes.c_int32]
    L.bsa_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


class BSAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def _check(status: int):
    if status != OK:
        raise BSAError(status, lib().bsa_last_error().decode())


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _dptr(t):
    if isinstance(t, int):
        return t
    return t.data_ptr()


class Plan:
    """An immutable execution plan (owns its host and device memory)."""

    def __init__(self, handle: int, L: int, H: int, B: int):
        self._h = handle
        self.L, self.H, self.B = L, H, B

    @property
    def handle(self):
        return self._h

    def info(self) -> dict:
        out = PlanInfo()
        _check(lib().bsa_plan_info(self._h, ctypes.byref(out)))
        return out.as_dict()

    def coverage(self, b: int, h: int):
        """Tile records of head (b, h) in task order, as dicts."""
        recs = []

        def sink(user, rp):
            r = rp.contents
            d = {"q0": r.q0, "q1": r.q1, "kind": r.kind, "predicate": r.predicate, "k0": r.k0, "k1": r.k1,
                 "sub_bits": r.sub_bits, "sub_q": r.sub_q, "sub_k": r.sub_k, "task": r.task}
            if r.predicate == PRED_LIST:
                d["keys"] = np.ctypeslib.as_array(r.keys, shape=(r.nkeys,)).copy() if r.nkeys else np.zeros(0, np.int32)
            recs.append(d)
            return 0

        cb = SINK(sink)
        _check(lib().bsa_plan_coverage(self._h, b, h, cb, None))
        return recs

    def close(self):
        if self._h:
            lib().bsa_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _arr(x, dt, keep):
    if x is None:
        return None
    a = np.ascontiguousarray(x, dtype=dt)
    keep.append(a)
    return a


def _host_mask(kind, data, row_ptr, col_idx, head_pattern, anchor_frame, radius, keep) -> MaskDesc:
    m = MaskDesc()
    m.kind = kind
    m.data = _ptr(_arr(data, np.uint8 if kind == MASK_BLOCK_U8 else np.uint64, keep))
    m.row_ptr = _ptr(_arr(row_ptr, np.int64, keep))
    m.col_idx = _ptr(_arr(col_idx, np.int32, keep))
    m.head_pattern = _ptr(_arr(head_pattern, np.uint8, keep))
    m.anchor_frame = anchor_frame
    m.radius = radius
    return m


def _opts(dtype, T, Hg, Wg, head_layout, force_regime, lut_path, device, task_order, keep) -> PlanOpts:
    o = PlanOpts()
    lib().bsa_plan_opts_default(ctypes.byref(o))
    o.dtype = dtype
    o.T, o.Hg, o.Wg = T, Hg, Wg
    o.head_layout = _ptr(_arr(head_layout, np.uint8, keep))
    o.force_regime = force_regime
    o.lut_path = lut_path.encode() if lut_path else None
    keep.append(o.lut_path)
    o.device = device
    o.task_order = task_order
    return o


def plan(kind: int, B: int, H: int, L: int, d: int, block_q: int, block_k: int, *, data=None, row_ptr=None,
         col_idx=None, head_pattern=None, anchor_frame: int = 0, radius: int = 2, dtype: int = DTYPE_BF16,
         T: int = 0, Hg: int = 0, Wg: int = 0, head_layout=None, force_regime: int = -1,
         lut_path: Optional[str] = None, device: int = 0, task_order: int = -1) -> Plan:
    """bsa_plan: build a plan for a logical mask (host numpy arrays)."""
    keep = []
    m = _host_mask(kind, data, row_ptr, col_idx, head_pattern, anchor_frame, radius, keep)
    o = _opts(dtype, T, Hg, Wg, head_layout, force_regime, lut_path, device, task_order, keep)
    h = ctypes.c_void_p()
    _check(lib().bsa_plan(ctypes.byref(m), B, H, L, d, block_q, block_k, ctypes.byref(o), ctypes.byref(h)))
    return Plan(h.value, L, H, B)


class Request:
    """bsa_request_*: plan + forward over a sequence of masks of one shape,
    with the planning of each mask overlapping the forwards already enqueued
    (at most `depth` plans alive). Masks are host numpy arrays, or, with
    on_device=True, BLOCK masks in device memory (torch tensors)."""

    def __init__(self, B: int, H: int, L: int, d: int, *, depth: int = 3, stream=None, plan_stream=None,
                 dtype: int = DTYPE_BF16, T: int = 0, Hg: int = 0, Wg: int = 0, head_layout=None,
                 force_regime: int = -1, lut_path: Optional[str] = None, device: int = 0, task_order: int = -1):
        keep = []
        desc = RequestDesc()
        desc.B, desc.H, desc.L, desc.d = B, H, L, d
        desc.opts = _opts(dtype, T, Hg, Wg, head_layout, force_regime, lut_path, device, task_order, keep)
        desc.stream = _stream_handle(stream)
        desc.plan_stream = _stream_handle(plan_stream) if plan_stream is not None else None
        desc.depth = depth
        h = ctypes.c_void_p()
        _check(lib().bsa_request_create(ctypes.byref(desc), ctypes.byref(h)))
        self._h = h.value
        self._depth = depth
        self._masks = []  # device masks of the plans that may still be in flight

    def submit(self, kind: int, block_q: int, block_k: int, q, k, v, o, *, data=None, row_ptr=None, col_idx=None,
               nnz: int = 0, head_pattern=None, anchor_frame: int = 0, radius: int = 2,
               on_device: bool = False) -> None:
        keep = []
        if on_device:
            m = MaskDesc()
            m.kind = kind
            m.data = _dptr(data) if data is not None else None
            m.row_ptr = _dptr(row_ptr) if row_ptr is not None else None
            m.col_idx = _dptr(col_idx) if col_idx is not None else None
            m.nnz = nnz
            # a plan (and the planning that read its mask) is retired once
            # `depth` newer plans exist: older masks may go
            self._masks.append((data, row_ptr, col_idx))
            if len(self._masks) > self._depth + 1:
                self._masks.pop(0)
        else:
            m = _host_mask(kind, data, row_ptr, col_idx, head_pattern, anchor_frame, radius, keep)
        _check(lib().bsa_request_submit(self._h, ctypes.byref(m), block_q, block_k, int(on_device), _dptr(q), _dptr(k),
                                        _dptr(v), _dptr(o)))

    def finish(self) -> None:
        _check(lib().bsa_request_finish(self._h))
        self._masks.clear()

    def stats(self) -> dict:
        st = RequestStats()
        _check(lib().bsa_request_stats(self._h, ctypes.byref(st)))
        return {"submitted": st.submitted, "plan_ns": st.plan_ns, "wait_ns": st.wait_ns}

    def close(self) -> None:
        if self._h:
            lib().bsa_request_destroy(self._h)
            self._h = None
            self._masks.clear()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _stream_handle(stream) -> int:
    """hipStream_t of a torch stream, a raw handle (int), or None (the
    current torch stream)."""
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def plan_device(kind: int, B: int, H: int, L: int, d: int, block_q: int, block_k: int, data=None, *, row_ptr=None,
                col_idx=None, nnz: int = 0, stream=None,
                dtype: int = DTYPE_BF16, T: int = 0, Hg: int = 0, Wg: int = 0, head_layout=None,
                force_regime: int = -1, lut_path: Optional[str] = None, device: int = 0,
                task_order: int = -1) -> Plan:
    """bsa_plan_device: build a plan on the device from a mask in device memory
    (contiguous torch tensors or raw device addresses: `data` bytes for
    BLOCK_U8 or 64-bit rows for BLOCK_BITS; `row_ptr` int64, `col_idx` int32
    and `nnz` for SLICE_CSR), enqueued on `stream`. The returned plan keeps
    references to the mask tensors."""
    L_ = lib()
    keep = []
    m = MaskDesc()
    m.kind = kind
    m.data = _dptr(data) if data is not None else None
    m.row_ptr = _dptr(row_ptr) if row_ptr is not None else None
    m.col_idx = _dptr(col_idx) if col_idx is not None else None
    m.nnz = nnz
    o = _opts(dtype, T, Hg, Wg, head_layout, force_regime, lut_path, device, task_order, keep)
    h = ctypes.c_void_p()
    _check(L_.bsa_plan_device(ctypes.byref(m), B, H, L, d, block_q, block_k, ctypes.byref(o), _stream_handle(stream),
                              ctypes.byref(h)))
    pl = Plan(h.value, L, H, B)
    pl._mask = (data, row_ptr, col_idx)
    return pl


def forward(p: Plan, q, k, v, o, stream=None) -> None:
    """bsa_forward: enqueue the forward pass on `stream` (torch stream, raw
    hipStream_t as int, or None for the current torch stream)."""
    _check(lib().bsa_forward(p.handle, _dptr(q), _dptr(k), _dptr(v), _dptr(o), _stream_handle(stream)))


def forward_stamped(p: Plan, q, k, v, o, stamps, stream=None) -> None:
    """bsa_forward_stamped: bsa_forward that also writes per-workgroup clock
    stamps into `stamps` (a device int64 tensor of 4 * workgroups entries)."""
    _check(lib().bsa_forward_stamped(p.handle, _dptr(q), _dptr(k), _dptr(v), _dptr(o), _dptr(stamps),
                                     _stream_handle(stream)))



def route_heads(q, k, v, B: int, H: int, L: int, d: int, T: int, Hg: int, Wg: int, rows, *, anchor_frame: int = 0,
                radius: int = 2, device: int = 0, stream=None):
    """bsa_route_heads: per head, the video pattern (PAT_SPATIAL or
    PAT_TEMPORAL) whose output over the sampled query tokens `rows` is nearer
    the dense output. Returns (pattern uint8 [H], err float64 [H][2]).
    Synchronises with `stream`."""
    r = np.ascontiguousarray(rows, dtype=np.int32)
    desc = RouteDesc()
    desc.T, desc.Hg, desc.Wg = T, Hg, Wg
    desc.anchor_frame, desc.radius = anchor_frame, radius
    desc.rows = _ptr(r)
    desc.n_rows = r.size
    desc.device = device
    pat = np.zeros(H, np.uint8)
    err = np.zeros((H, 2), np.float64)
    _check(lib().bsa_route_heads(_dptr(q), _dptr(k), _dptr(v), B, H, L, d, ctypes.byref(desc),
                                 _stream_handle(stream), _ptr(pat), _ptr(err)))
    return pat, err


def route_heads_noalloc(q, k, v, B: int, H: int, L: int, d: int, T: int, Hg: int, Wg: int, rows, *,
                        anchor_frame: int = 0, radius: int = 2, device: int = 0, stream=None):
    """bsa_route_heads_noalloc: route_heads with no memory allocation (a
    fixed scratch array per device). Returns (pattern uint8 [H], err float64
    [H][2]); synchronises with `stream`."""
    r = np.ascontiguousarray(rows, dtype=np.int32)
    desc = RouteDesc()
    desc.T, desc.Hg, desc.Wg = T, Hg, Wg
    desc.anchor_frame, desc.radius = anchor_frame, radius
    desc.rows = _ptr(r)
    desc.n_rows = r.size
    desc.device = device
    pat = np.zeros(H, np.uint8)
    err = np.zeros((H, 2), np.float64)
    _check(lib().bsa_route_heads_noalloc(_dptr(q), _dptr(k), _dptr(v), B, H, L, d, ctypes.byref(desc),
                                         _stream_handle(stream), _ptr(pat), _ptr(err)))
    return pat, err


def regimes():
    L_ = lib()
    out = []
    for r in range(L_.bsa_regime_count()):
        d = RegimeDesc()
        _check(L_.bsa_regime_info(r, ctypes.byref(d)))
        out.append({"family": d.family, "tile_q": d.tile_q, "tile_k": d.tile_k, "waves": d.waves,
                    "rows_per_wave": d.rows_per_wave})
    return out
