"""CPU oracle for masked (block-sparse) attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package. It shares no code with the GPU
path (``block_sparse_attention_fwd_amd``) and never imports it; the two meet
only in the seeded input generators of ``workloads``.

The arithmetic lives in ``oracle.c`` (plain fp64 C, OpenMP over rows); this
file only builds it and marshals arguments. See ``oracle.c`` for what is
computed and which passage of the source pages each rule follows.

Parity pins (what the oracle is checked against, in ``tests/``): brute force
with ``math.fsum`` on tiny inputs, a library attention routine (PyTorch CPU
float64 scaled-dot-product attention with a boolean mask built independently),
the definition's invariants (masked key == deleted key, block mask == its
element expansion, key/value permutation invariance, token-permutation
equivariance of temporal-major heads), closed forms (one kept key, constant V,
empty row, score shift, query/key rescale) and closed-form pair counts of the
video patterns, and the per-block key unions (``om_block_union``,
``om_union_total``) against an independent element-mask union and the
geometry's hand-computed totals. No function of this oracle is "parity
unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import types

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (-O2, OpenMP). Returns the library path."""
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-shared", "-fPIC", src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


class OmMask(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32), ("B", ctypes.c_int32), ("H", ctypes.c_int32),
        ("L", ctypes.c_int64),
        ("bq", ctypes.c_int32), ("bk", ctypes.c_int32),
        ("block_u8", ctypes.c_void_p), ("block_bits", ctypes.c_void_p),
        ("row_ptr", ctypes.c_void_p), ("col_idx", ctypes.c_void_p),
        ("head_pattern", ctypes.c_void_p),
        ("anchor", ctypes.c_int32), ("radius", ctypes.c_int32),
        ("T", ctypes.c_int32), ("Hg", ctypes.c_int32), ("Wg", ctypes.c_int32),
        ("head_layout", ctypes.c_void_p),
    ]


_lib = None


def lib(path: str = _LIB):
    global _lib
    if _lib is not None and path == _LIB:
        return _lib
    if not os.path.exists(path):
        build(out=path)
    L = ctypes.CDLL(path)
    L.om_row_keys.restype = ctypes.c_int64
    L.om_row_keys.argtypes = [ctypes.POINTER(OmMask), ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p]
    L.om_attend.restype = None
    L.om_attend.argtypes = [ctypes.POINTER(OmMask), ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    L.om_count_pairs.restype = ctypes.c_int64
    L.om_count_pairs.argtypes = [ctypes.POINTER(OmMask), ctypes.c_int32, ctypes.c_int32]
    L.om_union_total.restype = ctypes.c_int64
    L.om_union_total.argtypes = [ctypes.POINTER(OmMask), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    L.om_block_union.restype = None
    L.om_block_union.argtypes = [ctypes.POINTER(OmMask), ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                 ctypes.c_void_p]
    if path == _LIB:
        _lib = L
    return L


def _ptr(a):
    return None if a is None else a.ctypes.data


class Mask:
    """Oracle-side view of a workload's logical mask (keeps arrays alive)."""

    def __init__(self, w, bits: bool = False):
        self.keep = []
        m = OmMask()
        m.kind = 2 if (bits and w.kind == 1) else w.kind
        m.B, m.H, m.L = w.B, w.H, w.L
        m.bq, m.bk = w.bq, w.bk
        if w.kind == 1:
            if bits:
                arr = np.ascontiguousarray(w.block_bits())
                m.block_bits = _ptr(arr)
            else:
                arr = np.ascontiguousarray(w.block, dtype=np.uint8)
                m.block_u8 = _ptr(arr)
            self.keep.append(arr)
        if w.kind == 3:
            rp = np.ascontiguousarray(w.row_ptr, dtype=np.int64)
            ci = np.ascontiguousarray(w.col_idx, dtype=np.int32)
            m.row_ptr, m.col_idx = _ptr(rp), _ptr(ci)
            self.keep += [rp, ci]
        if w.kind == 4:
            hp = np.ascontiguousarray(w.head_pattern, dtype=np.uint8)
            m.head_pattern = _ptr(hp)
            self.keep.append(hp)
        m.anchor, m.radius = w.anchor, w.radius
        m.T, m.Hg, m.Wg = w.T, w.Hg, w.Wg
        if w.head_layout is not None:
            hl = np.ascontiguousarray(w.head_layout, dtype=np.uint8)
            m.head_layout = _ptr(hl)
            self.keep.append(hl)
        self.m = m
        self.L = w.L
        self.H = w.H
        self.B = w.B


_DT = {np.dtype(np.uint16): 0, np.dtype(np.float32): 1, np.dtype(np.float64): 2}


def attend(w, Q, K, V, rows=None, lib_path: str = _LIB, bits: bool = False, return_counts: bool = False):
    """fp64 attention output. rows: flat row ids (b*H + h)*L + q (default all).
    Returns [nrows][d] float64 (and per-row kept counts if asked)."""
    L_ = lib(lib_path)
    mk = Mask(w, bits=bits)
    Q = np.ascontiguousarray(Q)
    K = np.ascontiguousarray(K)
    V = np.ascontiguousarray(V)
    assert Q.dtype == K.dtype == V.dtype and Q.dtype in _DT
    d = Q.shape[-1]
    if rows is None:
        rows = np.arange(w.B * w.H * w.L, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, d), np.float64)
    cnt = np.zeros(rows.size, np.int64)
    L_.om_attend(ctypes.byref(mk.m), d, _DT[Q.dtype], _ptr(Q), _ptr(K), _ptr(V), _ptr(rows), rows.size, _ptr(out),
                 _ptr(cnt))
    return (out, cnt) if return_counts else out


def row_keys(w, b, h, q, lib_path: str = _LIB):
    L_ = lib(lib_path)
    mk = Mask(w)
    buf = np.zeros(max(1, w.L), np.int32)
    n = L_.om_row_keys(ctypes.byref(mk.m), b, h, q, _ptr(buf))
    return buf[:n].copy()


def count_pairs(w, b=0, h=0, lib_path: str = _LIB) -> int:
    L_ = lib(lib_path)
    mk = Mask(w)
    return int(L_.om_count_pairs(ctypes.byref(mk.m), b, h))


def block_union(w, b, h, blk, M=64, lib_path: str = _LIB):
    L_ = lib(lib_path)
    mk = Mask(w)
    used = np.zeros(w.L, np.uint8)
    L_.om_block_union(ctypes.byref(mk.m), b, h, blk, M, _ptr(used))
    return used


def union_total(w, b=0, h=0, M=64, lib_path: str = _LIB) -> int:
    """Sum over the M-row query blocks of head (b, h), in the head's logical
    order, of the number of distinct keys kept by any query of the block
    (FG-Attn, abstract: the keys relevant to a block of queries)."""
    L_ = lib(lib_path)
    mk = Mask(w)
    return int(L_.om_union_total(ctypes.byref(mk.m), b, h, M))


def gather_bytes(w, M=64, lib_path: str = _LIB) -> int:
    """Mask-defined gather bytes G of a workload: per head, every M-row query
    block loads each distinct key it keeps once as a K row and a V row, and the
    head's Q is read and O written once (d-wide rows of the input dtype; bf16
    here, 2 bytes). Heads with identical masks are counted once each."""
    row = 2 * w.d
    per = {}
    total = 0
    for b in range(w.B):
        for h in range(w.H):
            key = _head_key(w, b, h)
            if key is None or key not in per:
                u = union_total(w, b, h, M, lib_path=lib_path)
                if key is not None:
                    per[key] = u
            else:
                u = per[key]
            total += 2 * row * u + 2 * row * w.L
    return total


def _head_key(w, b, h):
    """A key that two heads share only when their masks are identical (video
    heads of one pattern and layout); None when heads must be counted alone."""
    if w.kind == 4:
        lay = int(w.head_layout[h]) if w.head_layout is not None else 0
        return (int(w.head_pattern[h]), lay)
    return None


def route_heads(Q, K, V, T: int, Hg: int, Wg: int, rows, anchor: int = 0, radius: int = 2, lib_path: str = _LIB):
    """Head routing, fp64 (Sparse VideoGen / Splash Attention summary, "Sparse
    VideoGen": each head is routed on the fly to a spatial or a temporal
    sparse pattern; the pages give no rule). Reading: per head, the pattern
    whose masked attention output is nearer the dense output, as the mean
    squared difference over the batch, the sampled query tokens ``rows``
    (frame-major) and the head dimension; ties go to spatial. The outputs are
    this oracle's masked attention under the video patterns (all heads dense,
    all spatial, all temporal). Returns (pattern uint8 [H]: 1 spatial,
    2 temporal; err float64 [H][2]: spatial, temporal)."""
    B, H, L, d = Q.shape
    rows = np.asarray(rows, dtype=np.int64)
    flat = ((np.arange(B)[:, None, None] * H + np.arange(H)[None, :, None]) * L + rows[None, None, :]).reshape(-1)
    outs = []
    for pat in (0, 1, 2):
        spec = types.SimpleNamespace(kind=4, B=B, H=H, L=L, bq=1, bk=1, head_pattern=np.full(H, pat, np.uint8),
                                     anchor=anchor, radius=radius, T=T, Hg=Hg, Wg=Wg, head_layout=None)
        outs.append(attend(spec, Q, K, V, rows=flat, lib_path=lib_path).reshape(B, H, rows.size, d))
    err = np.zeros((H, 2), np.float64)
    err[:, 0] = ((outs[1] - outs[0]) ** 2).mean(axis=(0, 2, 3))
    err[:, 1] = ((outs[2] - outs[0]) ** 2).mean(axis=(0, 2, 3))
    pattern = np.where(err[:, 0] <= err[:, 1], 1, 2).astype(np.uint8)
    return pattern, err
