"""CPU oracle for the neighbour-graph attention hot path (TEST INFRASTRUCTURE).

Plain, slow, obviously correct fp64 reference of what the GPU path computes:

* ``nl_row`` / ``nl_full``: brute-force neighbour rows over every atom and
  every periodic image, nearest-``sel`` by the total key (r2, j, n);
* ``attn_naive`` / ``attn_naive_centres``: per-centre multi-head attention in
  naive loops;
* ``attn_pairaxis``: the same layers in the ragged pair-axis form (pairs,
  segment softmax, index_add);
* ``block_gather`` / ``block_scatter``: the padded per-centre block through
  the destination CSR and its scatter back to the edge axis.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the GPU
library (``neighbour_graph_attention_amd``) and neither imports the other.
The arithmetic lives in ``oracle.c``; this module only marshals numpy
arrays through ctypes.  Sources are cited in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(verbose: bool = False) -> str:
    """Compile oracle.c into liboracle.so (gcc, OpenMP, no FP contraction)."""
    cmd = ["gcc", "-O3", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", _SRC, "-o", _LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_void_p
    lib.orc_nl_row.restype = i64
    lib.orc_nl_row.argtypes = [vp, i64, vp, dbl, i32, i64, vp, vp, vp, vp, vp]
    lib.orc_nl_rows.restype = ctypes.c_int
    lib.orc_nl_rows.argtypes = [vp, i64, vp, dbl, i32, vp, i64, vp, vp, vp, vp]
    lib.orc_nl_full.restype = i64
    lib.orc_nl_full.argtypes = [vp, i64, vp, dbl, i32, vp, vp, vp, vp, i64]
    for name in ("orc_attn_naive", "orc_attn_pairaxis"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [vp, vp, i64, i64, i32, i32, i32, vp, vp, vp]
    lib.orc_attn_smooth.restype = ctypes.c_int
    lib.orc_attn_smooth.argtypes = [vp, vp, i64, i64, i32, i32, i32, vp, vp, vp, vp]
    lib.orc_local_atten.restype = ctypes.c_int
    lib.orc_local_atten.argtypes = [vp, vp, i64, i64, i32, i32, i32, vp, vp, vp, vp]
    lib.orc_attn_naive_centres.restype = ctypes.c_int
    lib.orc_attn_naive_centres.argtypes = [vp, vp, vp, i64, i32, i32, i32, vp, vp, vp]
    for name in ("orc_block_gather", "orc_block_scatter"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [vp, vp, i64, i64, i32, i32, i32, vp, vp]
    lib.orc_num_threads.restype = ctypes.c_int
    lib.orc_num_threads.argtypes = []
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def num_threads() -> int:
    return int(_load().orc_num_threads())


def nl_row(pos, box, rcut: float, sel: int, i: int):
    """One centre's row: (col[k], shift[k][3], vec[k][3], r2[k], n_within)."""
    lib = _load()
    pos = _f64(pos)
    box = _f64(box)
    n = pos.shape[0]
    col = np.empty(sel, np.int32)
    shift = np.empty((sel, 3), np.int32)
    vec = np.empty((sel, 3), np.float64)
    r2 = np.empty(sel, np.float64)
    nw = ctypes.c_int64(0)
    k = lib.orc_nl_row(_ptr(pos), n, _ptr(box), float(rcut), int(sel), int(i), _ptr(col),
                       _ptr(shift), _ptr(vec), _ptr(r2), ctypes.byref(nw))
    if k < 0:
        raise MemoryError("oracle nl_row failed")
    return col[:k].copy(), shift[:k].copy(), vec[:k].copy(), r2[:k].copy(), int(nw.value)


def nl_rows(pos, box, rcut: float, sel: int, centres):
    """Rows of the listed centres as a CSR over the list: (row_ptr, col, shift, vec)."""
    lib = _load()
    pos = _f64(pos)
    box = _f64(box)
    centres = np.ascontiguousarray(centres, dtype=np.int64)
    m = centres.shape[0]
    counts = np.empty(m, np.int64)
    col = np.empty((max(m, 1), sel), np.int32)
    shift = np.empty((max(m, 1), sel, 3), np.int32)
    vec = np.empty((max(m, 1), sel, 3), np.float64)
    rc = lib.orc_nl_rows(_ptr(pos), pos.shape[0], _ptr(box), float(rcut), int(sel), _ptr(centres),
                         m, _ptr(counts), _ptr(col), _ptr(shift), _ptr(vec))
    if rc != 0:
        raise MemoryError("oracle nl_rows failed")
    row_ptr = np.zeros(m + 1, np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    keep = np.arange(sel)[None, :] < counts[:, None]
    return row_ptr, col[:m][keep], shift[:m][keep], vec[:m][keep]


def nl_full(pos, box, rcut: float, sel: int):
    """Whole destination CSR: (row_ptr[N+1] int64, col[E] int32, shift[E][3] int32, vec[E][3])."""
    lib = _load()
    pos = _f64(pos)
    box = _f64(box)
    n = pos.shape[0]
    cap = n * sel
    row_ptr = np.empty(n + 1, np.int64)
    col = np.empty(max(cap, 1), np.int32)
    shift = np.empty((max(cap, 1), 3), np.int32)
    vec = np.empty((max(cap, 1), 3), np.float64)
    e = lib.orc_nl_full(_ptr(pos), n, _ptr(box), float(rcut), int(sel), _ptr(row_ptr),
                        _ptr(col), _ptr(shift), _ptr(vec), cap)
    if e < 0:
        raise MemoryError("oracle nl_full failed")
    return row_ptr, col[:e].copy(), shift[:e].copy(), vec[:e].copy()


def _attn_args(row_ptr, order, x, w):
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int64)
    order = None if order is None else np.ascontiguousarray(order, dtype=np.int32)
    x = _f64(x)
    w = _f64(w)
    return row_ptr, order, x, w


def attn_naive(row_ptr, x, w, heads: int, order=None):
    """Stacked layers, layer by layer over all centres.  x: [E][c]; w: [L][4][c][c]."""
    lib = _load()
    row_ptr, order, x, w = _attn_args(row_ptr, order, x, w)
    e, c = x.shape
    y = np.zeros_like(x)
    rc = lib.orc_attn_naive(_ptr(row_ptr), _ptr(order), row_ptr.shape[0] - 1, e, c, heads,
                            w.shape[0], _ptr(w), _ptr(x), _ptr(y))
    if rc != 0:
        raise ValueError("oracle attn_naive failed")
    return y


def attn_smooth(row_ptr, x, w, heads: int, log_dtilde, order=None):
    """Smooth attention: stacked layers with each segment's softmax rescaled by
    sum_j e_j / D~.  log_dtilde: ln D~ as [L][E][heads], keyed by the query edge's row."""
    lib = _load()
    row_ptr, order, x, w = _attn_args(row_ptr, order, x, w)
    e, c = x.shape
    ldt = _f64(log_dtilde)
    if ldt.shape != (w.shape[0], e, heads):
        raise ValueError("log_dtilde must be [layers][E][heads]")
    y = np.zeros_like(x)
    rc = lib.orc_attn_smooth(_ptr(row_ptr), _ptr(order), row_ptr.shape[0] - 1, e, c, heads,
                             w.shape[0], _ptr(w), _ptr(x), _ptr(ldt), _ptr(y))
    if rc != 0:
        raise ValueError("oracle attn_smooth failed")
    return y


def local_atten(row_ptr, xc, x, w, heads: int, order=None):
    """LocalAtten: one query per centre (xc [N][c]) over the centre's edges (x [E][c]) as keys
    and values; stacked layers update xc.  Returns yc [N][c]."""
    lib = _load()
    row_ptr, order, x, w = _attn_args(row_ptr, order, x, w)
    xc = _f64(xc)
    e, c = x.shape
    n = row_ptr.shape[0] - 1
    if xc.shape != (n, c):
        raise ValueError("xc must be [n_centres][c]")
    yc = np.zeros_like(xc)
    rc = lib.orc_local_atten(_ptr(row_ptr), _ptr(order), n, e, c, heads, w.shape[0], _ptr(w),
                             _ptr(xc), _ptr(x), _ptr(yc))
    if rc != 0:
        raise ValueError("oracle local_atten failed")
    return yc


def attn_naive_centres(row_ptr, x, w, heads: int, centres, order=None):
    """Stacked layers for the listed centres only; other rows of the result are NaN."""
    lib = _load()
    row_ptr, order, x, w = _attn_args(row_ptr, order, x, w)
    centres = np.ascontiguousarray(centres, dtype=np.int64)
    e, c = x.shape
    y = np.full_like(x, np.nan)
    rc = lib.orc_attn_naive_centres(_ptr(row_ptr), _ptr(order), _ptr(centres), centres.shape[0],
                                    c, heads, w.shape[0], _ptr(w), _ptr(x), _ptr(y))
    if rc != 0:
        raise ValueError("oracle attn_naive_centres failed")
    return y


def attn_pairaxis(row_ptr, x, w, heads: int, order=None):
    """Stacked layers in the ragged pair-axis form.  x: [E][c]; w: [L][4][c][c]."""
    lib = _load()
    row_ptr, order, x, w = _attn_args(row_ptr, order, x, w)
    e, c = x.shape
    y = np.zeros_like(x)
    rc = lib.orc_attn_pairaxis(_ptr(row_ptr), _ptr(order), row_ptr.shape[0] - 1, e, c, heads,
                               w.shape[0], _ptr(w), _ptr(x), _ptr(y))
    if rc != 0:
        raise ValueError("oracle attn_pairaxis failed")
    return y


def block_gather(row_ptr, x, cap: int, order=None):
    """Padded per-centre block [n_centres][cap][c] of the rows of x (same dtype), zeros past
    each centre's row count."""
    lib = _load()
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int64)
    order = None if order is None else np.ascontiguousarray(order, dtype=np.int32)
    x = np.ascontiguousarray(x)
    e, c = x.shape
    nc = row_ptr.shape[0] - 1
    block = np.empty((nc, cap, c), dtype=x.dtype)
    rc = lib.orc_block_gather(_ptr(row_ptr), _ptr(order), nc, e, int(cap), c, x.itemsize,
                              _ptr(x), _ptr(block))
    if rc != 0:
        raise ValueError("oracle block_gather: row over cap or index out of range")
    return block


def block_scatter(row_ptr, block, y, order=None):
    """Write the valid rows of block [n_centres][cap][c] back into y [E][c] (in place; rows of
    no centre untouched); returns y."""
    lib = _load()
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int64)
    order = None if order is None else np.ascontiguousarray(order, dtype=np.int32)
    block = np.ascontiguousarray(block)
    if not (y.flags["C_CONTIGUOUS"] and y.dtype == block.dtype):
        raise ValueError("y must be C-contiguous with the block's dtype")
    nc, cap, c = block.shape
    rc = lib.orc_block_scatter(_ptr(row_ptr), _ptr(order), nc, y.shape[0], cap, c,
                               block.itemsize, _ptr(block), _ptr(y))
    if rc != 0:
        raise ValueError("oracle block_scatter: row over cap or index out of range")
    return y
