"""ctypes binding of libnga.so (the C ABI declared in include/nga.h).

Argument marshalling only: tensors are checked for dtype, shape, device and
contiguity, outputs and workspaces are allocated with torch when the caller
does not pass them, and the raw device pointers plus torch's current HIP
stream go to the library.  Every step of the computation runs in the
library's HIP kernels; there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnga.so")

NGA_OK, NGA_EINVAL, NGA_EBOX, NGA_EROWCAP, NGA_ECAP, NGA_EDTYPE, NGA_EWORKSPACE, NGA_EHIP, \
    NGA_EINDEX, NGA_ETOOBIG = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9
STATIC_SCRATCH_BYTES = 16 << 20
NGA_F64, NGA_F32, NGA_F32_SPLIT16 = 0, 1, 2
ROW_CAP = 512

EXPORTS = ("nl_build_workspace_bytes", "nl_build", "edge_csr_workspace_bytes", "edge_csr",
           "block_attn_workspace_bytes", "block_attn_forward", "nga_sync_status", "nga_strerror",
           "nga_attn_variant", "nga_attn_plan", "pair_attn_workspace_bytes", "pair_attn_forward",
           "block_attn_forward_smooth", "local_attn_workspace_bytes", "local_attn_forward",
           "nga_step_graph_create", "nga_step_graph_launch", "nga_step_graph_destroy",
           "nl_refine", "nl_max_displacement", "nl_build_batch_workspace_bytes",
           "nl_build_batch", "nl_build_static", "block_gather", "block_scatter")


class NGAError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} (status {code})")


_lib = None


def load() -> ctypes.CDLL:
    """Load libnga.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with neighbour_graph_attention_amd._build")
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, dbl, vp, sz = (ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_void_p,
                             ctypes.c_size_t)
    lib.nl_build_workspace_bytes.restype = sz
    lib.nl_build_workspace_bytes.argtypes = [i64, vp, dbl]
    lib.nl_build.restype = ctypes.c_int
    lib.nl_build.argtypes = [vp, i64, vp, dbl, i32, vp, vp, vp, vp, sz, vp]
    lib.edge_csr_workspace_bytes.restype = sz
    lib.edge_csr_workspace_bytes.argtypes = [i64, i32]
    lib.edge_csr.restype = ctypes.c_int
    lib.edge_csr.argtypes = [vp, vp, vp, i64, i32, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, sz, vp]
    lib.block_attn_workspace_bytes.restype = sz
    lib.block_attn_workspace_bytes.argtypes = [ctypes.c_int, i64, i32, i32, i32, i32]
    lib.block_attn_forward.restype = ctypes.c_int
    lib.block_attn_forward.argtypes = [ctypes.c_int, vp, vp, i64, i64, i32, i32, i32, i32, vp, vp,
                                       vp, vp, sz, vp]
    lib.block_attn_forward_smooth.restype = ctypes.c_int
    lib.block_attn_forward_smooth.argtypes = [ctypes.c_int, vp, vp, i64, i64, i32, i32, i32, i32,
                                              vp, vp, vp, vp, vp, sz, vp]
    for name in ("block_gather", "block_scatter"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_int, vp, vp, i64, i64, i32, i32, vp, vp, vp, sz, vp]
    lib.nl_build_static.restype = ctypes.c_int
    lib.nl_build_static.argtypes = [vp, i64, vp, dbl, i32, vp, vp, vp, vp, vp]
    lib.nl_build_batch_workspace_bytes.restype = sz
    lib.nl_build_batch_workspace_bytes.argtypes = [i32, vp, vp, dbl]
    lib.nl_build_batch.restype = ctypes.c_int
    lib.nl_build_batch.argtypes = [vp, i32, vp, vp, dbl, i32, vp, vp, vp, vp, sz, vp]
    lib.nl_refine.restype = ctypes.c_int
    lib.nl_refine.argtypes = [vp, i64, vp, dbl, i32, vp, vp, vp, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.nl_max_displacement.restype = ctypes.c_int
    lib.nl_max_displacement.argtypes = [vp, vp, i64, vp, vp, vp]
    lib.nga_step_graph_create.restype = ctypes.c_int
    lib.nga_step_graph_create.argtypes = [vp, i64, vp, dbl, i32, vp, vp, vp, vp, sz, vp, vp, vp,
                                          vp, vp, i64, vp, sz, ctypes.c_int, i32, i32, i32, vp,
                                          vp, vp, vp, sz, ctypes.POINTER(vp)]
    lib.nga_step_graph_launch.restype = ctypes.c_int
    lib.nga_step_graph_launch.argtypes = [vp, vp]
    lib.nga_step_graph_destroy.restype = ctypes.c_int
    lib.nga_step_graph_destroy.argtypes = [vp]
    lib.local_attn_workspace_bytes.restype = sz
    lib.local_attn_workspace_bytes.argtypes = [ctypes.c_int, i64, i32, i32, i32]
    lib.local_attn_forward.restype = ctypes.c_int
    lib.local_attn_forward.argtypes = [ctypes.c_int, vp, vp, i64, i64, i32, i32, i32, vp, vp, vp,
                                       vp, vp, sz, vp]
    lib.pair_attn_workspace_bytes.restype = sz
    lib.pair_attn_workspace_bytes.argtypes = [ctypes.c_int, i64, i64, i32, i32, i32, i64]
    lib.pair_attn_forward.restype = ctypes.c_int
    lib.pair_attn_forward.argtypes = [ctypes.c_int, vp, vp, i64, i64, i32, i32, i32, vp, vp, vp,
                                      i64, vp, sz, vp]
    lib.nga_sync_status.restype = ctypes.c_int
    lib.nga_sync_status.argtypes = [vp, vp]
    lib.nga_strerror.restype = ctypes.c_char_p
    lib.nga_strerror.argtypes = [ctypes.c_int]
    lib.nga_attn_variant.restype = ctypes.c_char_p
    lib.nga_attn_variant.argtypes = [ctypes.c_int, i32, i32, i32]
    lib.nga_attn_plan.restype = ctypes.c_char_p
    lib.nga_attn_plan.argtypes = [ctypes.c_int, i64, i32, i32, i32]
    _lib = lib
    return lib


def strerror(code: int) -> str:
    return load().nga_strerror(int(code)).decode()


def _check(code: int, where: str) -> None:
    if code != NGA_OK:
        raise NGAError(code, where)


def _box3(box) -> ctypes.Array:
    vals = [float(v) for v in box]
    if len(vals) != 3:
        raise ValueError("box must have 3 side lengths")
    return (ctypes.c_double * 3)(*vals)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class Workspace:
    """A zero-filled device byte buffer, grown on demand, holding the status word."""

    def __init__(self, device, nbytes: int = 256):
        self.device = torch.device(device)
        self.buf = torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=self.device)

    @property
    def nbytes(self) -> int:
        return self.buf.numel()

    def ensure(self, nbytes: int) -> "Workspace":
        if nbytes > self.nbytes:
            torch.cuda.current_stream(self.device).synchronize()
            self.buf = torch.zeros(int(nbytes), dtype=torch.uint8, device=self.device)
        return self

    def ptr(self):
        return ctypes.c_void_p(self.buf.data_ptr())


def _ws(ws, device, nbytes):
    if ws is None:
        ws = Workspace(device, nbytes)
    return ws.ensure(nbytes)


def sync_status(ws: Workspace) -> int:
    """Synchronise the current stream, return and clear the workspace's device error."""
    return int(load().nga_sync_status(ws.ptr(), _stream(ws.device)))


def check_status(ws: Workspace, where: str = "nga") -> None:
    _check(sync_status(ws), where)


def nl_build_workspace_bytes(n_atoms: int, box, rcut: float) -> int:
    return int(load().nl_build_workspace_bytes(int(n_atoms), _box3(box), float(rcut)))


def nl_build(pos: torch.Tensor, box, rcut: float, sel: int, *, nbr=None, nbr_shift=None,
             nnei=None, ws: Workspace | None = None):
    """Neighbour rows: returns (nbr [N][sel] int32, nbr_shift [N][sel][3] int32, nnei [N] int32)."""
    lib = load()
    dev = pos.device
    n = pos.shape[0]
    _need(pos, "pos", torch.float64, (n, 3), dev)
    nbytes = nl_build_workspace_bytes(n, box, rcut)
    if nbytes == 0:
        raise NGAError(NGA_EINVAL, "nl_build_workspace_bytes")
    ws = _ws(ws, dev, nbytes)
    if nbr is None:
        nbr = torch.empty((n, sel), dtype=torch.int32, device=dev)
    if nbr_shift is None:
        nbr_shift = torch.empty((n, sel, 3), dtype=torch.int32, device=dev)
    if nnei is None:
        nnei = torch.empty((n,), dtype=torch.int32, device=dev)
    _need(nbr, "nbr", torch.int32, (n, sel), dev)
    _need(nbr_shift, "nbr_shift", torch.int32, (n, sel, 3), dev)
    _need(nnei, "nnei", torch.int32, (n,), dev)
    rc = lib.nl_build(_ptr(pos), n, _box3(box), float(rcut), int(sel), _ptr(nbr), _ptr(nbr_shift),
                      _ptr(nnei), ws.ptr(), ws.nbytes, _stream(dev))
    _check(rc, "nl_build")
    return nbr, nbr_shift, nnei


def nl_build_static(pos: torch.Tensor, box, rcut: float, sel: int, status: Workspace, *,
                    nbr=None, nbr_shift=None, nnei=None):
    """nl_build without a workspace (the library's static device scratch; allocation-free on the
    library side).  Device-detected errors go to `status` (a Workspace of at least 256 bytes,
    read with sync_status / check_status).  Returns (nbr, nbr_shift, nnei)."""
    lib = load()
    dev = pos.device
    n = pos.shape[0]
    _need(pos, "pos", torch.float64, (n, 3), dev)
    if nbr is None:
        nbr = torch.empty((n, sel), dtype=torch.int32, device=dev)
    if nbr_shift is None:
        nbr_shift = torch.empty((n, sel, 3), dtype=torch.int32, device=dev)
    if nnei is None:
        nnei = torch.empty((n,), dtype=torch.int32, device=dev)
    _need(nbr, "nbr", torch.int32, (n, sel), dev)
    _need(nbr_shift, "nbr_shift", torch.int32, (n, sel, 3), dev)
    _need(nnei, "nnei", torch.int32, (n,), dev)
    if status.nbytes < 256 or status.device != dev:
        raise ValueError("status must be a Workspace of at least 256 bytes on the device")
    rc = lib.nl_build_static(_ptr(pos), n, _box3(box), float(rcut), int(sel), _ptr(nbr),
                             _ptr(nbr_shift), _ptr(nnei), status.ptr(), _stream(dev))
    _check(rc, "nl_build_static")
    return nbr, nbr_shift, nnei


def edge_csr(nbr: torch.Tensor, nbr_shift: torch.Tensor, nnei: torch.Tensor | None = None, *,
             pos: torch.Tensor | None = None, box=None, e_cap: int | None = None,
             want_dst: bool = True, want_edge_vec: bool = False, read_n_edges: bool = True,
             out: dict | None = None, ws: Workspace | None = None):
    """Destination CSR.  Returns a dict with row_ptr, col, shift, dst, edge_vec, n_edges.

    With read_n_edges (default) the call synchronises once and the edge arrays are trimmed
    to E; otherwise they keep e_cap rows and n_edges is None.
    """
    lib = load()
    dev = nbr.device
    n, sel = nbr.shape
    _need(nbr, "nbr", torch.int32, (n, sel), dev)
    _need(nbr_shift, "nbr_shift", torch.int32, (n, sel, 3), dev)
    if nnei is not None:
        _need(nnei, "nnei", torch.int32, (n,), dev)
    if e_cap is None:
        e_cap = n * sel
    o = dict(out or {})
    if "row_ptr" not in o:
        o["row_ptr"] = torch.empty((n + 1,), dtype=torch.int64, device=dev)
    if "col" not in o:
        o["col"] = torch.empty((e_cap,), dtype=torch.int32, device=dev)
    if "shift" not in o:
        o["shift"] = torch.empty((e_cap, 3), dtype=torch.int32, device=dev)
    if want_dst and "dst" not in o:
        o["dst"] = torch.empty((e_cap,), dtype=torch.int32, device=dev)
    if want_edge_vec and "edge_vec" not in o:
        o["edge_vec"] = torch.empty((e_cap, 3), dtype=torch.float64, device=dev)
    _need(o["row_ptr"], "row_ptr", torch.int64, (n + 1,), dev)
    _need(o["col"], "col", torch.int32, (e_cap,), dev)
    _need(o["shift"], "shift", torch.int32, (e_cap, 3), dev)
    dst = o.get("dst") if want_dst else None
    ev = o.get("edge_vec") if want_edge_vec else None
    if dst is not None:
        _need(dst, "dst", torch.int32, (e_cap,), dev)
    boxp = None
    if ev is not None:
        _need(ev, "edge_vec", torch.float64, (e_cap, 3), dev)
        _need(pos, "pos", torch.float64, (n, 3), dev)
        boxp = _box3(box)
    ws = _ws(ws, dev, int(lib.edge_csr_workspace_bytes(n, sel)))
    ne = ctypes.c_int64(-1)
    rc = lib.edge_csr(_ptr(nbr), _ptr(nbr_shift), _ptr(nnei), n, sel,
                      _ptr(pos) if ev is not None else None, boxp, _ptr(o["row_ptr"]),
                      _ptr(o["col"]), _ptr(o["shift"]), _ptr(dst), _ptr(ev), int(e_cap),
                      ctypes.byref(ne) if read_n_edges else None, ws.ptr(), ws.nbytes, _stream(dev))
    _check(rc, "edge_csr")
    res = {"row_ptr": o["row_ptr"], "col": o["col"], "shift": o["shift"], "dst": dst,
           "edge_vec": ev, "n_edges": None, "ws": ws}
    if read_n_edges:
        e = int(ne.value)
        res["n_edges"] = e
        for k in ("col", "shift", "dst", "edge_vec"):
            if res[k] is not None:
                res[k] = res[k][:e]
    return res


def _attn_dtype(t: torch.Tensor, split16: bool = False) -> int:
    if t.dtype == torch.float64:
        if split16:
            raise TypeError("split16 applies to float32 features only")
        return NGA_F64
    if t.dtype == torch.float32:
        return NGA_F32_SPLIT16 if split16 else NGA_F32
    raise TypeError(f"attention features must be float64 or float32, got {t.dtype}")


def block_attn_workspace_bytes(dtype: int, n_edges: int, nnei_cap: int, c: int, n_heads: int,
                               n_layers: int) -> int:
    return int(load().block_attn_workspace_bytes(dtype, n_edges, nnei_cap, c, n_heads, n_layers))


def attn_variant(dtype: int, nnei_cap: int, c: int, n_heads: int) -> str:
    return load().nga_attn_variant(dtype, nnei_cap, c, n_heads).decode()


def attn_plan(dtype: int, n_centres: int, nnei_cap: int, c: int, n_heads: int) -> str:
    """nga_attn_plan: the variant name, with the fp64 matrix-core path's layer plan for this
    many centres on the current device ("mfma_f64.merged" or "mfma_f64.per_head")."""
    return load().nga_attn_plan(dtype, int(n_centres), nnei_cap, c, n_heads).decode()


def block_attn_forward(row_ptr: torch.Tensor, x: torch.Tensor, weights: torch.Tensor,
                       n_heads: int, nnei_cap: int, *, order: torch.Tensor | None = None,
                       y: torch.Tensor | None = None, ws: Workspace | None = None,
                       log_dtilde: torch.Tensor | None = None, split16: bool = False):
    """Stacked block-dense attention layers; returns y [E][c] (same dtype as x).  With
    log_dtilde ([layers][E][n_heads], ln D~ per query edge and head) the smooth form,
    block_attn_forward_smooth, runs instead.  split16 (float32 only) asks for the
    NGA_F32_SPLIT16 arithmetic: contractions on f16 hi/lo pairs instead of fp32."""
    lib = load()
    dev = x.device
    e, c = x.shape
    dt = _attn_dtype(x, split16)
    n_centres = row_ptr.shape[0] - 1
    _need(row_ptr, "row_ptr", torch.int64, (n_centres + 1,), dev)
    if weights.dim() != 4:
        raise ValueError("weights must be [layers][4][c][c]")
    layers = weights.shape[0]
    _need(weights, "weights", x.dtype, (layers, 4, c, c), dev)
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    if order is not None:
        if order.dim() != 1 or order.dtype != torch.int32 or order.device != dev or \
                not order.is_contiguous():
            raise ValueError("order must be a contiguous int32 vector on the device")
    if y is None:
        y = torch.empty_like(x)
    _need(y, "y", x.dtype, (e, c), dev)
    ws = _ws(ws, dev, block_attn_workspace_bytes(dt, e, nnei_cap, c, n_heads, layers))
    if log_dtilde is None:
        rc = lib.block_attn_forward(dt, _ptr(row_ptr), _ptr(order), n_centres, e, int(nnei_cap),
                                    c, int(n_heads), int(layers), _ptr(weights), _ptr(x), _ptr(y),
                                    ws.ptr(), ws.nbytes, _stream(dev))
        _check(rc, "block_attn_forward")
    else:
        _need(log_dtilde, "log_dtilde", x.dtype, (layers, e, int(n_heads)), dev)
        rc = lib.block_attn_forward_smooth(dt, _ptr(row_ptr), _ptr(order), n_centres, e,
                                           int(nnei_cap), c, int(n_heads), int(layers),
                                           _ptr(weights), _ptr(x), _ptr(log_dtilde), _ptr(y),
                                           ws.ptr(), ws.nbytes, _stream(dev))
        _check(rc, "block_attn_forward_smooth")
    return y


def _copy_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float64:
        return NGA_F64
    if t.dtype == torch.float32:
        return NGA_F32
    raise TypeError(f"features must be float64 or float32, got {t.dtype}")


def block_gather(row_ptr: torch.Tensor, x: torch.Tensor, nnei_cap: int, *,
                 order: torch.Tensor | None = None, block: torch.Tensor | None = None,
                 ws: Workspace | None = None):
    """The padded per-centre block [n_centres][nnei_cap][c] of x's rows (zeros past each
    centre's row count)."""
    lib = load()
    dev = x.device
    e, c = x.shape
    n_centres = row_ptr.shape[0] - 1
    _need(row_ptr, "row_ptr", torch.int64, (n_centres + 1,), dev)
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    if order is not None:
        _need(order, "order", torch.int32, (order.shape[0],), dev)
    if block is None:
        block = torch.empty((n_centres, int(nnei_cap), c), dtype=x.dtype, device=dev)
    _need(block, "block", x.dtype, (n_centres, int(nnei_cap), c), dev)
    ws = _ws(ws, dev, 256)
    rc = lib.block_gather(_copy_dtype(x), _ptr(row_ptr), _ptr(order), n_centres, e,
                          int(nnei_cap), c, _ptr(x), _ptr(block), ws.ptr(), ws.nbytes,
                          _stream(dev))
    _check(rc, "block_gather")
    return block


def block_scatter(row_ptr: torch.Tensor, block: torch.Tensor, y: torch.Tensor, *,
                  order: torch.Tensor | None = None, ws: Workspace | None = None):
    """Write the valid rows of block [n_centres][cap][c] back into y [E][c] (in place)."""
    lib = load()
    dev = y.device
    e, c = y.shape
    n_centres, cap = block.shape[0], block.shape[1]
    _need(row_ptr, "row_ptr", torch.int64, (n_centres + 1,), dev)
    _need(block, "block", y.dtype, (n_centres, cap, c), dev)
    if not y.is_contiguous():
        raise ValueError("y must be contiguous")
    if order is not None:
        _need(order, "order", torch.int32, (order.shape[0],), dev)
    ws = _ws(ws, dev, 256)
    rc = lib.block_scatter(_copy_dtype(y), _ptr(row_ptr), _ptr(order), n_centres, e, cap, c,
                           _ptr(block), _ptr(y), ws.ptr(), ws.nbytes, _stream(dev))
    _check(rc, "block_scatter")
    return y


DEFAULT_PAIR_CHUNK = 1 << 24


def pair_attn_workspace_bytes(dtype: int, n_centres: int, n_edges: int, c: int, n_heads: int,
                              n_layers: int, pair_chunk: int = DEFAULT_PAIR_CHUNK) -> int:
    return int(load().pair_attn_workspace_bytes(dtype, n_centres, n_edges, c, n_heads, n_layers,
                                                int(pair_chunk)))


def pair_attn_forward(row_ptr: torch.Tensor, x: torch.Tensor, weights: torch.Tensor,
                      n_heads: int, *, order: torch.Tensor | None = None,
                      pair_chunk: int = DEFAULT_PAIR_CHUNK, y: torch.Tensor | None = None,
                      ws: Workspace | None = None):
    """The same attention by the ragged pair-axis route (chunks of at most pair_chunk pairs);
    returns y [E][c].  Synchronises the current stream once (chunk planning)."""
    lib = load()
    dev = x.device
    e, c = x.shape
    dt = _attn_dtype(x)
    n_centres = row_ptr.shape[0] - 1
    _need(row_ptr, "row_ptr", torch.int64, (n_centres + 1,), dev)
    if weights.dim() != 4:
        raise ValueError("weights must be [layers][4][c][c]")
    layers = weights.shape[0]
    _need(weights, "weights", x.dtype, (layers, 4, c, c), dev)
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    if order is not None:
        if order.dim() != 1 or order.dtype != torch.int32 or order.device != dev or \
                not order.is_contiguous():
            raise ValueError("order must be a contiguous int32 vector on the device")
    if y is None:
        y = torch.empty_like(x)
    _need(y, "y", x.dtype, (e, c), dev)
    ws = _ws(ws, dev, pair_attn_workspace_bytes(dt, n_centres, e, c, n_heads, layers, pair_chunk))
    rc = lib.pair_attn_forward(dt, _ptr(row_ptr), _ptr(order), n_centres, e, c, int(n_heads),
                               int(layers), _ptr(weights), _ptr(x), _ptr(y), int(pair_chunk),
                               ws.ptr(), ws.nbytes, _stream(dev))
    _check(rc, "pair_attn_forward")
    return y


def local_attn_forward(row_ptr: torch.Tensor, xc: torch.Tensor, x: torch.Tensor,
                       weights: torch.Tensor, n_heads: int, *, order: torch.Tensor | None = None,
                       yc: torch.Tensor | None = None, ws: Workspace | None = None):
    """LocalAtten: one query per centre (xc [N][c]) over its edges (x [E][c]); returns
    yc [N][c]."""
    lib = load()
    dev = x.device
    e, c = x.shape
    dt = _attn_dtype(x)
    n_centres = row_ptr.shape[0] - 1
    _need(row_ptr, "row_ptr", torch.int64, (n_centres + 1,), dev)
    _need(xc, "xc", x.dtype, (n_centres, c), dev)
    if weights.dim() != 4:
        raise ValueError("weights must be [layers][4][c][c]")
    layers = weights.shape[0]
    _need(weights, "weights", x.dtype, (layers, 4, c, c), dev)
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    if order is not None:
        if order.dim() != 1 or order.dtype != torch.int32 or order.device != dev or \
                not order.is_contiguous():
            raise ValueError("order must be a contiguous int32 vector on the device")
    if yc is None:
        yc = torch.empty_like(xc)
    _need(yc, "yc", x.dtype, (n_centres, c), dev)
    ws = _ws(ws, dev, int(lib.local_attn_workspace_bytes(dt, n_centres, c, int(n_heads),
                                                         int(layers))))
    rc = lib.local_attn_forward(dt, _ptr(row_ptr), _ptr(order), n_centres, e, c, int(n_heads),
                                int(layers), _ptr(weights), _ptr(xc), _ptr(x), _ptr(yc),
                                ws.ptr(), ws.nbytes, _stream(dev))
    _check(rc, "local_attn_forward")
    return yc


class StepGraph:
    """One step (nl_build, edge_csr without readback, block_attn_forward) captured as a HIP
    graph over fixed buffers; replay() launches it on the current stream.  The buffers are
    allocated here and exposed as attributes: pos (update in place between replays), nbr,
    nbr_shift, nnei, row_ptr, col, shift, dst, x, weights and y."""

    def __init__(self, pos: torch.Tensor, box, rcut: float, sel: int, x: torch.Tensor,
                 weights: torch.Tensor, n_heads: int):
        lib = load()
        dev = pos.device
        n = pos.shape[0]
        _need(pos, "pos", torch.float64, (n, 3), dev)
        e_cap = n * int(sel)
        c = x.shape[1]
        _need(x, "x", x.dtype, (e_cap, c), dev)
        layers = weights.shape[0]
        _need(weights, "weights", x.dtype, (layers, 4, c, c), dev)
        dt = _attn_dtype(x)
        self.pos, self.x, self.weights = pos, x, weights
        self.box = _box3(box)
        i32 = dict(dtype=torch.int32, device=dev)
        self.nbr = torch.empty((n, sel), **i32)
        self.nbr_shift = torch.empty((n, sel, 3), **i32)
        self.nnei = torch.empty((n,), **i32)
        self.row_ptr = torch.empty((n + 1,), dtype=torch.int64, device=dev)
        self.col = torch.empty((e_cap,), **i32)
        self.shift = torch.empty((e_cap, 3), **i32)
        self.dst = torch.empty((e_cap,), **i32)
        self.y = torch.empty_like(x)
        self.ws_nl = Workspace(dev, nl_build_workspace_bytes(n, box, rcut))
        self.ws_csr = Workspace(dev, int(lib.edge_csr_workspace_bytes(n, int(sel))))
        self.ws_attn = Workspace(dev, block_attn_workspace_bytes(dt, e_cap, sel, c, n_heads,
                                                                 layers))
        handle = ctypes.c_void_p()
        rc = lib.nga_step_graph_create(
            _ptr(pos), n, self.box, float(rcut), int(sel), _ptr(self.nbr), _ptr(self.nbr_shift),
            _ptr(self.nnei), self.ws_nl.ptr(), self.ws_nl.nbytes, _ptr(self.row_ptr),
            _ptr(self.col), _ptr(self.shift), _ptr(self.dst), None, e_cap, self.ws_csr.ptr(),
            self.ws_csr.nbytes, dt, c, int(n_heads), int(layers), _ptr(weights), _ptr(x),
            _ptr(self.y), self.ws_attn.ptr(), self.ws_attn.nbytes, ctypes.byref(handle))
        _check(rc, "nga_step_graph_create")
        self._lib, self._handle, self._dev = lib, handle, dev

    def replay(self) -> None:
        _check(self._lib.nga_step_graph_launch(self._handle, _stream(self._dev)),
               "nga_step_graph_launch")

    def check(self) -> None:
        """Synchronise and raise on any device-detected error of the replays so far."""
        for ws, name in ((self.ws_nl, "nl_build"), (self.ws_csr, "edge_csr"),
                         (self.ws_attn, "block_attn_forward")):
            check_status(ws, name)

    def __del__(self):
        if getattr(self, "_handle", None):
            self._lib.nga_step_graph_destroy(self._handle)
            self._handle = None


def nl_refine(pos: torch.Tensor, box, rcut: float, sel: int, cand_nbr: torch.Tensor,
              cand_shift: torch.Tensor, cand_nnei: torch.Tensor | None, cand_box, *, nbr=None,
              nbr_shift=None, nnei=None, ws: Workspace | None = None):
    """Neighbour rows at pos from candidate rows built by nl_build with rcut + skin in the box
    cand_box; returns (nbr [N][sel], nbr_shift [N][sel][3], nnei [N])."""
    lib = load()
    dev = pos.device
    n = pos.shape[0]
    _need(pos, "pos", torch.float64, (n, 3), dev)
    csel = cand_nbr.shape[1] if cand_nbr.dim() == 2 else -1
    _need(cand_nbr, "cand_nbr", torch.int32, (n, csel), dev)
    _need(cand_shift, "cand_shift", torch.int32, (n, csel, 3), dev)
    if cand_nnei is not None:
        _need(cand_nnei, "cand_nnei", torch.int32, (n,), dev)
    i32 = dict(dtype=torch.int32, device=dev)
    nbr = torch.empty((n, sel), **i32) if nbr is None else nbr
    nbr_shift = torch.empty((n, sel, 3), **i32) if nbr_shift is None else nbr_shift
    nnei = torch.empty((n,), **i32) if nnei is None else nnei
    _need(nbr, "nbr", torch.int32, (n, sel), dev)
    _need(nbr_shift, "nbr_shift", torch.int32, (n, sel, 3), dev)
    _need(nnei, "nnei", torch.int32, (n,), dev)
    ws = _ws(ws, dev, 256)
    rc = lib.nl_refine(_ptr(pos), n, _box3(box), float(rcut), int(sel), _ptr(cand_nbr),
                       _ptr(cand_shift), _ptr(cand_nnei), int(csel), _box3(cand_box), _ptr(nbr),
                       _ptr(nbr_shift), _ptr(nnei), ws.ptr(), ws.nbytes, _stream(dev))
    _check(rc, "nl_refine")
    return nbr, nbr_shift, nnei


def nl_max_displacement(pos: torch.Tensor, pos_ref: torch.Tensor, box,
                        out: torch.Tensor | None = None) -> torch.Tensor:
    """Largest plain (not minimum-image) displacement |pos - pos_ref| over the atoms, as a
    1-element device tensor (no synchronisation); a re-wrapped atom reads as about one box
    length."""
    lib = load()
    dev = pos.device
    n = pos.shape[0]
    _need(pos, "pos", torch.float64, (n, 3), dev)
    _need(pos_ref, "pos_ref", torch.float64, (n, 3), dev)
    out = torch.empty((1,), dtype=torch.float64, device=dev) if out is None else out
    _need(out, "out", torch.float64, (1,), dev)
    _check(lib.nl_max_displacement(_ptr(pos), _ptr(pos_ref), n, _box3(box), _ptr(out),
                                   _stream(dev)), "nl_max_displacement")
    return out


def nl_build_batch(pos: torch.Tensor, atom_ptr, boxes, rcut: float, sel: int, *, nbr=None,
                   nbr_shift=None, nnei=None, ws: Workspace | None = None):
    """Neighbour rows of several structures: pos [N][3] concatenated, atom_ptr [B+1] (host
    sequence), boxes [B][3] (host).  Returns (nbr [N][sel], nbr_shift [N][sel][3], nnei [N])
    with indices into the concatenated arrays."""
    lib = load()
    dev = pos.device
    ap = (ctypes.c_int64 * len(atom_ptr))(*[int(v) for v in atom_ptr])
    flat = [float(v) for b in boxes for v in b]
    bx = (ctypes.c_double * len(flat))(*flat)
    nstruct = len(atom_ptr) - 1
    if len(flat) != 3 * nstruct:
        raise ValueError("boxes must be [len(atom_ptr) - 1][3]")
    n = int(atom_ptr[-1])
    _need(pos, "pos", torch.float64, (n, 3), dev)
    i32 = dict(dtype=torch.int32, device=dev)
    nbr = torch.empty((n, sel), **i32) if nbr is None else nbr
    nbr_shift = torch.empty((n, sel, 3), **i32) if nbr_shift is None else nbr_shift
    nnei = torch.empty((n,), **i32) if nnei is None else nnei
    need = int(lib.nl_build_batch_workspace_bytes(nstruct, ap, bx, float(rcut)))
    if need == 0:
        raise NGAError(NGA_EINVAL, "nl_build_batch")
    ws = _ws(ws, dev, need)
    rc = lib.nl_build_batch(_ptr(pos), nstruct, ap, bx, float(rcut), int(sel), _ptr(nbr),
                            _ptr(nbr_shift), _ptr(nnei), ws.ptr(), ws.nbytes, _stream(dev))
    _check(rc, "nl_build_batch")
    return nbr, nbr_shift, nnei
