"""ctypes binding of ``libmate.so`` (the C ABI in ``include/mate.h``).

Argument marshalling only: tensors are torch CUDA tensors (contiguous,
channels-last ``[batch][T][H][W][heads][dim]``); their data pointers and the
current HIP stream are passed to the C functions of the same names. Every step
of the computation runs in the library's HIP kernels; if the library is
missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmate.so")

MATE_OK, MATE_ERR_NULL, MATE_ERR_SHAPE, MATE_ERR_UNSUPPORTED, MATE_ERR_WORKSPACE, MATE_ERR_DEVICE = range(6)
MATE_F32, MATE_BF16 = 0, 1
ALGO_AUTO, ALGO_PORTABLE, ALGO_FAST = 0, 1, 2
ORDER_ZIGZAG = 4  # MATE_ORDER_ZIGZAG: the snake path; orders 0..3 are the RMS orders

EXPORTED = (
    "mate_rms_reorder", "mate_bissd_workspace_size", "mate_bissd_scan", "mate_tesa",
    "mate_forward_workspace_size", "mate_forward", "mate_status_string", "mate_last_error",
    "mate_abi_version", "mate_timing_begin", "mate_timing_end", "mate_bimamba_workspace_size",
    "mate_bimamba_scan", "mate_tesa_backward_workspace_size", "mate_tesa_backward", "mate_bissd_scan_noalloc",
    "mate_bissd_backward_workspace_size", "mate_bissd_backward", "mate_layer_workspace_size", "mate_layer",
)
STATIC_SCRATCH_BYTES = 64 << 20  # MATE_STATIC_SCRATCH_BYTES


class MateError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{detail} (status {status})")
        self.status = status
        self.detail = detail


class Grid(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int64), ("W", ctypes.c_int64)]


class SsdDesc(ctypes.Structure):
    _fields_ = [("nheads", ctypes.c_int32), ("headdim", ctypes.c_int32), ("d_state", ctypes.c_int32),
                ("ngroups", ctypes.c_int32), ("chunk", ctypes.c_int32), ("pool_t", ctypes.c_int32),
                ("pool_h", ctypes.c_int32), ("pool_w", ctypes.c_int32), ("dtype", ctypes.c_int),
                ("algo", ctypes.c_int)]


class SsdTensors(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("b", ctypes.c_void_p), ("c", ctypes.c_void_p), ("dt", ctypes.c_void_p),
                ("a", ctypes.c_void_p), ("d", ctypes.c_void_p), ("y", ctypes.c_void_p)]


class SsdGradTensors(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("x", "b", "c", "dt", "a", "d", "dy", "dx", "db", "dc", "ddt", "da",
                                                "dd")]


class MambaDesc(ctypes.Structure):
    _fields_ = [("channels", ctypes.c_int32), ("d_state", ctypes.c_int32), ("pool_t", ctypes.c_int32),
                ("pool_h", ctypes.c_int32), ("pool_w", ctypes.c_int32), ("dtype", ctypes.c_int)]


class TesaDesc(ctypes.Structure):
    _fields_ = [("nheads", ctypes.c_int32), ("headdim", ctypes.c_int32), ("win_t", ctypes.c_int32),
                ("win_h", ctypes.c_int32), ("win_w", ctypes.c_int32), ("shift_t", ctypes.c_int32),
                ("shift_h", ctypes.c_int32), ("shift_w", ctypes.c_int32), ("scale", ctypes.c_float),
                ("dtype", ctypes.c_int), ("algo", ctypes.c_int)]


class TesaTensors(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("o", ctypes.c_void_p)]


LAYER_WEIGHTS = ("w_x", "w_z", "w_b", "w_c", "w_dt", "w_ma_out", "dt_bias", "a", "d", "norm_w", "w_q", "w_k", "w_v",
                 "w_te_out")


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_WEIGHTS]


class LayerDesc(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("norm_eps", ctypes.c_float)]


class TesaGradTensors(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("q", "k", "v", "dout", "dq", "dk", "dv")]


_lib = None


def lib() -> ctypes.CDLL:
    """Loads the HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with linear_complexity_video_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.mate_rms_reorder.argtypes = [P, P, Grid, I64, I32, I32, I32, P]
    L.mate_bissd_workspace_size.argtypes = [Grid, ctypes.POINTER(SsdDesc)]
    L.mate_bissd_workspace_size.restype = SZ
    L.mate_bissd_scan.argtypes = [ctypes.POINTER(SsdTensors), Grid, I32, ctypes.POINTER(SsdDesc), P, SZ, P]
    L.mate_bissd_scan_noalloc.argtypes = [ctypes.POINTER(SsdTensors), Grid, I32, ctypes.POINTER(SsdDesc), P]
    L.mate_bissd_backward_workspace_size.argtypes = [Grid, ctypes.POINTER(SsdDesc)]
    L.mate_bissd_backward_workspace_size.restype = SZ
    L.mate_bissd_backward.argtypes = [ctypes.POINTER(SsdGradTensors), Grid, I32, ctypes.POINTER(SsdDesc), P, SZ, P]
    L.mate_tesa.argtypes = [ctypes.POINTER(TesaTensors), Grid, ctypes.POINTER(TesaDesc), P]
    L.mate_tesa_backward_workspace_size.argtypes = [Grid, ctypes.POINTER(TesaDesc)]
    L.mate_tesa_backward_workspace_size.restype = SZ
    L.mate_tesa_backward.argtypes = [ctypes.POINTER(TesaGradTensors), Grid, ctypes.POINTER(TesaDesc), P, SZ, P]
    L.mate_bimamba_workspace_size.argtypes = [Grid, ctypes.POINTER(MambaDesc)]
    L.mate_bimamba_workspace_size.restype = SZ
    L.mate_bimamba_scan.argtypes = [ctypes.POINTER(SsdTensors), Grid, I32, ctypes.POINTER(MambaDesc), P, SZ, P]
    L.mate_forward_workspace_size.argtypes = [Grid, ctypes.POINTER(SsdDesc), ctypes.POINTER(TesaDesc)]
    L.mate_forward_workspace_size.restype = SZ
    L.mate_forward.argtypes = [ctypes.POINTER(SsdTensors), ctypes.POINTER(SsdDesc), ctypes.POINTER(TesaTensors),
                               ctypes.POINTER(TesaDesc), Grid, I32, P, SZ, P]
    L.mate_layer_workspace_size.argtypes = [Grid, ctypes.POINTER(LayerDesc), ctypes.POINTER(SsdDesc),
                                            ctypes.POINTER(TesaDesc)]
    L.mate_layer_workspace_size.restype = SZ
    L.mate_layer.argtypes = [P, P, ctypes.POINTER(LayerWeights), ctypes.POINTER(LayerDesc), ctypes.POINTER(SsdDesc),
                             ctypes.POINTER(TesaDesc), Grid, I32, P, SZ, P]
    for f in ("mate_rms_reorder", "mate_bissd_scan", "mate_bissd_scan_noalloc", "mate_bissd_backward",
              "mate_bimamba_scan", "mate_tesa", "mate_tesa_backward", "mate_forward", "mate_layer"):
        getattr(L, f).restype = ctypes.c_int
    L.mate_status_string.argtypes = [ctypes.c_int]
    L.mate_status_string.restype = ctypes.c_char_p
    L.mate_last_error.restype = ctypes.c_char_p
    L.mate_abi_version.restype = ctypes.c_int
    L.mate_timing_begin.argtypes = [ctypes.c_char_p]
    L.mate_timing_begin.restype = ctypes.c_int
    L.mate_timing_end.argtypes = [ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double)]
    L.mate_timing_end.restype = ctypes.c_int
    _lib = L
    return L


def _check(status: int):
    if status != MATE_OK:
        raise MateError(status, lib().mate_last_error().decode())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _dtype(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return MATE_F32
    if t.dtype == torch.bfloat16:
        return MATE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16 expected")


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _dev(*ts):
    for t in ts:
        _need(t.is_cuda and t.is_contiguous(), "tensors must be contiguous device tensors")


# Shape and dtype checks of every wrapper. The C ABI receives raw pointers and
# cannot see extents, so a tensor smaller than its descriptor says would be
# read or written past its end on the device; these checks run before any
# pointer leaves Python.

def _shape(t, shape, name):
    _need(tuple(t.shape) == tuple(shape), f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _is_f32(t, name):
    import torch
    _need(t.dtype == torch.float32, f"{name} must be float32, got {t.dtype}")


def _same_dtype(ref, name_ref, **ts):
    for n, t in ts.items():
        _need(t.dtype == ref.dtype, f"{n} has dtype {t.dtype}, expected {ref.dtype} (the dtype of {name_ref})")


def _check_ssd_tensors(x, b, c, dt, a, d, y):
    """x, y [batch][T][H][W][nheads][headdim]; b, c [batch][T][H][W][ngroups][d_state] in x's dtype;
    dt float32 [batch][T][H][W][nheads]; a, d float32 [nheads]."""
    _need(x.dim() == 6, f"x must be [batch][T][H][W][nheads][headdim], got {x.dim()} dims")
    _dtype(x)
    grid, nh = tuple(x.shape[:4]), x.shape[4]
    _shape(y, x.shape, "y")
    _need(b.dim() == 6 and tuple(b.shape[:4]) == grid, f"b must be [{grid}][ngroups][d_state], got {tuple(b.shape)}")
    _shape(c, b.shape, "c")
    _same_dtype(x, "x", y=y, b=b, c=c)
    _shape(dt, grid + (nh,), "dt")
    _shape(a, (nh,), "a")
    _shape(d, (nh,), "d")
    for n, t in (("dt", dt), ("a", a), ("d", d)):
        _is_f32(t, n)


def _check_mamba_tensors(x, b, c, dt, a, d, y):
    """x, y [batch][T][H][W][channels]; b, c [batch][T][H][W][d_state] in x's dtype;
    dt float32 [batch][T][H][W][channels]; a float32 [channels][d_state]; d float32 [channels]."""
    _need(x.dim() == 5, f"x must be [batch][T][H][W][channels], got {x.dim()} dims")
    _dtype(x)
    grid, nch = tuple(x.shape[:4]), x.shape[4]
    _shape(y, x.shape, "y")
    _need(b.dim() == 5 and tuple(b.shape[:4]) == grid, f"b must be [{grid}][d_state], got {tuple(b.shape)}")
    _shape(c, b.shape, "c")
    _same_dtype(x, "x", y=y, b=b, c=c)
    _shape(dt, x.shape, "dt")
    _shape(a, (nch, b.shape[4]), "a")
    _shape(d, (nch,), "d")
    for n, t in (("dt", dt), ("a", a), ("d", d)):
        _is_f32(t, n)


def _check_token_tensors(ref_name, ref, **ts):
    """Attention tensors: all [batch][T][H][W][nheads][headdim] of one shape and dtype."""
    _need(ref.dim() == 6, f"{ref_name} must be [batch][T][H][W][nheads][headdim], got {ref.dim()} dims")
    _dtype(ref)
    for n, t in ts.items():
        _shape(t, ref.shape, n)
    _same_dtype(ref, ref_name, **ts)


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def grid_of(t) -> Grid:
    """Grid of a [batch][T][H][W][...] tensor."""
    return Grid(*t.shape[:4])


# ---------------------------------------------------------------------------
# Rotary Major Scan
# ---------------------------------------------------------------------------

def mate_rms_reorder(src, dst, grid, order: int, flip: bool = False, inverse: bool = False, stream=None):
    """Row permutation src -> dst in RMS ``order`` (see include/mate.h)."""
    _dev(src, dst)
    g = Grid(*grid)
    rows = g.batch * g.T * g.H * g.W
    nbytes = src.numel() * src.element_size()
    _need(nbytes == dst.numel() * dst.element_size() and nbytes % rows == 0, "src/dst size mismatch with grid")
    _check(lib().mate_rms_reorder(_ptr(src), _ptr(dst), g, nbytes // rows, order, int(flip), int(inverse),
                                  _stream(stream)))


# ---------------------------------------------------------------------------
# Bidirectional SSD scan
# ---------------------------------------------------------------------------

def ssd_desc(x, b, chunk: int, pool=(0, 0, 0), algo: int = ALGO_AUTO) -> SsdDesc:
    return SsdDesc(x.shape[-2], x.shape[-1], b.shape[-1], b.shape[-2], chunk, pool[0], pool[1], pool[2],
                   _dtype(x), algo)


def mate_bissd_workspace_size(grid, desc: SsdDesc) -> int:
    return int(lib().mate_bissd_workspace_size(Grid(*grid), ctypes.byref(desc)))


def _workspace(nbytes: int, like):
    import torch
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=like.device)


def mate_bissd_scan(x, b, c, dt, a, d, y, order: int, chunk: int, pool=(0, 0, 0), algo: int = ALGO_AUTO,
                    workspace=None, stream=None):
    """y = bidirectional Mamba2 scan of x in RMS ``order`` (see include/mate.h)."""
    _check_ssd_tensors(x, b, c, dt, a, d, y)
    _dev(x, b, c, dt, a, d, y)
    grid = tuple(x.shape[:4])
    desc = ssd_desc(x, b, chunk, pool, algo)
    if workspace is None:
        workspace = _workspace(mate_bissd_workspace_size(grid, desc), x)
    t = SsdTensors(_ptr(x), _ptr(b), _ptr(c), _ptr(dt), _ptr(a), _ptr(d), _ptr(y))
    _check(lib().mate_bissd_scan(ctypes.byref(t), Grid(*grid), order, ctypes.byref(desc), _ptr(workspace),
                                 _nbytes(workspace), _stream(stream)))


def mate_bissd_scan_noalloc(x, b, c, dt, a, d, y, order: int, chunk: int, pool=(0, 0, 0), algo: int = ALGO_AUTO,
                            stream=None):
    """mate_bissd_scan on the library's static scratch: no workspace, nothing allocated (see include/mate.h)."""
    _check_ssd_tensors(x, b, c, dt, a, d, y)
    _dev(x, b, c, dt, a, d, y)
    desc = ssd_desc(x, b, chunk, pool, algo)
    t = SsdTensors(_ptr(x), _ptr(b), _ptr(c), _ptr(dt), _ptr(a), _ptr(d), _ptr(y))
    _check(lib().mate_bissd_scan_noalloc(ctypes.byref(t), grid_of(x), order, ctypes.byref(desc), _stream(stream)))


def mate_bissd_backward_workspace_size(grid, desc: SsdDesc) -> int:
    return int(lib().mate_bissd_backward_workspace_size(Grid(*grid), ctypes.byref(desc)))


def mate_bissd_backward(x, b, c, dt, a, d, dy, dx, db, dc, ddt, da, dd, order: int, pool=(0, 0, 0),
                        workspace=None, stream=None):
    """Gradients (dx, db, dc, ddt, da, dd) of mate_bissd_scan for the upstream gradient dy (see include/mate.h)."""
    _check_ssd_tensors(x, b, c, dt, a, d, dx)
    _shape(dy, x.shape, "dy")
    _shape(db, b.shape, "db")
    _shape(dc, b.shape, "dc")
    _shape(ddt, dt.shape, "ddt")
    _shape(da, a.shape, "da")
    _shape(dd, d.shape, "dd")
    _same_dtype(x, "x", dy=dy, db=db, dc=dc)
    for n, t in (("ddt", ddt), ("da", da), ("dd", dd)):
        _is_f32(t, n)
    _dev(x, b, c, dt, a, d, dy, dx, db, dc, ddt, da, dd)
    grid = tuple(x.shape[:4])
    desc = ssd_desc(x, b, 64, pool)
    if workspace is None:
        workspace = _workspace(mate_bissd_backward_workspace_size(grid, desc), x)
    t = SsdGradTensors(*(_ptr(v) for v in (x, b, c, dt, a, d, dy, dx, db, dc, ddt, da, dd)))
    _check(lib().mate_bissd_backward(ctypes.byref(t), Grid(*grid), order, ctypes.byref(desc), _ptr(workspace),
                                     _nbytes(workspace), _stream(stream)))


# ---------------------------------------------------------------------------
# Bidirectional Mamba (selective scan)
# ---------------------------------------------------------------------------

def mamba_desc(x, b, pool=(0, 0, 0)) -> MambaDesc:
    return MambaDesc(x.shape[-1], b.shape[-1], pool[0], pool[1], pool[2], _dtype(x))


def mate_bimamba_workspace_size(grid, desc: MambaDesc) -> int:
    return int(lib().mate_bimamba_workspace_size(Grid(*grid), ctypes.byref(desc)))


def mate_bimamba_scan(x, b, c, dt, a, d, y, order: int, pool=(0, 0, 0), workspace=None, stream=None):
    """y = bidirectional Mamba selective scan of x (channels last) in ``order`` (see include/mate.h)."""
    _check_mamba_tensors(x, b, c, dt, a, d, y)
    _dev(x, b, c, dt, a, d, y)
    grid = tuple(x.shape[:4])
    desc = mamba_desc(x, b, pool)
    if workspace is None:
        workspace = _workspace(mate_bimamba_workspace_size(grid, desc), x)
    t = SsdTensors(_ptr(x), _ptr(b), _ptr(c), _ptr(dt), _ptr(a), _ptr(d), _ptr(y))
    _check(lib().mate_bimamba_scan(ctypes.byref(t), Grid(*grid), order, ctypes.byref(desc), _ptr(workspace),
                                   _nbytes(workspace), _stream(stream)))


# ---------------------------------------------------------------------------
# TESA
# ---------------------------------------------------------------------------

def tesa_desc(q, window, shift=(0, 0, 0), scale: float = 0.0, algo: int = ALGO_AUTO) -> TesaDesc:
    return TesaDesc(q.shape[-2], q.shape[-1], window[0], window[1], window[2], shift[0], shift[1], shift[2],
                    scale, _dtype(q), algo)


def mate_tesa(q, k, v, o, window, shift=(0, 0, 0), scale: float = 0.0, algo: int = ALGO_AUTO, stream=None):
    """o = attention of q, k, v inside (shifted) 3D windows (see include/mate.h)."""
    _check_token_tensors("q", q, k=k, v=v, o=o)
    _dev(q, k, v, o)
    desc = tesa_desc(q, window, shift, scale, algo)
    t = TesaTensors(_ptr(q), _ptr(k), _ptr(v), _ptr(o))
    _check(lib().mate_tesa(ctypes.byref(t), grid_of(q), ctypes.byref(desc), _stream(stream)))


def mate_tesa_backward_workspace_size(grid, desc: TesaDesc) -> int:
    return int(lib().mate_tesa_backward_workspace_size(Grid(*grid), ctypes.byref(desc)))


def mate_tesa_backward(q, k, v, dout, dq, dk, dv, window, shift=(0, 0, 0), scale: float = 0.0, workspace=None,
                       stream=None):
    """(dq, dk, dv) of mate_tesa for the upstream gradient dout (see include/mate.h)."""
    _check_token_tensors("q", q, k=k, v=v, dout=dout, dq=dq, dk=dk, dv=dv)
    _dev(q, k, v, dout, dq, dk, dv)
    desc = tesa_desc(q, window, shift, scale)
    if workspace is None:
        workspace = _workspace(mate_tesa_backward_workspace_size(tuple(q.shape[:4]), desc), q)
    t = TesaGradTensors(*(_ptr(a) for a in (q, k, v, dout, dq, dk, dv)))
    _check(lib().mate_tesa_backward(ctypes.byref(t), grid_of(q), ctypes.byref(desc), _ptr(workspace),
                                    _nbytes(workspace), _stream(stream)))


# ---------------------------------------------------------------------------
# MATE core forward
# ---------------------------------------------------------------------------

def mate_forward_workspace_size(grid, sdesc: SsdDesc, tdesc: TesaDesc) -> int:
    return int(lib().mate_forward_workspace_size(Grid(*grid), ctypes.byref(sdesc), ctypes.byref(tdesc)))


def mate_forward(ssd: dict, tesa: dict, order: int, chunk: int, pool, window, shift, scale: float = 0.0,
                 algo: int = ALGO_AUTO, workspace=None, stream=None):
    """One layer's MATE core: ssd{x,b,c,dt,a,d,y} and tesa{q,k,v,o} (see include/mate.h)."""
    x = ssd["x"]
    _check_ssd_tensors(*(ssd[k] for k in ("x", "b", "c", "dt", "a", "d", "y")))
    _check_token_tensors("q", tesa["q"], k=tesa["k"], v=tesa["v"], o=tesa["o"])
    _need(tuple(tesa["q"].shape[:4]) == tuple(x.shape[:4]),
          f"the TESA tensors' grid {tuple(tesa['q'].shape[:4])} differs from the scan's {tuple(x.shape[:4])}")
    _dev(*ssd.values(), *tesa.values())
    grid = tuple(x.shape[:4])
    sdesc = ssd_desc(x, ssd["b"], chunk, pool, algo)
    tdesc = tesa_desc(tesa["q"], window, shift, scale, algo)
    if workspace is None:
        workspace = _workspace(mate_forward_workspace_size(grid, sdesc, tdesc), x)
    st = SsdTensors(*(_ptr(ssd[k]) for k in ("x", "b", "c", "dt", "a", "d", "y")))
    tt = TesaTensors(*(_ptr(tesa[k]) for k in ("q", "k", "v", "o")))
    _check(lib().mate_forward(ctypes.byref(st), ctypes.byref(sdesc), ctypes.byref(tt), ctypes.byref(tdesc),
                              Grid(*grid), order, _ptr(workspace), _nbytes(workspace), _stream(stream)))


# ---------------------------------------------------------------------------
# One MATE layer
# ---------------------------------------------------------------------------

def layer_descs(grid, d_model: int, ssd: dict, tesa: dict, norm_eps: float = 1e-5):
    """(LayerDesc, SsdDesc, TesaDesc) of a bf16 layer. ssd: nheads, headdim, d_state, ngroups, chunk, pool;
    tesa: nheads, headdim, window, shift (and optional scale)."""
    ld = LayerDesc(d_model, norm_eps)
    pool = ssd.get("pool", (0, 0, 0))
    sd = SsdDesc(ssd["nheads"], ssd["headdim"], ssd["d_state"], ssd.get("ngroups", 1), ssd["chunk"], pool[0],
                 pool[1], pool[2], MATE_BF16, ALGO_AUTO)
    win, sh = tesa["window"], tesa.get("shift", (0, 0, 0))
    td = TesaDesc(tesa["nheads"], tesa["headdim"], win[0], win[1], win[2], sh[0], sh[1], sh[2],
                  tesa.get("scale", 0.0), MATE_BF16, ALGO_AUTO)
    return ld, sd, td


def mate_layer_workspace_size(grid, ld: LayerDesc, sd: SsdDesc, td: TesaDesc) -> int:
    return int(lib().mate_layer_workspace_size(Grid(*grid), ctypes.byref(ld), ctypes.byref(sd), ctypes.byref(td)))


def _check_layer(h, out, w: dict, ld: LayerDesc, sd: SsdDesc, td: TesaDesc):
    import torch
    dm, inner, bc = ld.d_model, sd.nheads * sd.headdim, sd.ngroups * sd.d_state
    tin = td.nheads * td.headdim
    _need(h.dim() == 5 and h.shape[-1] == dm, f"h must be [batch][T][H][W][{dm}], got {tuple(h.shape)}")
    _shape(out, h.shape, "out")
    shapes = {"w_x": (dm, inner), "w_z": (dm, inner), "w_b": (dm, bc), "w_c": (dm, bc), "w_dt": (dm, sd.nheads),
              "w_ma_out": (inner, dm), "dt_bias": (sd.nheads,), "a": (sd.nheads,), "d": (sd.nheads,),
              "norm_w": (inner,), "w_q": (dm, tin), "w_k": (dm, tin), "w_v": (dm, tin), "w_te_out": (tin, dm)}
    for n, shp in shapes.items():
        _shape(w[n], shp, n)
        want = torch.float32 if n in ("dt_bias", "a", "d", "norm_w") else torch.bfloat16
        _need(w[n].dtype == want, f"{n} must be {want}, got {w[n].dtype}")
    _need(h.dtype == torch.bfloat16 and out.dtype == torch.bfloat16, "h and out must be bfloat16")
    _dev(h, out, *w.values())


def mate_layer(h, out, weights: dict, d_model: int, ssd: dict, tesa: dict, order: int, norm_eps: float = 1e-5,
               workspace=None, stream=None):
    """One MATE layer: out = MA(h) + TE(h) with their projections (see include/mate.h). weights holds the
    LAYER_WEIGHTS tensors; ssd and tesa the branch sizes as for layer_descs."""
    grid = tuple(h.shape[:4])
    ld, sd, td = layer_descs(grid, d_model, ssd, tesa, norm_eps)
    _check_layer(h, out, weights, ld, sd, td)
    if workspace is None:
        workspace = _workspace(mate_layer_workspace_size(grid, ld, sd, td), h)
    w = LayerWeights(*(_ptr(weights[n]) for n in LAYER_WEIGHTS))
    _check(lib().mate_layer(_ptr(h), _ptr(out), ctypes.byref(w), ctypes.byref(ld), ctypes.byref(sd),
                            ctypes.byref(td), Grid(*grid), order, _ptr(workspace), _nbytes(workspace),
                            _stream(stream)))


def mate_timing_begin(kernel: str):
    """Arms HIP event timing of every later launch of one library kernel."""
    status = lib().mate_timing_begin(kernel.encode())
    if status != MATE_OK:
        raise MateError(status, f"mate_timing_begin({kernel!r}) refused")


def mate_timing_end():
    """Disarms the timing; returns (launches, summed milliseconds)."""
    n, ms = ctypes.c_int64(0), ctypes.c_double(0.0)
    status = lib().mate_timing_end(ctypes.byref(n), ctypes.byref(ms))
    if status != MATE_OK:
        raise MateError(status, "mate_timing_end failed")
    return int(n.value), float(ms.value)
