"""Plain CPU oracle for the MATE token-mixing core (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It wraps ``mate_oracle.c`` (plain C,
double precision, explicit loops) through ctypes and shares nothing with the
HIP library in ``linear_complexity_video_amd``.

Functions take numpy arrays (float32 for tensors, laid out channels-last as
``[batch][T][H][W][...]``) and return float64 results.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mate_oracle.c")
_LIB = os.path.join(_HERE, "libmate_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2; no fast-math, no vector intrinsics)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    i64, i32, p = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.oracle_rms_sequence.argtypes = [i64, i64, i64, i32, i32, p]
    lib.oracle_rms_reorder.argtypes = [p, p, i64, i64, i64, i64, i64, i32, i32, i32]
    lib.oracle_review_pool.argtypes = [p, i64, i64, i64, i64, i32, i32, i32, i32, p]
    lib.oracle_bissd.argtypes = [p, p, p, p, p, p, i64, i64, i64, i64] + [i32] * 11 + [p]
    lib.oracle_bissd_backward.argtypes = [p, p, p, p, p, p, p, i64, i64, i64, i64] + [i32] * 11 + [p] * 6
    lib.oracle_biscan1.argtypes = [p, p, p, p, p, p, i64, i64, i64, i64] + [i32] * 9 + [p]
    lib.oracle_tesa_region_counts.argtypes = [i64, i64, i64] + [i32] * 6 + [p]
    lib.oracle_tesa.argtypes = (
        [p, p, p, i64, i64, i64, i64] + [i32] * 8 + [ctypes.c_double, i32, i32, p, i64, i32, p]
    )
    lib.oracle_tesa_backward.argtypes = (
        [p, p, p, p, i64, i64, i64, i64] + [i32] * 8 + [ctypes.c_double, i32, i32, p, i64, i32, p, p, p]
    )
    for f in ("oracle_rms_sequence", "oracle_rms_reorder", "oracle_review_pool", "oracle_bissd", "oracle_bissd_backward",
              "oracle_biscan1", "oracle_tesa_region_counts", "oracle_tesa", "oracle_tesa_backward"):
        getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


ORACLE_EINVAL, ORACLE_ENOMEM = -1, -2


def _check(rc: int, what: str):
    if rc == ORACLE_ENOMEM:
        raise MemoryError(f"oracle {what} could not allocate its scratch memory")
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (code {rc})")


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def rms_sequence(T: int, H: int, W: int, order: int, flip: bool = False) -> np.ndarray:
    """Scan position -> canonical token index for RMS order ``order``."""
    seq = np.empty(T * H * W, dtype=np.int64)
    _check(_load().oracle_rms_sequence(T, H, W, order, int(flip), _ptr(seq)), "rms_sequence")
    return seq


def rms_reorder(src: np.ndarray, T: int, H: int, W: int, order: int, flip: bool, inverse: bool) -> np.ndarray:
    """Whole-row permutation of ``src`` viewed as [batch][N][row bytes]."""
    src = np.ascontiguousarray(src)
    N = T * H * W
    batch = src.shape[0]
    row_bytes = src.nbytes // (batch * N)
    dst = np.empty_like(src)
    _check(_load().oracle_rms_reorder(_ptr(src), _ptr(dst), batch, T, H, W, row_bytes, order,
                                      int(flip), int(inverse)), "rms_reorder")
    return dst


def review_pool(src: np.ndarray, T: int, H: int, W: int, pool, order: int) -> np.ndarray:
    """Average-pool one batch element ([T][H][W][C] float32) and unroll in ``order``."""
    src = _f32(src)
    C = src.size // (T * H * W)
    pt, ph, pw = pool
    R = (T // pt) * (H // ph) * (W // pw)
    out = np.empty((R, C), dtype=np.float64)
    _check(_load().oracle_review_pool(_ptr(src), T, H, W, C, pt, ph, pw, order, _ptr(out)), "review_pool")
    return out


def bissd(x, B, C, dt, A, D, grid, order: int, pool=(0, 0, 0), heads=None, nthreads=None) -> np.ndarray:
    """Bidirectional Mamba2 scan; returns y[b][T][H][W][nh][P] (float64) for ``heads``.

    x [b][T][H][W][nheads][P], B/C [b][T][H][W][G][S], dt [b][T][H][W][nheads],
    A/D [nheads]. ``heads`` is a (lo, hi) range, default all heads.
    """
    batch, T, H, W = grid
    x, B, C, dt, A, D = (_f32(a) for a in (x, B, C, dt, A, D))
    nheads, P = x.shape[-2], x.shape[-1]
    G, S = B.shape[-2], B.shape[-1]
    lo, hi = heads if heads is not None else (0, nheads)
    y = np.full((batch, T, H, W, hi - lo, P), np.nan, dtype=np.float64)
    rc = _load().oracle_bissd(_ptr(x), _ptr(B), _ptr(C), _ptr(dt), _ptr(A), _ptr(D), batch, T, H, W,
                              nheads, P, S, G, order, pool[0], pool[1], pool[2], lo, hi,
                              nthreads or default_threads(), _ptr(y))
    _check(rc, "bissd")
    return y


def bissd_backward(x, B, C, dt, A, D, dy, grid, order: int, pool=(0, 0, 0), heads=None, nthreads=None) -> dict:
    """Gradients of ``bissd`` for the upstream gradient ``dy`` (same layout as y), float64:
    dx [b][T][H][W][nh][P], dB and dC [b][T][H][W][G][S] (summed over the heads in ``heads`` only),
    ddt [b][T][H][W][nh], dA and dD [nh] (summed over the batch); ``heads`` is a (lo, hi) range."""
    batch, T, H, W = grid
    x, B, C, dt, A, D, dy = (_f32(a) for a in (x, B, C, dt, A, D, dy))
    nheads, P = x.shape[-2], x.shape[-1]
    G, S = B.shape[-2], B.shape[-1]
    assert dy.shape == x.shape
    lo, hi = heads if heads is not None else (0, nheads)
    nh = hi - lo
    out = {"dx": np.full((batch, T, H, W, nh, P), np.nan), "dB": np.full((batch, T, H, W, G, S), np.nan),
           "dC": np.full((batch, T, H, W, G, S), np.nan), "ddt": np.full((batch, T, H, W, nh), np.nan),
           "dA": np.full(nh, np.nan), "dD": np.full(nh, np.nan)}
    rc = _load().oracle_bissd_backward(_ptr(x), _ptr(B), _ptr(C), _ptr(dt), _ptr(A), _ptr(D), _ptr(dy), batch, T, H,
                                       W, nheads, P, S, G, order, pool[0], pool[1], pool[2], lo, hi,
                                       nthreads or default_threads(),
                                       *(_ptr(out[k]) for k in ("dx", "dB", "dC", "ddt", "dA", "dD")))
    _check(rc, "bissd_backward")
    return out


def biscan1(x, B, C, dt, A, D, grid, order: int, pool=(0, 0, 0), channels=None, nthreads=None) -> np.ndarray:
    """Bidirectional Mamba (selective scan); returns y[b][T][H][W][nc] (float64) for ``channels``.

    x, dt [b][T][H][W][nch], B/C [b][T][H][W][S], A [nch][S], D [nch]. ``channels`` is a (lo, hi)
    range, default all channels.
    """
    batch, T, H, W = grid
    x, B, C, dt, A, D = (_f32(a) for a in (x, B, C, dt, A, D))
    nch, S = x.shape[-1], B.shape[-1]
    assert A.shape == (nch, S) and dt.shape[-1] == nch and D.shape == (nch,)
    lo, hi = channels if channels is not None else (0, nch)
    y = np.full((batch, T, H, W, hi - lo), np.nan, dtype=np.float64)
    rc = _load().oracle_biscan1(_ptr(x), _ptr(B), _ptr(C), _ptr(dt), _ptr(A), _ptr(D), batch, T, H, W,
                                nch, S, order, pool[0], pool[1], pool[2], lo, hi,
                                nthreads or default_threads(), _ptr(y))
    _check(rc, "biscan1")
    return y


def tesa_region_counts(T, H, W, window, shift):
    out = np.empty(3, dtype=np.int64)
    _check(_load().oracle_tesa_region_counts(T, H, W, *window, *shift, _ptr(out)), "tesa_region_counts")
    return tuple(int(v) for v in out)


def tesa(q, k, v, grid, window, shift=(0, 0, 0), scale: float = 0.0, heads=None, regions=None,
         nthreads=None) -> np.ndarray:
    """Shifted-window attention; returns o[b][T][H][W][nh][d] (float64).

    With ``regions`` (list of linear region ids) only those regions' tokens are
    written; the rest of the result is NaN.
    """
    batch, T, H, W = grid
    q, k, v = _f32(q), _f32(k), _f32(v)
    nheads, d = q.shape[-2], q.shape[-1]
    lo, hi = heads if heads is not None else (0, nheads)
    o = np.full((batch, T, H, W, hi - lo, d), np.nan, dtype=np.float64)
    if regions is None:
        rp, nr = None, 0
    else:
        reg = np.ascontiguousarray(regions, dtype=np.int64)
        rp, nr = _ptr(reg), reg.size
    rc = _load().oracle_tesa(_ptr(q), _ptr(k), _ptr(v), batch, T, H, W, nheads, d, *window, *shift,
                             float(scale), lo, hi, rp, nr, nthreads or default_threads(), _ptr(o))
    _check(rc, "tesa")
    return o


def tesa_backward(q, k, v, dout, grid, window, shift=(0, 0, 0), scale: float = 0.0, heads=None, regions=None,
                  nthreads=None):
    """Gradients (dq, dk, dv) of shifted-window attention for the upstream gradient ``dout``;
    each [b][T][H][W][nh][d] (float64). With ``regions`` only those regions' tokens are
    written; the rest is NaN."""
    batch, T, H, W = grid
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    nheads, d = q.shape[-2], q.shape[-1]
    lo, hi = heads if heads is not None else (0, nheads)
    out = [np.full((batch, T, H, W, hi - lo, d), np.nan, dtype=np.float64) for _ in range(3)]
    if regions is None:
        rp, nr = None, 0
    else:
        reg = np.ascontiguousarray(regions, dtype=np.int64)
        rp, nr = _ptr(reg), reg.size
    rc = _load().oracle_tesa_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), batch, T, H, W, nheads, d, *window,
                                      *shift, float(scale), lo, hi, rp, nr, nthreads or default_threads(),
                                      *(_ptr(a) for a in out))
    _check(rc, "tesa_backward")
    return tuple(out)
