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


def bf16_round(a) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even), returned as float64: the float32 value's low 16 bits
    are rounded away (finite inputs)."""
    u = np.asarray(a, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return u.view(np.float32).astype(np.float64)


def layer(h, w: dict, grid, order: int, ssd: dict, tesa_sizes: dict, norm_eps: float = 1e-5,
          storage=None, nthreads=None) -> np.ndarray:
    """One MATE layer in float64: returns out[b][T][H][W][d_model].

    The MATE block replaces a DiT layer's self-attention with the MA and TE
    branches (QbitAI article on LinGen, section "方法"); the projections and the
    MA branch's per-token steps around the scan are the Mamba2 block's, which
    the pages do not spell out (the reading stated with ``mate_layer`` in
    include/mate.h):
        x, z, B, C = h Wx, h Wz, h Wb, h Wc;  dt = softplus(h Wdt + dt_bias)
        y = bissd(x, B, C, dt, A, D);  g = y * silu(z), RMS-normalised per group
        of nheads*headdim/ngroups channels (eps), times norm_w
        q, k, v = h Wq, h Wk, h Wv;  o = tesa(q, k, v)
        out = g Wma_out + o Wte_out
    The products are numpy float64 matmuls; the scan and TESA are the oracle's
    own (they take their inputs as float32, a rounding of 2^-24 relative).
    ``w`` maps the names of mate_layer_weights to arrays; ``ssd`` holds nheads,
    headdim, d_state, ngroups, pool; ``tesa_sizes`` nheads, headdim, window,
    shift and optionally scale. With ``storage="bf16"`` the intermediates are
    rounded to bfloat16 where mate_layer stores them (x, z, B, C, q, k, v, y,
    o, g and out; dt stays exact): the documented layer with exact arithmetic
    between the stores.
    """
    rnd = bf16_round if storage == "bf16" else (lambda a: a)
    batch, T, H, W = grid
    f = lambda n: np.asarray(w[n], dtype=np.float64)
    hb = np.asarray(h, dtype=np.float64).reshape(-1, h.shape[-1])
    nh, P, S, G = ssd["nheads"], ssd["headdim"], ssd["d_state"], ssd.get("ngroups", 1)
    th, td = tesa_sizes["nheads"], tesa_sizes["headdim"]
    tok = (batch, T, H, W)
    x = rnd(hb @ f("w_x")).reshape(tok + (nh, P))
    z = rnd(hb @ f("w_z"))
    Bm = rnd(hb @ f("w_b")).reshape(tok + (G, S))
    Cm = rnd(hb @ f("w_c")).reshape(tok + (G, S))
    dt = np.logaddexp(0.0, hb @ f("w_dt") + f("dt_bias")).reshape(tok + (nh,))
    y = rnd(bissd(x, Bm, Cm, dt, f("a"), f("d"), grid, order, ssd.get("pool", (0, 0, 0)), nthreads=nthreads))
    gv = y.reshape(-1, nh * P) * (z / (1.0 + np.exp(-z)))
    gv = gv.reshape(gv.shape[0], G, -1)
    gv = gv / np.sqrt(np.mean(gv * gv, axis=-1, keepdims=True) + norm_eps)
    gv = rnd(gv.reshape(-1, nh * P) * f("norm_w"))
    q, k, v = (rnd(hb @ f(n)).reshape(tok + (th, td)) for n in ("w_q", "w_k", "w_v"))
    o = rnd(tesa(q, k, v, grid, tesa_sizes["window"], tesa_sizes.get("shift", (0, 0, 0)),
                 tesa_sizes.get("scale", 0.0), nthreads=nthreads))
    out = gv @ f("w_ma_out") + o.reshape(-1, th * td) @ f("w_te_out")
    return rnd(out).reshape(tok + (hb.shape[1],))
