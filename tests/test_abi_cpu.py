"""Host-side checks of the C ABI: the library loads, exports what include/mate.h
declares, and rejects bad arguments before touching a device (no GPU needed:
every call here fails validation, so nothing is launched)."""
import ctypes
import os
import re
import subprocess

import pytest

from linear_complexity_video_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mate.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="libmate.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mate_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert sorted(B.EXPORTED) == declared_functions()


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for name in declared_functions():
        assert name in exported, name
    lib = B.lib()
    for name in declared_functions():
        assert hasattr(lib, name)
    assert lib.mate_abi_version() == 1


def test_status_strings():
    lib = B.lib()
    for s in range(6):
        assert lib.mate_status_string(s).decode().startswith("MATE_")


FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: validation fails first


def test_rms_validation():
    lib = B.lib()
    g = B.Grid(1, 2, 2, 2)
    assert lib.mate_rms_reorder(None, FAKE, g, 16, 0, 0, 0, None) == B.MATE_ERR_NULL
    assert lib.mate_rms_reorder(FAKE, ctypes.c_void_p(0x900000), g, 16, 5, 0, 0, None) == B.MATE_ERR_SHAPE
    assert "order" in lib.mate_last_error().decode()
    assert lib.mate_rms_reorder(FAKE, ctypes.c_void_p(0x900000), g, 16, -1, 0, 0, None) == B.MATE_ERR_SHAPE
    assert lib.mate_rms_reorder(FAKE, ctypes.c_void_p(0x900000), B.Grid(1, 0, 2, 2), 16, 0, 0, 0, None) == B.MATE_ERR_SHAPE
    assert lib.mate_rms_reorder(FAKE, ctypes.c_void_p(0x900000), g, 0, 0, 0, 0, None) == B.MATE_ERR_SHAPE
    # overlapping buffers
    assert lib.mate_rms_reorder(FAKE, ctypes.c_void_p(0x100010), g, 16, 0, 0, 0, None) == B.MATE_ERR_SHAPE
    assert "overlap" in lib.mate_last_error().decode()
    # more than 2^31 tokens
    assert lib.mate_rms_reorder(FAKE, ctypes.c_void_p(0x900000), B.Grid(1, 2048, 2048, 1024), 2, 0, 0, 0,
                                None) == B.MATE_ERR_UNSUPPORTED
    # rows of 4 GiB or more (the kernels count a row's vectors in 32 bits)
    assert lib.mate_rms_reorder(FAKE, ctypes.c_void_p(0x900000), B.Grid(1, 1, 1, 2), 1 << 32, 0, 0, 0,
                                None) == B.MATE_ERR_UNSUPPORTED
    assert "4 GiB" in lib.mate_last_error().decode()


def _ssd(**kw):
    d = dict(nheads=2, headdim=16, d_state=8, ngroups=1, chunk=8, pool_t=0, pool_h=0, pool_w=0,
             dtype=B.MATE_F32, algo=B.ALGO_AUTO)
    d.update(kw)
    return B.SsdDesc(**d)


def _ssd_t(**kw):
    d = {k: 0x100000 + 0x1000 * i for i, k in enumerate(("x", "b", "c", "dt", "a", "d", "y"))}
    d.update(kw)
    return B.SsdTensors(**d)


def _scan(t, g, order, desc, ws=0x800000, wsb=1 << 40):
    return B.lib().mate_bissd_scan(ctypes.byref(t), g, order, ctypes.byref(desc), ctypes.c_void_p(ws), wsb, None)


def _mamba(**kw):
    d = dict(channels=12, d_state=16, pool_t=0, pool_h=0, pool_w=0, dtype=B.MATE_BF16)
    d.update(kw)
    return B.MambaDesc(**d)


def _mscan(t, g, order, desc, ws=0x800000, wsb=1 << 40):
    return B.lib().mate_bimamba_scan(ctypes.byref(t), g, order, ctypes.byref(desc), ctypes.c_void_p(ws), wsb, None)


def test_mamba_validation():
    g = B.Grid(1, 2, 4, 4)
    assert _mscan(_ssd_t(dt=0), g, 0, _mamba()) == B.MATE_ERR_NULL
    assert B.lib().mate_bimamba_scan(ctypes.byref(_ssd_t()), g, 0, None, ctypes.c_void_p(0x800000), 1 << 40,
                                     None) == B.MATE_ERR_NULL
    assert _mscan(_ssd_t(), g, 5, _mamba()) == B.MATE_ERR_SHAPE
    assert _mscan(_ssd_t(), g, B.ORDER_ZIGZAG, _mamba(), wsb=16) == B.MATE_ERR_WORKSPACE  # zigzag is accepted
    assert _mscan(_ssd_t(), g, 0, _mamba(channels=0)) == B.MATE_ERR_SHAPE
    assert _mscan(_ssd_t(), g, 0, _mamba(pool_t=2, pool_h=3, pool_w=2)) == B.MATE_ERR_SHAPE
    assert _mscan(_ssd_t(), g, 0, _mamba(pool_t=2, pool_h=0, pool_w=2)) == B.MATE_ERR_SHAPE
    assert _mscan(_ssd_t(), g, 0, _mamba(d_state=12)) == B.MATE_ERR_UNSUPPORTED
    assert _mscan(_ssd_t(), g, 0, _mamba(dtype=7)) == B.MATE_ERR_SHAPE
    assert _mscan(_ssd_t(x=0x100008), g, 0, _mamba()) == B.MATE_ERR_UNSUPPORTED  # misaligned x
    assert _mscan(_ssd_t(), g, 0, _mamba(), ws=0) == B.MATE_ERR_WORKSPACE
    assert _mscan(_ssd_t(), g, 0, _mamba(), ws=0x800010) == B.MATE_ERR_WORKSPACE
    # workspace: a bf16 partial of y and 256 spare elements, plus the pooled review x (bf16), dt (fp32)
    # and B (bf16) when pooled
    n = 2 * 4 * 4
    al = lambda v: (v + 255) // 256 * 256
    assert B.mate_bimamba_workspace_size((1, 2, 4, 4), _mamba()) == al(n * 12 * 2) + al(256 * 2)
    R = 1 * 2 * 2
    assert B.mate_bimamba_workspace_size((1, 2, 4, 4), _mamba(pool_t=2, pool_h=2, pool_w=2)) == \
        al(n * 12 * 2) + al(256 * 2) + al(R * 12 * 2) + al(R * 12 * 4) + al(R * 16 * 2)
    assert B.mate_bimamba_workspace_size((1, 2, 4, 4), _mamba(d_state=12)) == 0


def test_launch_grid_extents_rejected_before_launch():
    """Batch, head and review-token counts above 65535 (the launch grids' y and z extents) fail validation
    with MATE_ERR_UNSUPPORTED instead of failing at a launch."""
    lib = B.lib()
    big = 70000
    err = lambda: lib.mate_last_error().decode()
    assert _scan(_ssd_t(), B.Grid(big, 1, 1, 2), 0, _ssd()) == B.MATE_ERR_UNSUPPORTED and "batch" in err()
    assert _scan(_ssd_t(), B.Grid(1, 2, 2, 2), 0, _ssd(nheads=big)) == B.MATE_ERR_UNSUPPORTED and "nheads" in err()
    one = B.Grid(1, 1, 256, 257)  # 65792 tokens, each its own review token under a 1x1x1 pool
    assert _scan(_ssd_t(), one, 0, _ssd(pool_t=1, pool_h=1, pool_w=1)) == B.MATE_ERR_UNSUPPORTED
    assert "review tokens" in err()
    assert _mscan(_ssd_t(), one, 0, _mamba(pool_t=1, pool_h=1, pool_w=1)) == B.MATE_ERR_UNSUPPORTED
    assert _mscan(_ssd_t(), B.Grid(big, 1, 1, 2), 0, _mamba()) == B.MATE_ERR_UNSUPPORTED
    ptrs = {n: 0x100000 + 0x1000 * i for i, n in enumerate(("q", "k", "v", "o"))}
    desc = lambda **kw: B.TesaDesc(**{**dict(nheads=2, headdim=64, win_t=1, win_h=1, win_w=2, shift_t=0, shift_h=0,
                                             shift_w=0, scale=0.0, dtype=B.MATE_BF16, algo=B.ALGO_AUTO), **kw})
    tesa = lambda g, d: lib.mate_tesa(ctypes.byref(B.TesaTensors(**ptrs)), g, ctypes.byref(d), None)
    assert tesa(B.Grid(big, 1, 1, 2), desc()) == B.MATE_ERR_UNSUPPORTED and "batch" in err()
    assert tesa(B.Grid(1, 1, 1, 2), desc(nheads=big)) == B.MATE_ERR_UNSUPPORTED and "nheads" in err()
    # more than 2^22 one-token windows, scan chunks of 8 tokens, or 2^26 Mamba channels
    assert tesa(B.Grid(1, 2, 2048, 1025), desc(win_w=1)) == B.MATE_ERR_UNSUPPORTED and "regions" in err()
    assert _scan(_ssd_t(), B.Grid(1, 2, 4096, 4097), 0, _ssd()) == B.MATE_ERR_UNSUPPORTED and "chunks" in err()
    assert _mscan(_ssd_t(), B.Grid(1, 1, 1, 2), 0, _mamba(channels=(1 << 26) + 8)) == B.MATE_ERR_UNSUPPORTED
    assert "channels" in err()


def test_ssd_backward_validation():
    lib = B.lib()
    g = B.Grid(1, 2, 4, 4)
    ptrs = {f[0]: 0x100000 + 0x1000 * i for i, f in enumerate(B.SsdGradTensors._fields_)}
    t = lambda **kw: B.SsdGradTensors(**{**ptrs, **kw})
    call = lambda tt, gg, dd, ws=0x800000, wsb=1 << 40: lib.mate_bissd_backward(
        ctypes.byref(tt), gg, 0, ctypes.byref(dd), ctypes.c_void_p(ws), wsb, None)
    assert call(t(dy=0), g, _ssd()) == B.MATE_ERR_NULL
    assert call(t(dd=0), g, _ssd()) == B.MATE_ERR_NULL
    assert call(t(dx=0x100008), g, _ssd()) == B.MATE_ERR_UNSUPPORTED            # misaligned
    assert call(t(), g, _ssd(chunk=0)) == B.MATE_ERR_SHAPE
    assert call(t(), g, _ssd(headdim=24)) == B.MATE_ERR_UNSUPPORTED
    assert call(t(), g, _ssd(d_state=12)) == B.MATE_ERR_UNSUPPORTED
    # 65535 review tokens (a 1x1x1 pool) and 5000 heads: the review-gradient launch would pass 2^32
    # work-items
    big = B.Grid(1, 1, 255, 257)
    assert call(t(), big, _ssd(nheads=5000, pool_t=1, pool_h=1, pool_w=1)) == B.MATE_ERR_UNSUPPORTED
    assert "2^24" in lib.mate_last_error().decode()
    assert call(t(), g, _ssd(), wsb=16) == B.MATE_ERR_WORKSPACE
    assert call(t(), g, _ssd(), ws=0x800010) == B.MATE_ERR_WORKSPACE
    assert call(t(), g, _ssd(), ws=0) == B.MATE_ERR_WORKSPACE


def test_tesa_backward_validation():
    lib = B.lib()
    g = B.Grid(1, 4, 4, 4)
    desc = lambda **kw: B.TesaDesc(**{**dict(nheads=2, headdim=64, win_t=2, win_h=2, win_w=2, shift_t=0, shift_h=0,
                                             shift_w=0, scale=0.0, dtype=B.MATE_BF16, algo=B.ALGO_AUTO), **kw})
    ptrs = {n: 0x100000 + 0x1000 * i for i, n in enumerate(("q", "k", "v", "dout", "dq", "dk", "dv"))}
    t = lambda **kw: B.TesaGradTensors(**{**ptrs, **kw})
    call = lambda tt, dd, ws=0x800000, wsb=1 << 40: lib.mate_tesa_backward(ctypes.byref(tt), g, ctypes.byref(dd),
                                                                           ctypes.c_void_p(ws), wsb, None)
    assert call(t(dout=0), desc()) == B.MATE_ERR_NULL
    assert call(t(dv=0), desc()) == B.MATE_ERR_NULL
    assert call(t(dq=0x100008), desc()) == B.MATE_ERR_UNSUPPORTED           # misaligned
    assert call(t(), desc(win_t=3)) == B.MATE_ERR_SHAPE                     # does not divide the grid
    assert call(t(), desc(shift_t=2)) == B.MATE_ERR_SHAPE                   # shift not below the window
    assert call(t(), desc(headdim=32)) == B.MATE_ERR_UNSUPPORTED
    assert call(t(), desc(dtype=B.MATE_F32)) == B.MATE_ERR_UNSUPPORTED
    assert call(t(), desc(), wsb=16) == B.MATE_ERR_WORKSPACE
    assert call(t(), desc(), ws=0x800010) == B.MATE_ERR_WORKSPACE
    # two floats per token and head
    assert B.mate_tesa_backward_workspace_size((1, 4, 4, 4), desc()) == 64 * 2 * 8
    assert B.mate_tesa_backward_workspace_size((1, 4, 4, 4), desc(headdim=32)) == 0


def test_last_error_is_per_thread():
    """mate_last_error is thread-local: two threads that fail for different reasons each read their own
    reason, also after the other thread's failure."""
    import threading
    lib = B.lib()
    g = B.Grid(1, 2, 2, 2)
    both_failed = threading.Barrier(2)
    got = {}

    def run(name, order, row_bytes):
        status = lib.mate_rms_reorder(FAKE, ctypes.c_void_p(0x900000), g, row_bytes, order, 0, 0, None)
        both_failed.wait(timeout=30)
        got[name] = (status, lib.mate_last_error().decode())

    threads = [threading.Thread(target=run, args=("order", 5, 16)), threading.Thread(target=run, args=("rows", 0, 0))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert got["order"][0] == B.MATE_ERR_SHAPE and "order" in got["order"][1] and "row_bytes" not in got["order"][1]
    assert got["rows"][0] == B.MATE_ERR_SHAPE and "row_bytes" in got["rows"][1] and "order" not in got["rows"][1]


def test_ssd_validation():
    g = B.Grid(1, 2, 4, 4)
    assert _scan(_ssd_t(y=0), g, 0, _ssd()) == B.MATE_ERR_NULL
    assert _scan(_ssd_t(), g, 5, _ssd()) == B.MATE_ERR_SHAPE
    assert _scan(_ssd_t(), g, 0, _ssd(chunk=0)) == B.MATE_ERR_SHAPE
    assert _scan(_ssd_t(), g, 0, _ssd(nheads=3, ngroups=2)) == B.MATE_ERR_SHAPE
    assert _scan(_ssd_t(), g, 0, _ssd(pool_t=2, pool_h=3, pool_w=2)) == B.MATE_ERR_SHAPE   # 3 does not divide 4
    assert _scan(_ssd_t(), g, 0, _ssd(pool_t=2, pool_h=0, pool_w=2)) == B.MATE_ERR_SHAPE
    assert _scan(_ssd_t(), g, 0, _ssd(headdim=256)) == B.MATE_ERR_UNSUPPORTED
    assert _scan(_ssd_t(), g, 0, _ssd(chunk=256)) == B.MATE_ERR_UNSUPPORTED
    assert _scan(_ssd_t(), g, 0, _ssd(dtype=7)) == B.MATE_ERR_SHAPE
    # fp32 has no MFMA kernel
    assert _scan(_ssd_t(), g, 0, _ssd(algo=B.ALGO_FAST)) == B.MATE_ERR_UNSUPPORTED
    # workspace too small, NULL, or misaligned
    assert _scan(_ssd_t(), g, 0, _ssd(), wsb=16) == B.MATE_ERR_WORKSPACE
    assert _scan(_ssd_t(), g, 0, _ssd(), ws=0) == B.MATE_ERR_WORKSPACE
    assert _scan(_ssd_t(), g, 0, _ssd(), ws=0x800010) == B.MATE_ERR_WORKSPACE


def test_ssd_workspace_size_is_positive_and_grows():
    lib = B.lib()
    small = lib.mate_bissd_workspace_size(B.Grid(1, 2, 4, 4), ctypes.byref(_ssd()))
    big = lib.mate_bissd_workspace_size(B.Grid(1, 4, 4, 4), ctypes.byref(_ssd()))
    pooled = lib.mate_bissd_workspace_size(B.Grid(1, 2, 4, 4), ctypes.byref(_ssd(pool_t=2, pool_h=2, pool_w=2)))
    assert 0 < small < big and small < pooled
    assert lib.mate_bissd_workspace_size(B.Grid(1, 2, 4, 4), ctypes.byref(_ssd(chunk=0))) == 0


def _tesa(**kw):
    d = dict(nheads=2, headdim=16, win_t=2, win_h=2, win_w=2, shift_t=0, shift_h=0, shift_w=0, scale=0.0,
             dtype=B.MATE_F32, algo=B.ALGO_AUTO)
    d.update(kw)
    return B.TesaDesc(**d)


def _att(t, g, desc):
    return B.lib().mate_tesa(ctypes.byref(t), g, ctypes.byref(desc), None)


def test_tesa_validation():
    g = B.Grid(1, 2, 4, 4)
    t = B.TesaTensors(0x100000, 0x200000, 0x300000, 0x400000)
    assert _att(B.TesaTensors(0x100000, 0, 0x300000, 0x400000), g, _tesa()) == B.MATE_ERR_NULL
    assert _att(t, g, _tesa(win_h=3)) == B.MATE_ERR_SHAPE
    assert _att(t, g, _tesa(shift_t=2)) == B.MATE_ERR_SHAPE
    assert _att(t, g, _tesa(shift_w=-1)) == B.MATE_ERR_SHAPE
    assert _att(t, g, _tesa(headdim=12)) == B.MATE_ERR_UNSUPPORTED
    assert _att(t, g, _tesa(algo=B.ALGO_FAST)) == B.MATE_ERR_UNSUPPORTED
    assert B.lib().mate_tesa(None, g, ctypes.byref(_tesa()), None) == B.MATE_ERR_NULL
    # Windows above 4096 tokens have a kernel only when one window spans the whole unshifted grid.
    big = B.Grid(1, 16, 48, 48)
    bf = dict(headdim=128, dtype=B.MATE_BF16, win_t=8, win_h=48, win_w=48)
    assert _att(t, big, _tesa(**bf)) == B.MATE_ERR_UNSUPPORTED
    assert _att(t, big, _tesa(**dict(bf, win_t=16, shift_t=4))) == B.MATE_ERR_UNSUPPORTED
    assert _att(t, big, _tesa(**dict(bf, win_t=16, dtype=B.MATE_F32))) == B.MATE_ERR_UNSUPPORTED


def test_forward_validation_rejects_before_launch():
    lib = B.lib()
    g = B.Grid(1, 2, 4, 4)
    st, sd = _ssd_t(), _ssd()
    tt, td = B.TesaTensors(0x100000, 0x200000, 0x300000, 0x400000), _tesa(win_t=3)
    rc = lib.mate_forward(ctypes.byref(st), ctypes.byref(sd), ctypes.byref(tt), ctypes.byref(td), g, 0,
                          ctypes.c_void_p(0x800000), 1 << 40, None)
    assert rc == B.MATE_ERR_SHAPE
    assert lib.mate_forward_workspace_size(g, ctypes.byref(sd), ctypes.byref(td)) == 0


def test_misaligned_token_tensors_are_rejected():
    g = B.Grid(1, 2, 4, 4)
    assert _scan(_ssd_t(x=0x100008), g, 0, _ssd()) == B.MATE_ERR_UNSUPPORTED
    assert "16-byte" in B.lib().mate_last_error().decode()
    assert _scan(_ssd_t(dt=0x103002), g, 0, _ssd()) == B.MATE_ERR_UNSUPPORTED
    t = B.TesaTensors(0x100000, 0x200000, 0x300004, 0x400000)
    assert _att(t, g, _tesa()) == B.MATE_ERR_UNSUPPORTED


def test_timing_arming_rules():
    """Arming and disarming touch no device when nothing was launched."""
    lib = B.lib()
    assert lib.mate_timing_begin(b"no_such_kernel") == B.MATE_ERR_SHAPE
    assert lib.mate_timing_begin(None) == B.MATE_ERR_NULL
    B.mate_timing_begin("ssd_out")
    assert lib.mate_timing_begin(b"tesa") == B.MATE_ERR_SHAPE      # one timing at a time
    assert lib.mate_timing_end(None, None) == B.MATE_ERR_NULL      # stays armed
    assert B.mate_timing_end() == (0, 0.0)
    for name in ("rms_reorder", "ssd_pool", "ssd_prep", "ssd_cb", "ssd_states", "ssd_seg_pass", "ssd_out", "tesa",
                 "mamba_scan", "tesa_backward"):
        B.mate_timing_begin(name)
        assert B.mate_timing_end() == (0, 0.0)


def test_noalloc_scan_validation_and_scratch_limit():
    """The entry point without a workspace validates like mate_bissd_scan and rejects problems whose scan
    workspace exceeds the library's static scratch before touching a device."""
    lib = B.lib()
    g = B.Grid(1, 8, 16, 16)
    desc = _ssd(nheads=16, headdim=64, d_state=64, chunk=64, dtype=B.MATE_BF16)
    need = lib.mate_bissd_workspace_size(g, ctypes.byref(desc))
    assert 0 < need <= B.STATIC_SCRATCH_BYTES  # the 8x16x16 workload fits
    t = _ssd_t()
    assert lib.mate_bissd_scan_noalloc(None, g, 0, ctypes.byref(desc), None) == B.MATE_ERR_NULL
    assert lib.mate_bissd_scan_noalloc(ctypes.byref(t), g, 7, ctypes.byref(desc), None) == B.MATE_ERR_SHAPE
    big = _ssd(nheads=80, headdim=64, d_state=128, chunk=128, dtype=B.MATE_BF16)
    g2 = B.Grid(1, 32, 32, 32)
    assert lib.mate_bissd_workspace_size(g2, ctypes.byref(big)) > B.STATIC_SCRATCH_BYTES
    assert lib.mate_bissd_scan_noalloc(ctypes.byref(t), g2, 0, ctypes.byref(big), None) == B.MATE_ERR_WORKSPACE
    assert "static scratch" in lib.mate_last_error().decode()


def test_layer_validation_rejects_before_launch():
    """mate_layer checks pointers, alignment, both descriptors (bf16 only), d_model and the workspace before
    any device call; its workspace size is the intermediates, the joint B/C/dt weights, the scan's workspace
    and 64 MiB."""
    lib = B.lib()
    g = B.Grid(1, 8, 16, 16)
    ld, sd, td = B.layer_descs((1, 8, 16, 16), 256, dict(nheads=16, headdim=64, d_state=64, chunk=64),
                               dict(nheads=8, headdim=64, window=(4, 8, 8)))
    need = lib.mate_layer_workspace_size(g, ctypes.byref(ld), ctypes.byref(sd), ctypes.byref(td))
    n = 8 * 16 * 16
    nbcd = 2 * 64 + 16  # the joint B, C and dt projection's width
    y_region = max(1024 * 2, nbcd * 4)  # y, which first holds the joint projection's fp32 rows
    inter = n * (2 * 1024 * 2 + y_region + 2 * 64 * 2 + 16 * 4 + 4 * 512 * 2) + 256 * nbcd * 2
    scan = lib.mate_bissd_workspace_size(g, ctypes.byref(sd))
    assert inter + scan + (64 << 20) <= need <= inter + scan + (64 << 20) + 16 * 256
    w = B.LayerWeights(*([0x200000] * len(B.LAYER_WEIGHTS)))
    h, out, ws = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x900000), ctypes.c_void_p(0x4000000)
    call = lambda w_, ld_, sd_, td_, ws_=ws, wsb=need, order=0, h_=h: lib.mate_layer(
        h_, out, ctypes.byref(w_), ctypes.byref(ld_), ctypes.byref(sd_), ctypes.byref(td_), g, order, ws_, wsb, None)
    assert call(B.LayerWeights(*([0x200000] * 13 + [0])), ld, sd, td) == B.MATE_ERR_NULL
    assert call(w, ld, sd, td, h_=None) == B.MATE_ERR_NULL
    assert call(w, ld, sd, td, h_=ctypes.c_void_p(0x100008)) == B.MATE_ERR_UNSUPPORTED
    assert call(w, B.LayerDesc(250, 1e-5), sd, td) == B.MATE_ERR_SHAPE
    assert call(w, B.LayerDesc(256, -1.0), sd, td) == B.MATE_ERR_SHAPE
    sd32 = B.SsdDesc(16, 64, 64, 1, 64, 0, 0, 0, B.MATE_F32, B.ALGO_AUTO)
    assert call(w, ld, sd32, td) == B.MATE_ERR_UNSUPPORTED
    assert "bf16" in lib.mate_last_error().decode()
    assert call(w, ld, sd, td, order=9) == B.MATE_ERR_SHAPE
    assert call(w, ld, sd, td, wsb=need - 1) == B.MATE_ERR_WORKSPACE
    assert call(w, ld, sd, td, ws_=ctypes.c_void_p(0x4000080)) == B.MATE_ERR_WORKSPACE
    assert lib.mate_layer_workspace_size(g, ctypes.byref(B.LayerDesc(0, 1e-5)), ctypes.byref(sd),
                                         ctypes.byref(td)) == 0
