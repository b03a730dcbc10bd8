#!/usr/bin/env python3
"""MATE-core forward throughput on one MI355X.

One step is the four-layer schedule of the long-grid workload (128 x 48 x 48
latent tokens, LinGen-4B widths): layer l scans in RMS order l and its TESA
windows are shifted on odd layers. Each layer is one ``mate_forward`` call
(bidirectional SSD with review tokens + TESA) through the C ABI. Inputs are
seeded synthetic tensors already resident in HBM when timing starts.

Prints one JSON line with tokens/s (tokens = T*H*W per layer forward), the
roofline position of the dominant kernel, per-call timings and the CPU oracle
timed on a bounded sample on this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MATE-core tokens/sec (bi-SSD + TESA fwd) at 1 GPU; % MFMA / HBM roofline"
PEAK_BF16_TFLOPS = 2500.0   # dense MFMA, MI355X
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
COPY_BYTES = 1 << 30


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# Algorithmic work (what the method must compute and move)
# ---------------------------------------------------------------------------

def region_sizes(D, w, s):
    if s == 0:
        return [w] * (D // w)
    return [s] + [w] * ((D - s) // w) + ([D - s - ((D - s) // w) * w] if (D - s) % w else [])


def tesa_pairs(wl, shift):
    """Sum over windows of |window|^2 (in-window query-key pairs)."""
    st = [a * a for a in region_sizes(wl.T, wl.window[0], shift[0])]
    sh = [a * a for a in region_sizes(wl.H, wl.window[1], shift[1])]
    sw = [a * a for a in region_sizes(wl.W, wl.window[2], shift[2])]
    return sum(st) * sum(sh) * sum(sw)


def work(wl):
    e = 2 if wl.dtype == "bf16" else 4
    Hs, P, S, G, Q = wl.nheads, wl.headdim, wl.d_state, wl.ngroups, wl.chunk
    scanned = wl.N + wl.R
    ssd_flops = 2.0 * (Hs * (4 * P * S + P * (Q + 1)) + G * S * (Q + 1)) * scanned
    ssd_bytes = (2 * Hs * P * e + 2 * G * S * e + 4 * Hs) * wl.N
    tesa_bytes = 4 * wl.t_heads * wl.t_dim * e * wl.N
    tesa_flops = {sh: 4.0 * wl.t_dim * wl.t_heads * tesa_pairs(wl, wl.layer_shift(sh)) * wl.batch
                  for sh in (False, True)}
    # The output sweep (one launch per scan) runs over the N main tokens: the intra-chunk product (both
    # triangles and the diagonal), the forward state update and both inter-chunk read-outs; it reads x, B, C,
    # dt once and writes y once, i.e. all of the scan's algorithmic bytes.
    out_flops = 2.0 * Hs * (3 * P * S + P * (Q + 1)) * wl.N * wl.batch
    out_bytes = ssd_bytes * wl.batch
    return dict(ssd_flops=ssd_flops * wl.batch, ssd_bytes=ssd_bytes * wl.batch, tesa_flops=tesa_flops,
                tesa_bytes=tesa_bytes * wl.batch, reorder_bytes=2 * wl.N * Hs * P * e * wl.batch,
                out_flops=out_flops, out_bytes=out_bytes)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ssd_out_long_grid_traffic.txt")
OUT_KERNEL_SOURCE = os.path.join(ROOT, "linear_complexity_video_amd", "csrc", "ssd_fast.hip")


def measured_traffic(wl):
    """HBM bytes per output-sweep launch from the committed rocprofv3 counter summary, scaled by the copy-kernel
    calibration recorded with it; None when there is none for this workload or the kernel source changed since."""
    import hashlib

    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    digest = hashlib.sha256(open(OUT_KERNEL_SOURCE, "rb").read()).hexdigest()
    if kv.get("source_sha256") != digest or kv.get("workload") != wl.name:
        return None
    copy_kib = float(kv["copy_bytes"]) / 1024.0
    fetch = float(kv["fetch_kib_per_dispatch"]) * copy_kib / float(kv["copy_fetch_kib"])
    write = float(kv["write_kib_per_dispatch"]) * copy_kib / float(kv["copy_write_kib"])
    return (fetch + write) * 1024.0


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the same layers
# ---------------------------------------------------------------------------

def cpu_baseline(wl, si, ti, threads):
    import numpy as np

    import oracle
    from linear_complexity_video_amd import synth

    def f32(t, hs=None):
        a = t.dev if hs is None else t.dev[..., hs[0]:hs[1], :]
        return synth.bf16_bits_to_f32(a) if a.dtype == np.uint16 else np.ascontiguousarray(a)

    hs = max(1, threads // 2)  # (head, direction) units: one per thread
    x = f32(si["x"], (0, hs))
    Bm, Cm = f32(si["B"]), f32(si["C"])
    dt = np.ascontiguousarray(si["dt"].dev[..., :hs])
    t0 = time.perf_counter()
    oracle.bissd(x, Bm, Cm, dt, si["A"].dev[:hs], si["D"].dev[:hs], wl.grid, 0, wl.pool, nthreads=threads)
    t_ssd = (time.perf_counter() - t0) * wl.nheads / hs
    qkv = [f32(ti[k], (0, 1)) for k in ("q", "k", "v")]
    t_tesa = {}
    for shifted in (False, True):
        t0 = time.perf_counter()
        oracle.tesa(*qkv, wl.grid, wl.window, wl.layer_shift(shifted), nthreads=threads)
        t_tesa[shifted] = (time.perf_counter() - t0) * wl.t_heads
    layer_s = sum(t_ssd + t_tesa[sh] for _, sh in wl.schedule) / len(wl.schedule)
    return {
        "value": wl.N / layer_s,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"bi-SSD heads 0..{hs - 1} of {wl.nheads} (order 0, review tokens) and TESA head 0 of "
                   f"{wl.t_heads} (unshifted and shifted) over the full {wl.T}x{wl.H}x{wl.W} grid; "
                   f"per-layer time scaled by heads and averaged over the layer schedule"),
        "layer_seconds_est": layer_s,
    }


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------

def scaling_sweep(torch, np, B, reps):
    """Per-layer forward time of the MATE core against full self-attention as the video grows.

    T = 32, 64, 128 latent frames at 48x48 (the 1:2:4 ratio of 17, 34 and 68 s clips). MATE core: one
    mate_forward at LinGen-4B widths (bi-SSD 80 x 64, d_s 128, chunk 128, 8^3 review pooling; TESA 20 x
    128, 8^3 windows). Full attention: the same TESA kernel with one window spanning the whole grid, at
    DiT-4B width (24 heads x 128). Inputs are synthetic (N(0,1)/sqrt(dim); dt, A as the long-grid
    workload). Prints one JSON line.
    """
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(0)
    stream = torch.cuda.current_stream()

    def rn(*shape, scale=1.0):
        return (torch.randn(*shape, device=dev, generator=g) * scale).to(torch.bfloat16)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(max(2, reps)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts))

    points = []
    for T in (32, 64, 128):
        H = W = 48
        N = T * H * W
        log(f"scaling: T={T} ({N} tokens)")
        ssd = {"x": rn(1, T, H, W, 80, 64, scale=1 / 8), "b": rn(1, T, H, W, 1, 128, scale=128 ** -0.5),
               "c": rn(1, T, H, W, 1, 128, scale=128 ** -0.5)}
        ssd["dt"] = torch.nn.functional.softplus(torch.randn(1, T, H, W, 80, device=dev, generator=g) * 0.5 - 2)
        ssd["a"] = -torch.exp(torch.rand(80, device=dev, generator=g) * 2)
        ssd["d"] = torch.randn(80, device=dev, generator=g)
        ssd["y"] = torch.empty_like(ssd["x"])
        att = {k: rn(1, T, H, W, 20, 128, scale=128 ** -0.5) for k in ("q", "k", "v")}
        att["o"] = torch.empty_like(att["q"])
        ws = torch.empty(B.mate_forward_workspace_size((1, T, H, W), B.ssd_desc(ssd["x"], ssd["b"], 128, (8, 8, 8)),
                                                       B.tesa_desc(att["q"], (8, 8, 8))),
                         dtype=torch.uint8, device=dev)
        t_mate = timed(lambda: B.mate_forward(ssd, att, 0, 128, (8, 8, 8), (8, 8, 8), (0, 0, 0), workspace=ws))
        del ssd, att, ws
        full = {k: rn(1, T, H, W, 24, 128, scale=128 ** -0.5) for k in ("q", "k", "v")}
        full["o"] = torch.empty_like(full["q"])
        t_full = timed(lambda: B.mate_tesa(full["q"], full["k"], full["v"], full["o"], (T, H, W), (0, 0, 0)))
        del full
        attn_flops = 4.0 * N * N * 24 * 128
        points.append({"T": T, "H": H, "W": W, "tokens": N, "mate_core_ms": t_mate * 1e3,
                       "full_attention_ms": t_full * 1e3, "full_over_mate": t_full / t_mate,
                       "mate_core_tokens_per_s": N / t_mate,
                       "full_attention_tflops": attn_flops / t_full / 1e12})
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "per-layer forward time: MATE core vs full self-attention (one MI355X)",
                      "unit": "ms", "data": "synthetic", "points": points}), flush=True)


def table2_variants(torch, np, B, wl, ssd, att, ws, reps, algo):
    """Per-layer cost of the variants the pages compare in their ablation (xllm-io review, Table 2 and
    section 五): the RMS layer schedule against the zigzag scan, the layer without review tokens, and
    each branch alone, all on the same inputs at the workload's full size. The pages' zigzag overhead
    comes from reordering large 3D tensors; here every order is index math inside the scan's gathers,
    so the cost of materializing a scan order as tensors (x, B, C and dt gathered into it, y scattered
    back, each a `mate_rms_reorder`) is reported beside it. The Mamba row runs the selective scan
    (`mate_bimamba_scan`) on the same x as 5120 channels, with per-channel dt and A and d_state 16
    (sizes the pages do not give), then TESA. Prints one JSON line.
    """
    stream = torch.cuda.current_stream()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(max(3, reps)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    def forward(order, shifted, pool):
        return timed(lambda: B.mate_forward(ssd, att, order, wl.chunk, pool, wl.window, wl.layer_shift(shifted),
                                            algo=algo, workspace=ws))

    sched = list(wl.schedule)
    mean = lambda xs: float(np.mean(xs))
    log("variants: RMS schedule")
    rms = [forward(o, sh, wl.pool) for o, sh in sched]
    log("variants: zigzag")
    zig = [forward(B.ORDER_ZIGZAG, sh, wl.pool) for _, sh in sched]
    log("variants: no review tokens")
    norev = [forward(o, sh, (0, 0, 0)) for o, sh in sched]
    log("variants: branches alone")
    te = [timed(lambda sh=sh: B.mate_tesa(att["q"], att["k"], att["v"], att["o"], wl.window, wl.layer_shift(sh),
                                          0.0, algo)) for _, sh in sched]
    ma = {o: timed(lambda o=o: B.mate_bissd_scan(ssd["x"], ssd["b"], ssd["c"], ssd["dt"], ssd["a"], ssd["d"],
                                                 ssd["y"], o, wl.chunk, wl.pool, algo, workspace=ws))
          for o in [o for o, _ in sched] + [B.ORDER_ZIGZAG]}
    log("variants: materialized reorders")
    mat = {}
    for order in (2, B.ORDER_ZIGZAG):
        total = 0.0
        for key, inverse in (("x", False), ("b", False), ("c", False), ("dt", False), ("y", True)):
            src = ssd[key]
            dst = torch.empty_like(src)
            total += timed(lambda src=src, dst=dst: B.mate_rms_reorder(src, dst, wl.grid, order, False, inverse))
            del dst
        mat["zigzag" if order == B.ORDER_ZIGZAG else f"rms_order_{order}"] = total
    torch.cuda.empty_cache()
    log("variants: Mamba (selective scan) MA branch")
    T, H, W = wl.T, wl.H, wl.W
    dev = ssd["x"].device
    g = torch.Generator(device=dev).manual_seed(7)
    nch, S1 = ssd["x"].shape[-2] * ssd["x"].shape[-1], 16
    mx = ssd["x"].view(wl.batch, T, H, W, nch)
    mB = (torch.randn(wl.batch, T, H, W, S1, device=dev, generator=g) / 4).to(torch.bfloat16)
    mC = (torch.randn(wl.batch, T, H, W, S1, device=dev, generator=g) / 4).to(torch.bfloat16)
    mdt = torch.nn.functional.softplus(torch.randn(wl.batch, T, H, W, nch, device=dev, generator=g) * 0.5 - 2)
    mA = -torch.exp(torch.rand(nch, S1, device=dev, generator=g) * 2)
    mD = torch.randn(nch, device=dev, generator=g)
    my = torch.empty_like(mx)
    mws = torch.empty(B.mate_bimamba_workspace_size(wl.grid, B.mamba_desc(mx, mB, wl.pool)), dtype=torch.uint8,
                      device=dev)
    mamba_ma = {o: timed(lambda o=o: B.mate_bimamba_scan(mx, mB, mC, mdt, mA, mD, my, o, wl.pool, workspace=mws))
                for o in sorted(set(o for o, _ in sched))}

    def mamba_layer(o, sh):
        B.mate_bimamba_scan(mx, mB, mC, mdt, mA, mD, my, o, wl.pool, workspace=mws)
        B.mate_tesa(att["q"], att["k"], att["v"], att["o"], wl.window, wl.layer_shift(sh), 0.0, algo)

    mamba = [timed(lambda o=o, sh=sh: mamba_layer(o, sh)) for o, sh in sched]
    del mB, mC, mdt, my, mws
    torch.cuda.empty_cache()
    ms_rms = mean(rms)
    rows = {
        "rms_schedule": {"ms": ms_rms, "per_layer_ms": rms},
        "zigzag": {"ms": mean(zig), "per_layer_ms": zig, "vs_rms": mean(zig) / ms_rms},
        "no_review_tokens": {"ms": mean(norev), "per_layer_ms": norev, "vs_rms": mean(norev) / ms_rms},
        "te_branch_only": {"ms": mean(te), "vs_rms": mean(te) / ms_rms},
        "ma_branch_only": {"ms": mean([ma[o] for o, _ in sched]),
                           "per_order_ms": {str(o): t for o, t in ma.items() if o != B.ORDER_ZIGZAG},
                           "zigzag_ms": ma[B.ORDER_ZIGZAG]},
        "materialized_scan_order": {"ms": mat, "tensors": "x, B, C, dt gathered; y scattered back"},
        "mamba_selective_scan": {"ms": mean(mamba), "per_layer_ms": mamba, "vs_rms": mean(mamba) / ms_rms,
                                 "ma_branch_ms": mean(list(mamba_ma.values())),
                                 "ma_branch_per_order_ms": {str(o): t for o, t in mamba_ma.items()},
                                 "channels": nch, "d_state": S1},
    }
    print(json.dumps({"metric": "per-layer forward time of the ablation variants (one MI355X)", "unit": "ms",
                      "data": "synthetic",
                      "config": {"workload": wl.name, "grid": list(wl.grid), "chunk": wl.chunk,
                                 "pool": list(wl.pool), "window": list(wl.window)},
                      "variants": rows}), flush=True)


def backward_bench(torch, np, B, wl, att, ssd, ws_fwd, reps):
    """Per-layer time of the two backward passes beside their forwards on the workload's inputs: TESA's
    (`mate_tesa_backward`: dq, dk, dv for an upstream gradient), unshifted and shifted, and the
    bidirectional scan's (`mate_bissd_backward`), per RMS order of the schedule. TESA's algorithmic work:
    the forward's two products per in-window pair (4 d flops), the backward's five (recomputed scores, dP,
    dV, dQ, dK: 10 d flops). Prints one JSON line."""
    stream = torch.cuda.current_stream()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(max(3, reps)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    g = torch.Generator(device=att["q"].device).manual_seed(11)
    dout = (torch.randn(att["q"].shape, device=att["q"].device, generator=g) / 11.3).to(att["q"].dtype)
    dq, dk, dv = (torch.empty_like(att["q"]) for _ in range(3))
    ws = torch.empty(max(1, B.mate_tesa_backward_workspace_size(wl.grid, B.tesa_desc(att["q"], wl.window))),
                     dtype=torch.uint8, device=att["q"].device)
    rows = {}
    for shifted in (False, True):
        shift = wl.layer_shift(shifted)
        pairs = tesa_pairs(wl, shift) * wl.batch * wl.t_heads
        log(f"tesa backward: shift {shift}")
        tf = timed(lambda: B.mate_tesa(att["q"], att["k"], att["v"], att["o"], wl.window, shift))
        tb = timed(lambda: B.mate_tesa_backward(att["q"], att["k"], att["v"], dout, dq, dk, dv, wl.window, shift,
                                                workspace=ws))
        ff, fb = 4.0 * wl.t_dim * pairs, 10.0 * wl.t_dim * pairs
        rows["shifted" if shifted else "unshifted"] = {
            "forward_ms": tf, "backward_ms": tb, "backward_over_forward": tb / tf,
            "forward_tflops": ff / tf / 1e9, "backward_tflops": fb / tb / 1e9,
            "backward_mfma_frac": fb / tb / 1e9 / PEAK_BF16_TFLOPS}
    del dq, dk, dv, ws
    torch.cuda.empty_cache()
    # The scan's backward (mate_bissd_backward: dx, dB, dC, ddt, dA, dD) beside its forward, per RMS order.
    # Algorithmic work of the backward: the chunked evaluation's products per token and head (both
    # directions): the two state contributions and the two adjoint contributions, M^T dy and the four
    # state products of dx, dB and dC (each 2 P S flops), and the intra-chunk products
    # DX = dy x^T, M^T dy, Z B, Z^T C (2 Q P or 2 Q S flops each), Q the backward's chunk.
    Hs, P, S, Q = wl.nheads, wl.headdim, wl.d_state, 64
    flops_per_token = Hs * (2 * P * S * (4 + 2 + 4) + 2 * Q * (2 * P + 2 * S))
    g2 = torch.Generator(device=ssd["x"].device).manual_seed(12)
    dy = torch.randn(ssd["x"].shape, device=ssd["x"].device, generator=g2).to(ssd["x"].dtype)
    grads = {"dx": torch.empty_like(ssd["x"]), "db": torch.empty_like(ssd["b"]), "dc": torch.empty_like(ssd["c"]),
             "ddt": torch.empty_like(ssd["dt"]), "da": torch.empty_like(ssd["a"]), "dd": torch.empty_like(ssd["d"])}
    bws = torch.empty(max(1, B.mate_bissd_backward_workspace_size(wl.grid, B.ssd_desc(ssd["x"], ssd["b"], 64,
                                                                                       wl.pool))),
                      dtype=torch.uint8, device=ssd["x"].device)
    log(f"scan backward: workspace {bws.numel() / 2**30:.1f} GiB")
    scan_rows = {}
    for order in sorted(set(o for o, _ in wl.schedule)):
        tf = timed(lambda: B.mate_bissd_scan(ssd["x"], ssd["b"], ssd["c"], ssd["dt"], ssd["a"], ssd["d"], ssd["y"],
                                             order, wl.chunk, wl.pool, workspace=ws_fwd))
        tb = timed(lambda: B.mate_bissd_backward(ssd["x"], ssd["b"], ssd["c"], ssd["dt"], ssd["a"], ssd["d"], dy,
                                                 grads["dx"], grads["db"], grads["dc"], grads["ddt"], grads["da"],
                                                 grads["dd"], order, wl.pool, workspace=bws))
        fb = flops_per_token * wl.N * wl.batch
        scan_rows[str(order)] = {"forward_ms": tf, "backward_ms": tb, "backward_over_forward": tb / tf,
                                 "backward_tflops": fb / tb / 1e9,
                                 "backward_fp32_frac": fb / tb / 1e9 / PEAK_FP32_TFLOPS}
    print(json.dumps({"metric": "backward vs forward per layer: TESA and the bidirectional scan (one MI355X)",
                      "unit": "ms", "data": "synthetic",
                      "config": {"workload": wl.name, "grid": list(wl.grid), "tesa": [wl.t_heads, wl.t_dim],
                                 "window": list(wl.window), "ssd": [Hs, P, S], "pool": list(wl.pool),
                                 "ssd_backward_chunk": Q, "ssd_backward_workspace_gib": bws.numel() / 2**30},
                      "tesa_layers": rows, "ssd_backward_per_order": scan_rows}), flush=True)


def block_bench(torch, np, B, wl, reps):
    """LinGen-4B layers through the library's mate_layer (projections on hipBLASLt, the MATE core, the MA
    branch's gate and norm, the MA+TE sum). Widths from the xllm-io review's model table (2560-wide rows,
    20 heads) and the core's own (MA: 80 heads x 64 = 2 x 2560, d_state 128; TE: 20 x 128). Times one layer
    per (order, shift) of the schedule, a real 32-layer stack (order l mod 4, shift on odd l; random weights
    per layer, the output of one layer the input of the next), and, for a Table 2-style split, the MA and TE
    branches' core calls on the same grid. Prints one JSON line."""
    stream = torch.cuda.current_stream()
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(13)
    N, d = wl.N * wl.batch, 2560
    Hs, P, S, th, td = wl.nheads, wl.headdim, wl.d_state, wl.t_heads, wl.t_dim
    bf = torch.bfloat16
    grid = wl.grid
    nlayers = 32

    def weights():
        m = lambda i, o: (torch.randn(i, o, device=dev, generator=g) / np.sqrt(i)).to(bf)
        return {"w_x": m(d, Hs * P), "w_z": m(d, Hs * P), "w_b": m(d, S), "w_c": m(d, S),
                "w_dt": (m(d, Hs).float() * 0.3).to(bf), "w_ma_out": m(Hs * P, d),
                "dt_bias": torch.randn(Hs, device=dev, generator=g) * 0.5 - 1.0,
                "a": -torch.exp(torch.rand(Hs, device=dev, generator=g) * 2),
                "d": torch.randn(Hs, device=dev, generator=g),
                "norm_w": 1 + 0.1 * torch.randn(Hs * P, device=dev, generator=g),
                "w_q": m(d, th * td), "w_k": m(d, th * td), "w_v": m(d, th * td), "w_te_out": m(th * td, d)}

    log("block: weights of 32 layers")
    layers = [weights() for _ in range(nlayers)]
    ssd = dict(nheads=Hs, headdim=P, d_state=S, ngroups=1, chunk=wl.chunk, pool=wl.pool)
    te = lambda shifted: dict(nheads=th, headdim=td, window=wl.window, shift=wl.layer_shift(shifted))
    ld, sd, tdesc = B.layer_descs(grid, d, ssd, te(False))
    ws = torch.empty(B.mate_layer_workspace_size(grid, ld, sd, tdesc), dtype=torch.uint8, device=dev)
    h = [torch.randn(*grid, d, device=dev, generator=g).to(bf), torch.empty(*grid, d, device=dev, dtype=bf)]

    def layer(i, src, dst):
        B.mate_layer(src, dst, layers[i], d, ssd, te(i % 2 == 1), i % 4, workspace=ws)

    def timed(fn, n=None):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(n or max(3, reps)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    log("block: one layer per schedule entry")
    t_layer = [timed(lambda i=i: layer(i, h[0], h[1])) for i in range(4)]

    def stack():
        for i in range(nlayers):
            layer(i, h[i % 2], h[(i + 1) % 2])

    log("block: 32-layer stack")
    t_stack = timed(stack, 3)
    ok = bool(torch.isfinite(h[0].float()).all().item())
    # the two branches' core calls alone, on tensors of the layer's shapes
    x = torch.randn(*grid, Hs, P, device=dev, generator=g).to(bf)
    bc = torch.randn(*grid, 1, S, device=dev, generator=g).to(bf)
    dt = torch.nn.functional.softplus(torch.randn(*grid, Hs, device=dev, generator=g) - 1.0)
    y = torch.empty_like(x)
    q = torch.randn(*grid, th, td, device=dev, generator=g).to(bf)
    o = torch.empty_like(q)
    swsp = torch.empty(B.mate_bissd_workspace_size(grid, B.ssd_desc(x, bc, wl.chunk, wl.pool)), dtype=torch.uint8,
                       device=dev)
    t_ma = [timed(lambda o_=o_: B.mate_bissd_scan(x, bc, bc, dt, layers[0]["a"], layers[0]["d"], y, o_, wl.chunk,
                                                  wl.pool, workspace=swsp)) for o_ in range(4)]
    t_te = [timed(lambda s_=s_: B.mate_tesa(q, q, q, o, wl.window, wl.layer_shift(s_))) for s_ in (False, True)]
    gemm_flops = 2.0 * N * d * (2 * Hs * P + 2 * S + Hs + 3 * th * td) + 2.0 * N * d * (Hs * P + th * td)
    mean = lambda xs: float(np.mean(xs))
    print(json.dumps({"metric": "LinGen-4B MATE layers through mate_layer (one MI355X)", "unit": "ms",
                      "data": "synthetic, random weights",
                      "config": {"workload": wl.name, "tokens": N, "embedding": d, "ma": [Hs, P, S], "te": [th, td],
                                 "layers": nlayers},
                      "layer_ms_per_schedule_entry": t_layer, "layer_ms": mean(t_layer),
                      "stack_32_layers_ms": t_stack, "stack_output_finite": ok,
                      "ma_core_ms": mean(t_ma), "te_core_ms": mean(t_te),
                      "ma_share_of_core": mean(t_ma) / (mean(t_ma) + mean(t_te)),
                      "projection_gemm_tflop_per_layer": gemm_flops / 1e12}), flush=True)


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None where there is none)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def device_info(torch):
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2**30, 1)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=4, help="workload index (default: the long grid)")
    ap.add_argument("--algo", choices=("auto", "portable", "fast"), default="auto")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=5, help="timed repetitions of each single call")
    ap.add_argument("--scaling", action="store_true",
                    help="instead of the throughput line: MATE core vs full attention per layer as T grows")
    ap.add_argument("--block", action="store_true",
                    help="instead of the throughput line: LinGen-4B layers through mate_layer (one layer per schedule "
                         "entry and a 32-layer stack)")
    ap.add_argument("--backward", action="store_true",
                    help="instead of the throughput line: the backward passes (TESA, the scan) beside their "
                         "forwards, per layer")
    ap.add_argument("--variants", action="store_true",
                    help="instead of the throughput line: per-layer time of the ablation variants (zigzag scan, "
                         "no review tokens, each branch alone)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="finish with a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the MATE core here runs on a single MI355X; "
              f"--gpus {args.gpus} (WORLD_SIZE {world}) is not supported.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from linear_complexity_video_amd import binding as B
    from linear_complexity_video_amd import synth
    from linear_complexity_video_amd.workloads import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    B.lib()
    if args.scaling:
        scaling_sweep(torch, np, B, args.kernel_reps)
        return
    if args.block:
        block_bench(torch, np, B, WORKLOADS[args.config], args.kernel_reps)
        return
    algo = {"auto": B.ALGO_AUTO, "portable": B.ALGO_PORTABLE, "fast": B.ALGO_FAST}[args.algo]
    wl = WORKLOADS[args.config]
    dev = torch.device("cuda:0")

    log(f"generating inputs for {wl.name} ...")
    t0 = time.perf_counter()
    si = synth.make_ssd_inputs(wl, keep_f32=False)
    ti = synth.make_tesa_inputs(wl, keep_f32=False)

    def to_dev(t):
        a = t.dev
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    ssd = {k: to_dev(si[n]) for k, n in (("x", "x"), ("b", "B"), ("c", "C"), ("dt", "dt"), ("a", "A"), ("d", "D"))}
    att = {k: to_dev(ti[k]) for k in ("q", "k", "v")}
    ssd["y"] = torch.empty_like(ssd["x"])
    att["o"] = torch.empty_like(att["q"])
    sdesc = B.ssd_desc(ssd["x"], ssd["b"], wl.chunk, wl.pool, algo)
    tdesc = B.tesa_desc(att["q"], wl.window, (0, 0, 0), 0.0, algo)
    ws = torch.empty(max(1, B.mate_forward_workspace_size(wl.grid, sdesc, tdesc)), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s; workspace {ws.numel() / 2**30:.2f} GiB")
    if args.variants:
        table2_variants(torch, np, B, wl, ssd, att, ws, args.kernel_reps, algo)
        return
    if args.backward:
        backward_bench(torch, np, B, wl, att, ssd, ws, args.kernel_reps)
        return

    def layer(order, shifted):
        B.mate_forward(ssd, att, order, wl.chunk, wl.pool, wl.window, wl.layer_shift(shifted), algo=algo,
                       workspace=ws)

    def step():
        for order, shifted in wl.schedule:
            layer(order, shifted)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done")

    # Timed region: the output sweep of the scan (the dominant kernel) is bracketed by HIP events on the
    # stream it runs on, launch by launch, through the library's timing hook.
    torch.cuda.synchronize()
    B.mate_timing_begin("ssd_out")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    out_launches, out_ms_total = B.mate_timing_end()
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_step = wl.N * wl.batch * len(wl.schedule)
    value = tokens_per_step * args.steps / elapsed
    t_out = out_ms_total / max(1, out_launches) * 1e-3
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step, {value / 1e6:.3f} M tokens/s; "
        f"output sweep {t_out * 1e3:.3f} ms over {out_launches} launches")

    # Per-kernel timings: the library brackets each launch of the named kernel with HIP events on its
    # stream (host launch latency of the Python calls is not included). A whole scan call is timed with
    # events on torch's current stream, which it launches on.
    stream = torch.cuda.current_stream()

    def time_kernel(kernel, fn, reps):
        fn()
        torch.cuda.synchronize()
        B.mate_timing_begin(kernel)
        for _ in range(reps):
            fn()
        n, ms = B.mate_timing_end()
        return ms / max(1, n) * 1e-3

    def time_call(fn, reps):
        fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3

    w = work(wl)
    reps = args.kernel_reps
    t_tesa = {sh: time_kernel("tesa", lambda sh=sh: B.mate_tesa(att["q"], att["k"], att["v"], att["o"], wl.window,
                                                                wl.layer_shift(sh), 0.0, algo), reps)
              for sh in (False, True)}
    t_ssd = time_call(lambda: B.mate_bissd_scan(ssd["x"], ssd["b"], ssd["c"], ssd["dt"], ssd["a"], ssd["d"],
                                                ssd["y"], 0, wl.chunk, wl.pool, algo, workspace=ws), reps)
    # One layer per RMS order (mate_forward alone, events on torch's stream, which every kernel of the
    # call is launched on): median of the repetitions.
    layers = []
    for order, shifted in wl.schedule:
        ts = []
        for _ in range(max(3, reps)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            layer(order, shifted)
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        t = float(np.median(ts))
        layers.append({"order": order, "tesa_shifted": shifted, "ms": t * 1e3,
                       "tokens_per_s": wl.N * wl.batch / t})
    xr = ssd["x"].view(wl.batch, wl.N, -1)
    xo = torch.empty_like(xr)
    t_rms = time_kernel("rms_reorder", lambda: B.mate_rms_reorder(xr, xo, wl.grid, 1, True, False), reps)
    t_states = time_kernel("ssd_states", lambda: B.mate_bissd_scan(ssd["x"], ssd["b"], ssd["c"], ssd["dt"], ssd["a"],
                                                                   ssd["d"], ssd["y"], 0, wl.chunk, wl.pool, algo,
                                                                   workspace=ws), reps)

    peak_flops = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_FP32_TFLOPS
    tesa_tf = w["tesa_flops"][False] / t_tesa[False] / 1e12
    ssd_tf = w["ssd_flops"] / t_ssd / 1e12
    out_tf = w["out_flops"] / t_out / 1e12
    out_gbs = w["out_bytes"] / t_out / 1e9
    kernels = {
        "ssd_out_sweep": {"ms": t_out * 1e3, "tflops": out_tf, "mfma_frac": out_tf / peak_flops, "gbs": out_gbs,
                          "hbm_frac": out_gbs / PEAK_HBM_GBS, "launches_timed": out_launches},
        "ssd_states_sweep_avg_of_review_and_main": {"ms": t_states * 1e3},
        "bissd_call": {"ms": t_ssd * 1e3, "tflops": ssd_tf, "mfma_frac": ssd_tf / peak_flops,
                       "hbm_frac": w["ssd_bytes"] / t_ssd / 1e9 / PEAK_HBM_GBS},
        "tesa_unshifted": {"ms": t_tesa[False] * 1e3, "tflops": tesa_tf, "mfma_frac": tesa_tf / peak_flops,
                           "hbm_frac": w["tesa_bytes"] / t_tesa[False] / 1e9 / PEAK_HBM_GBS},
        "tesa_shifted": {"ms": t_tesa[True] * 1e3, "tflops": w["tesa_flops"][True] / t_tesa[True] / 1e12,
                         "mfma_frac": w["tesa_flops"][True] / t_tesa[True] / 1e12 / peak_flops},
        "rms_reorder_x": {"ms": t_rms * 1e3, "gbs": w["reorder_bytes"] / t_rms / 1e9,
                          "hbm_frac": w["reorder_bytes"] / t_rms / 1e9 / PEAK_HBM_GBS},
    }
    # Roofline of the dominant kernel: whichever of its algorithmic flops and bytes takes longer at peak.
    hbm_bound = w["out_bytes"] / (PEAK_HBM_GBS * 1e9) >= w["out_flops"] / (peak_flops * 1e12)
    roofline = {"bound": "hbm" if hbm_bound else "mfma",
                "achieved": out_gbs if hbm_bound else out_tf,
                "peak": PEAK_HBM_GBS if hbm_bound else peak_flops,
                "unit": "GB/s" if hbm_bound else "TFLOP/s",
                "frac": out_gbs / PEAK_HBM_GBS if hbm_bound else out_tf / peak_flops,
                "traffic": measured_traffic(wl),
                "kernel": "bi-SSD output sweep (k_out)",
                "algorithmic_per_launch": {"flops": w["out_flops"], "bytes": w["out_bytes"]},
                "mfma_frac": out_tf / peak_flops}
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: batch {wl.batch}, {wl.N} tokens, four-layer schedule "
                        f"(RMS order l, TESA shifted on odd l)",
            "grid": [wl.T, wl.H, wl.W], "batch": wl.batch, "tokens_per_layer": wl.N,
            "layers_per_step": len(wl.schedule), "review_tokens": wl.R,
            "ssd": {"heads": wl.nheads, "headdim": wl.headdim, "d_state": wl.d_state, "groups": wl.ngroups,
                    "chunk": wl.chunk, "pool": list(wl.pool)},
            "tesa": {"heads": wl.t_heads, "headdim": wl.t_dim, "window": list(wl.window), "shift": list(wl.shift)},
            "algo": args.algo,
        },
        "roofline": roofline,
        "layers": layers,
        "kernels": kernels,
        "device": device_info(torch),
    }
    if args.calibrate_copy:
        # A plain streaming kernel of known size (reads and writes COPY_BYTES once each: an elementwise
        # negation), for scaling HBM byte counters taken on this same run.
        src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = COPY_BYTES
    if not args.no_cpu_baseline:
        # Every host CPU this process may run on, up to the 16 threads that one GPU's share of a GPU host
        # is sized for.
        host_cpus = len(os.sched_getaffinity(0))
        threads = max(1, min(16, host_cpus))
        log(f"timing the CPU oracle on a sample with {threads} threads ...")
        out["cpu_baseline"] = cpu_baseline(wl, si, ti, threads)
        out["cpu_baseline"]["host_cpus"] = host_cpus
        out["cpu_baseline"]["cpu_model"] = cpu_model()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
