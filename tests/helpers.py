"""Shared helpers of the GPU tests: device copies of synthetic inputs and the
parity error metric."""
from __future__ import annotations

import functools

import numpy as np

from linear_complexity_video_amd import synth
from linear_complexity_video_amd.workloads import WORKLOADS

TOL = {0: 1e-4, 1: 2e-2, 2: 2e-2, 3: 2e-2, 4: 2e-2}


def parity_error(g: np.ndarray, r: np.ndarray) -> float:
    """max_i |g_i - r_i| / max(|r_i|, rms(r)): a relative error that does not
    blow up where the reference crosses zero."""
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    if r.size == 0:
        return 0.0
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    rms = float(np.sqrt(np.mean(r * r)))
    denom = np.maximum(np.abs(r), max(rms, 1e-30))
    return float(np.max(np.abs(g - r) / denom))


def torch_dev(t: synth.Tensor):
    import torch
    a = t.dev
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


@functools.lru_cache(maxsize=2)
def ssd_inputs(cfg: int):
    return synth.make_ssd_inputs(WORKLOADS[cfg], keep_f32=(cfg <= 3))


@functools.lru_cache(maxsize=2)
def tesa_inputs(cfg: int):
    return synth.make_tesa_inputs(WORKLOADS[cfg], keep_f32=(cfg <= 3))


def f32_of(t: synth.Tensor, head_slice=None) -> np.ndarray:
    """float32 values of a synth tensor (optionally only heads [lo, hi) of the
    second-to-last axis), converting bf16 bit patterns when needed."""
    if t.f32 is not None:
        a = t.f32
        return a[..., head_slice[0]:head_slice[1], :] if head_slice else a
    a = t.dev if head_slice is None else t.dev[..., head_slice[0]:head_slice[1], :]
    return synth.bf16_bits_to_f32(a) if a.dtype == np.uint16 else np.ascontiguousarray(a)
