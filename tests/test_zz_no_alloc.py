"""The scan entry point that allocates nothing (mate_bissd_scan_noalloc), called through the C ABI, against
the entry point with a caller workspace (mate_bissd_scan) on the same inputs: two calls in a row on the
library's static scratch, the second with a smaller problem, so the second runs on scratch the first left
behind."""
from __future__ import annotations

import numpy as np
import pytest

from linear_complexity_video_amd import binding as B
from linear_complexity_video_amd import synth
from linear_complexity_video_amd.workloads import WORKLOADS
from tests.helpers import TOL, parity_error, ssd_inputs, to_f64, torch_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def _ragged_inputs():
    """105 tokens (3x5x7), 4 heads of 64, d_state 64, 2 groups, batch 2: a smaller problem than the first."""
    rng = np.random.default_rng(21)
    bsz, T, H, W, nh, P, S, G = 2, 3, 5, 7, 4, 64, 64, 2
    rnd = lambda *s: synth.bf16_bits_to_f32(synth.f32_to_bf16_bits((rng.standard_normal(s) / 8).astype(np.float32)))
    x, Bm, Cm = rnd(bsz, T, H, W, nh, P), rnd(bsz, T, H, W, G, S), rnd(bsz, T, H, W, G, S)
    dt = np.log1p(np.exp(rng.normal(-1, 0.5, (bsz, T, H, W, nh)))).astype(np.float32)
    A = -np.exp(rng.uniform(0, 1, nh)).astype(np.float32)
    D = rng.standard_normal(nh).astype(np.float32)
    return [torch.from_numpy(a).cuda().to(torch.bfloat16) for a in (x, Bm, Cm)] + \
           [torch.from_numpy(a).cuda() for a in (dt, A, D)]


def _both(dev, order, chunk, pool):
    y_ws = torch.full_like(dev[0], float("nan"))
    y_na = torch.full_like(dev[0], float("nan"))
    B.mate_bissd_scan(*dev, y_ws, order, chunk, pool)
    B.mate_bissd_scan_noalloc(*dev, y_na, order, chunk, pool)
    torch.cuda.synchronize()
    return y_ws, y_na


def test_noalloc_scan_matches_workspace_scan_twice():
    wl = WORKLOADS[1]
    inp = ssd_inputs(1)
    big = [torch_dev(inp[k]) for k in ("x", "B", "C", "dt", "A", "D")]
    print(f"noalloc call 1: {wl.name}, order 2", flush=True)
    y_ws, y_na = _both(big, 2, wl.chunk, wl.pool)
    assert not torch.isnan(y_na).any().item()
    assert parity_error(to_f64(y_na), to_f64(y_ws)) <= TOL[1]
    assert torch.equal(y_na, y_ws)
    print("noalloc call 2: 3x5x7 grid, batch 2, review tokens 3x1x7, order 4", flush=True)
    small = _ragged_inputs()
    y_ws, y_na = _both(small, 4, 64, (3, 1, 7))
    assert not torch.isnan(y_na).any().item()
    assert parity_error(to_f64(y_na), to_f64(y_ws)) <= 2e-2
    assert torch.equal(y_na, y_ws)


def test_noalloc_rejects_problems_beyond_the_scratch():
    inp = ssd_inputs(1)
    dev = [torch_dev(inp[k]) for k in ("x", "B", "C", "dt", "A", "D")]
    # the same tokens as 4x as many heads: the scan's workspace exceeds the static scratch
    x = dev[0].repeat(1, 1, 1, 1, 8, 1)
    dt, A, D = dev[3].repeat(1, 1, 1, 1, 8), dev[4].repeat(8), dev[5].repeat(8)
    y = torch.empty_like(x)
    with pytest.raises(B.MateError) as e:
        B.mate_bissd_scan_noalloc(x, dev[1], dev[2], dt, A, D, y, 0, 64)
    assert e.value.status == B.MATE_ERR_WORKSPACE
