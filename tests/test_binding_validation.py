"""The Python binding rejects mismatched tensors before any pointer reaches
the C ABI (which cannot see extents): CPU tensors with wrong shapes or dtypes
raise ValueError naming the tensor, so nothing would be read or written past a
buffer's end on the device. No GPU and no library are needed: the checks run
before the library is loaded."""
import pytest

from linear_complexity_video_amd import binding as B

torch = pytest.importorskip("torch")


def ssd_set(grid=(1, 2, 4, 4), nh=3, P=16, G=1, S=8, dtype=torch.bfloat16):
    x = torch.zeros(*grid, nh, P, dtype=dtype)
    return dict(x=x, b=torch.zeros(*grid, G, S, dtype=dtype), c=torch.zeros(*grid, G, S, dtype=dtype),
                dt=torch.ones(*grid, nh), a=-torch.ones(nh), d=torch.zeros(nh), y=torch.zeros_like(x))


def call_ssd(t):
    B.mate_bissd_scan(t["x"], t["b"], t["c"], t["dt"], t["a"], t["d"], t["y"], 0, 8)


@pytest.mark.parametrize("name,bad,msg", [
    ("y", torch.zeros(1, 2, 4, 4, 3, 8, dtype=torch.bfloat16), "y has shape"),
    ("y", torch.zeros(1, 2, 4, 4, 3, 16), "y has dtype"),
    ("b", torch.zeros(1, 2, 4, 2, 1, 8, dtype=torch.bfloat16), "b must be"),
    ("c", torch.zeros(1, 2, 4, 4, 1, 4, dtype=torch.bfloat16), "c has shape"),
    ("c", torch.zeros(1, 2, 4, 4, 1, 8), "c has dtype"),
    ("dt", torch.ones(1, 2, 4, 4, 2), "dt has shape"),
    ("dt", torch.ones(1, 2, 4, 4, 3, dtype=torch.bfloat16), "dt must be float32"),
    ("a", -torch.ones(4), "a has shape"),
    ("d", torch.zeros(3, dtype=torch.float64), "d must be float32"),
])
def test_bissd_rejects_mismatched_tensors(name, bad, msg):
    t = ssd_set()
    t[name] = bad
    with pytest.raises(ValueError, match=msg):
        call_ssd(t)


def test_bissd_reaches_the_device_check_when_tensors_agree():
    with pytest.raises(ValueError, match="device tensors"):
        call_ssd(ssd_set())


def test_bimamba_rejects_mismatched_tensors():
    grid, nch, S = (1, 2, 4, 4), 6, 8
    x = torch.zeros(*grid, nch, dtype=torch.bfloat16)
    good = dict(x=x, b=torch.zeros(*grid, S, dtype=torch.bfloat16), c=torch.zeros(*grid, S, dtype=torch.bfloat16),
                dt=torch.ones(*grid, nch), a=-torch.ones(nch, S), d=torch.zeros(nch), y=torch.zeros_like(x))
    for name, bad, msg in (("a", -torch.ones(nch), "a has shape"), ("dt", torch.ones(*grid, nch + 1), "dt has shape"),
                           ("y", torch.zeros(*grid, nch), "y has dtype"), ("c", torch.zeros(*grid, 4, dtype=torch.bfloat16),
                                                                          "c has shape")):
        t = dict(good)
        t[name] = bad
        with pytest.raises(ValueError, match=msg):
            B.mate_bimamba_scan(*(t[k] for k in ("x", "b", "c", "dt", "a", "d", "y")), 0)


def test_tesa_and_backward_reject_mismatched_tensors():
    q = torch.zeros(1, 2, 4, 4, 2, 16, dtype=torch.bfloat16)
    small = torch.zeros(1, 2, 4, 4, 1, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="o has shape"):
        B.mate_tesa(q, q, q, small, (2, 2, 2))
    with pytest.raises(ValueError, match="k has dtype"):
        B.mate_tesa(q, q.float(), q, q, (2, 2, 2))
    with pytest.raises(ValueError, match="dv has shape"):
        B.mate_tesa_backward(q, q, q, q, q, q, small, (2, 2, 2))
    with pytest.raises(ValueError, match="q must be"):
        B.mate_tesa(q[0], q[0], q[0], q[0], (2, 2, 2))


def test_forward_rejects_grids_that_differ():
    s = ssd_set()
    att = {k: torch.zeros(1, 2, 4, 2, 2, 16, dtype=torch.bfloat16) for k in ("q", "k", "v", "o")}
    with pytest.raises(ValueError, match="grid"):
        B.mate_forward(s, att, 0, 8, (0, 0, 0), (2, 2, 2), (0, 0, 0))
    att = {k: torch.zeros(1, 2, 4, 4, 2, 16, dtype=torch.bfloat16) for k in ("q", "k", "v", "o")}
    s["y"] = torch.zeros(1, 2, 4, 4, 3, 16)
    with pytest.raises(ValueError, match="y has dtype"):
        B.mate_forward(s, att, 0, 8, (0, 0, 0), (2, 2, 2), (0, 0, 0))
