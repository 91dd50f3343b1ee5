"""GPU parity of fa_fwd against the float64 oracle (through the C ABI)."""
import numpy as np
import pytest

import fa_inputs
from oracle import attention as orc
from tests.util import assert_close, to_device, to_f64

pytestmark = pytest.mark.gpu


def _run(B, H, N, d, dtype, causal, seed, tau=None):
    import io_aware_tiled_03_amd as fa
    x = fa_inputs.dense_inputs(B, H, N, d, dtype, seed)
    q, k, v = (to_device(x[n]) for n in ("q", "k", "v"))
    tau = 1.0 / np.sqrt(d) if tau is None else tau
    o, lse = fa.fwd(q, k, v, tau=tau, causal=causal)
    return x, tau, to_f64(o), to_f64(lse)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 7, 63, 64, 129, 300, 1000])
def test_fwd_bf16_small(N, causal, d):
    B, H = 2, 3
    x, tau, o, lse = _run(B, H, N, d, "bf16", causal, 7000 + N)
    qf, kf, vf = (x[n].f64() for n in ("q", "k", "v"))
    ro, rl = orc.attention_fwd(qf, kf, vf, tau, causal)
    assert_close(o, ro, "bf16", "O")
    assert_close(lse, rl, "bf16", "LSE", kind="lse")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 33, 256, 257])
def test_fwd_f32_small(N, causal, d):
    B, H = 1, 2
    x, tau, o, lse = _run(B, H, N, d, "f32", causal, 8000 + N)
    qf, kf, vf = (x[n].f64() for n in ("q", "k", "v"))
    ro, rl = orc.attention_fwd(qf, kf, vf, tau, causal)
    assert_close(o, ro, "f32", "O")
    assert_close(lse, rl, "f32", "LSE", kind="lse")


def test_fwd_tiny_fp32_workload():
    """Workload 1: B=1, H=1, N=256, d=64, fp32, tau=1/8, non-causal, full comparison."""
    w = fa_inputs.WORKLOADS[1]
    x, tau, o, lse = _run(w.B, w.H, w.N, w.d, w.dtype, False, w.seed, tau=w.tau)
    ro, rl = orc.attention_fwd(*(x[n].f64() for n in ("q", "k", "v")), w.tau, False)
    assert_close(o, ro, "f32", "O")
    assert_close(lse, rl, "f32", "LSE", kind="lse")


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_gpt2_medium_workload(causal):
    """Workload 2 at full size (8x16x1024x64 bf16): every row of 6 sampled heads."""
    w = fa_inputs.WORKLOADS[2]
    x, tau, o, lse = _run(w.B, w.H, w.N, w.d, w.dtype, causal, w.seed, tau=w.tau)
    qf, kf, vf = (x[n].f64() for n in ("q", "k", "v"))
    for b, h in ((0, 0), (1, 5), (3, 15), (5, 8), (7, 0), (7, 15)):
        ro, rl = orc.attention_fwd_head(qf[b, h], kf[b, h], vf[b, h], w.tau, causal)
        assert_close(o[b, h], ro, "bf16", "O[%d,%d]" % (b, h))
        assert_close(lse[b, h], rl, "bf16", "LSE[%d,%d]" % (b, h), kind="lse")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


def test_fwd_long_causal_workload():
    """Workload 3 at full size (1x32x16384x128 bf16, causal): sampled rows of 4 heads,
    including the first rows, tile edges and the last rows."""
    w = fa_inputs.WORKLOADS[3]
    x, tau, o, lse = _run(w.B, w.H, w.N, w.d, w.dtype, True, w.seed, tau=w.tau)
    qf, kf, vf = (x[n].f64() for n in ("q", "k", "v"))
    rng = np.random.Generator(np.random.PCG64(33))
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, 8191, 8192, 16255, 16256, 16383],
                                     rng.integers(0, w.N, 120)]))
    for h in (0, 9, 22, 31):
        ro, rl = orc.attention_fwd_head(qf[0, h], kf[0, h], vf[0, h], w.tau, True, rows=rows)
        assert_close(o[0, h, rows], ro, "bf16", "O[h=%d]" % h)
        assert_close(lse[0, h, rows], rl, "bf16", "LSE[h=%d]" % h, kind="lse")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


def test_fwd_ones_value_gives_ones():
    """Rows of P sum to one: V = 1 must give O = 1 (up to bf16 rounding of P)."""
    import io_aware_tiled_03_amd as fa
    import torch
    x = fa_inputs.dense_inputs(2, 4, 777, 128, "bf16", 91)
    q, k = to_device(x["q"]), to_device(x["k"])
    v = torch.ones_like(q)
    for causal in (False, True):
        o, _ = fa.fwd(q, k, v, causal=causal)
        assert torch.all((o.float() - 1).abs() <= 2e-2)


def test_fwd_deterministic():
    import io_aware_tiled_03_amd as fa
    import torch
    x = fa_inputs.dense_inputs(2, 4, 1000, 64, "bf16", 92)
    q, k, v = (to_device(x[n]) for n in ("q", "k", "v"))
    o1, l1 = fa.fwd(q, k, v, causal=True)
    o2, l2 = fa.fwd(q, k, v, causal=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
