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
    tag = "1: tiny fp32 forward 1x1x256x64"
    assert_close(o, ro, "f32", "O", tag=(tag, "O"))
    assert_close(lse, rl, "f32", "LSE", kind="lse", tag=(tag, "LSE"))


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_gpt2_medium_workload(causal):
    """Workload 2 at full size (8x16x1024x64 bf16): every row of every head."""
    w = fa_inputs.WORKLOADS[2]
    x, tau, o, lse = _run(w.B, w.H, w.N, w.d, w.dtype, causal, w.seed, tau=w.tau)
    ro, rl = orc.attention_fwd(*(x[n].f64() for n in ("q", "k", "v")), w.tau, causal)
    tag = "2: GPT-2-medium-shaped forward 8x16x1024x64, %s" % ("causal" if causal else "non-causal")
    assert_close(o, ro, "bf16", "O", tag=(tag, "O"))
    assert_close(lse, rl, "bf16", "LSE", kind="lse", tag=(tag, "LSE"))


def _long_rows(seed):
    """Rows of one head of the long prefill: both edges of every 128-row block
    (the key tile; query tiles are 256 rows, waves 32) and 256 more drawn
    uniformly: 512 rows."""
    edges = np.concatenate([np.arange(0, 16384, 128), np.arange(127, 16384, 128)])
    rng = np.random.Generator(np.random.PCG64(seed))
    rest = np.setdiff1d(np.arange(16384), edges)
    return np.sort(np.concatenate([edges, rng.choice(rest, 256, replace=False)]))


def test_fwd_long_causal_workload():
    """Workload 3 at full size (1x32x16384x128 bf16, causal): all 32 heads, every
    row of heads 0 and 31 and 512 rows (every tile edge included) of the others."""
    w = fa_inputs.WORKLOADS[3]
    x, tau, o, lse = _run(w.B, w.H, w.N, w.d, w.dtype, True, w.seed, tau=w.tau)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    qf, kf, vf = (x[n].f64() for n in ("q", "k", "v"))
    tag = "3: long causal prefill 1x32x16384x128"
    for h in range(w.H):
        rows = None if h in (0, 31) else _long_rows(3300 + h)
        ro, rl = orc.attention_fwd_head(qf[0, h], kf[0, h], vf[0, h], w.tau, True, rows=rows)
        sel = slice(None) if rows is None else rows
        assert_close(o[0, h, sel], ro, "bf16", "O[h=%d]" % h, tag=(tag, "O"))
        assert_close(lse[0, h, sel], rl, "bf16", "LSE[h=%d]" % h, kind="lse", tag=(tag, "LSE"))


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
