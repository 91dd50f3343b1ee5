"""GPU parity of the sliding-window mask with sink tokens (fa_fwd_window)
against the float64 oracle."""
import numpy as np
import pytest

import fa_inputs
from oracle import attention as orc
from tests.util import assert_close, bwd_allowance, to_device, to_f64

pytestmark = pytest.mark.gpu


def _fwd(x, tau, window, sinks):
    import io_aware_tiled_03_amd as fa
    q, k, v = (to_device(x[n]) for n in ("q", "k", "v"))
    o, lse = fa.fwd(q, k, v, tau=tau, causal=True, window=window, sinks=sinks)
    return to_f64(o), to_f64(lse)


WINDOWS = [(1, 0), (2, 1), (16, 0), (100, 4), (129, 0), (257, 3), (64, 64), (5000, 0)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("w,s", WINDOWS)
@pytest.mark.parametrize("N", [1, 7, 130, 300, 1000])
def test_window_bf16_small(N, w, s, d):
    x = fa_inputs.dense_inputs(2, 2, N, d, "bf16", 11000 + N + w + s)
    tau = 1.0 / np.sqrt(d)
    o, lse = _fwd(x, tau, w, s)
    ro, rl = orc.attention_fwd(*(x[n].f64() for n in ("q", "k", "v")), tau, True, window=w, sinks=s)
    assert_close(o, ro, "bf16", "O")
    assert_close(lse, rl, "bf16", "LSE", kind="lse")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("w,s", [(1, 0), (40, 2), (100, 0)])
@pytest.mark.parametrize("N", [33, 257])
def test_window_f32_small(N, w, s, d):
    x = fa_inputs.dense_inputs(1, 2, N, d, "f32", 12000 + N + w + s)
    tau = 1.0 / np.sqrt(d)
    o, lse = _fwd(x, tau, w, s)
    ro, rl = orc.attention_fwd(*(x[n].f64() for n in ("q", "k", "v")), tau, True, window=w, sinks=s)
    assert_close(o, ro, "f32", "O")
    assert_close(lse, rl, "f32", "LSE", kind="lse")


@pytest.mark.parametrize("d", [64, 128])
def test_window_covering_everything_is_the_causal_kernel(d):
    """window >= N and no sinks runs exactly the causal forward: same bits."""
    import io_aware_tiled_03_amd as fa
    import torch
    x = fa_inputs.dense_inputs(2, 3, 999, d, "bf16", 13000 + d)
    q, k, v = (to_device(x[n]) for n in ("q", "k", "v"))
    o1, l1 = fa.fwd(q, k, v, causal=True)
    o2, l2 = fa.fwd(q, k, v, causal=True, window=999)
    o3, l3 = fa.fwd(q, k, v, causal=True, window=1 << 30)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


@pytest.mark.parametrize("w,s", [(4096, 0), (1020, 4)])
def test_window_long_prefill(w, s):
    """The long prefill shape (1x32x16384x128 bf16) as a local layer with a
    4096-key window, and as a StreamingLLM-style window of 1020 keys plus 4
    sinks: sampled rows of 4 heads around tile and window edges."""
    wl = fa_inputs.WORKLOADS[3]
    x = fa_inputs.workload_inputs(wl)
    o, lse = _fwd(x, wl.tau, w, s)
    qf, kf, vf = (x[n].f64() for n in ("q", "k", "v"))
    rng = np.random.Generator(np.random.PCG64(34))
    edges = [0, 1, 3, 4, 5, 127, 128, w - 1, w, w + 1, w + 127, w + 128, 8191, 8192, 16383]
    rows = np.unique(np.concatenate([edges, rng.integers(0, wl.N, 100)]))
    for h in (0, 7, 20, 31):
        ro, rl = orc.attention_fwd_head(qf[0, h], kf[0, h], vf[0, h], wl.tau, True, rows=rows,
                                        window=w, sinks=s)
        tag = "next 2: window %d + %d sinks, 1x32x16384x128 (sampled rows)" % (w, s)
        assert_close(o[0, h, rows], ro, "bf16", "O[h=%d]" % h, tag=(tag, "O"))
        assert_close(lse[0, h, rows], rl, "bf16", "LSE[h=%d]" % h, kind="lse", tag=(tag, "LSE"))
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


def _bwd(x, tau, window, sinks):
    import io_aware_tiled_03_amd as fa
    q, k, v, do = (to_device(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, tau=tau, causal=True, window=window, sinks=sinks)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, tau=tau, causal=True, window=window, sinks=sinks)
    return {"o": to_f64(o), "dq": to_f64(dq), "dk": to_f64(dk), "dv": to_f64(dv)}


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("w,s", [(1, 0), (2, 1), (16, 0), (100, 4), (129, 0), (200, 130),
                                 (64, 64), (5000, 0)])
@pytest.mark.parametrize("N", [7, 130, 300, 600])
def test_window_bwd_small(N, w, s, d):
    x = fa_inputs.dense_inputs(2, 2, N, d, "bf16", 14000 + N + w + s, with_do=True)
    tau = 1.0 / np.sqrt(d)
    g = _bwd(x, tau, w, s)
    qf, kf, vf, dof = (x[n].f64() for n in ("q", "k", "v", "do"))
    for b in range(2):
        for h in range(2):
            # Exact gradients; the allowance models the kernels' bf16 steps:
            # D formed from the stored bf16 O (with a window of a few keys P
            # is close to one and D's error passes into dS undamped), P and dS
            # rounded to bf16 before their products, and one bf16 ulp for
            # entries above |x| = 5 (their storage rounding alone exceeds 2e-2).
            ref = orc.attention_bwd_head(qf[b, h], kf[b, h], vf[b, h], dof[b, h], tau, True,
                                         window=w, sinks=s)
            extra = bwd_allowance(ref, g["o"][b, h], qf[b, h], kf[b, h], dof[b, h], tau)
            for name in ("dq", "dk", "dv"):
                assert_close(g[name][b, h], ref[name], "bf16", "%s[%d,%d]" % (name, b, h),
                             ulp_allow=True, extra=extra[name])


@pytest.mark.parametrize("d", [64, 128])
def test_window_bwd_covering_everything_is_causal(d):
    """window >= N and no sinks: the causal backward's bits."""
    import io_aware_tiled_03_amd as fa
    import torch
    x = fa_inputs.dense_inputs(2, 2, 700, d, "bf16", 15000 + d, with_do=True)
    q, k, v, do = (to_device(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=True)
    g1 = fa.bwd(q, k, v, o, lse, do, causal=True)
    g2 = fa.bwd(q, k, v, o, lse, do, causal=True, window=700)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_window_bwd_workload():
    """The backward shape (4x16x4096x64 bf16) as a local layer with a
    1024-key window and 4 sinks: 3 sampled heads element by element."""
    wl = fa_inputs.WORKLOADS[5]
    x = fa_inputs.workload_inputs(wl)
    g = _bwd(x, wl.tau, 1024, 4)
    qf, kf, vf, dof = (x[n].f64() for n in ("q", "k", "v", "do"))
    for b, h in ((0, 3), (1, 10), (3, 15)):
        ref = orc.attention_bwd_head(qf[b, h], kf[b, h], vf[b, h], dof[b, h], wl.tau, True,
                                     window=1024, sinks=4)
        for name in ("dq", "dk", "dv"):
            assert_close(g[name][b, h], ref[name], "bf16", "%s[%d,%d]" % (name, b, h),
                         tag=("next 2: window 1024 + 4 sinks backward 4x16x4096x64 (3 heads)", name))
