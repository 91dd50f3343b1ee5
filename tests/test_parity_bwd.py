"""GPU parity of fa_bwd (D preprocess, dK/dV, dQ) against the float64 oracle."""
import numpy as np
import pytest

import fa_inputs
from oracle import attention as orc
from tests.util import assert_close, record, to_device, to_f64

pytestmark = pytest.mark.gpu


def _run(x, causal, tau):
    import io_aware_tiled_03_amd as fa
    import torch
    q, k, v, do = (to_device(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, tau=tau, causal=causal)
    B, H, N, d = q.shape
    ws = torch.empty(fa.bwd_workspace_bytes(B, H, N) // 4, dtype=torch.float32, device="cuda")
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, tau=tau, causal=causal, workspace=ws)
    return {"dq": to_f64(dq), "dk": to_f64(dk), "dv": to_f64(dv), "D": to_f64(ws).reshape(B, H, N)}


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 7, 63, 130, 257, 600])
def test_bwd_small(N, causal, d):
    B, H = 2, 2
    x = fa_inputs.dense_inputs(B, H, N, d, "bf16", 10000 + N, with_do=True)
    tau = 1.0 / np.sqrt(d)
    g = _run(x, causal, tau)
    ref = orc.attention_bwd(*(x[n].f64() for n in ("q", "k", "v", "do")), tau, causal)
    for name in ("dq", "dk", "dv"):
        assert_close(g[name], ref[name], "bf16", name)
    # D is computed from the forward's bf16 output O, so it inherits O's error:
    # |D_gpu - D| <= sum_d |dO_d| * (|O_d - bf16(O_d)| + |err of O_d|), with the
    # bf16 rounding of O bounded by 2^-8 |O_d| (one unit in the last place, so a
    # rounding that lands on the other side is covered) and O's error by the
    # mean tolerance 2e-3.
    do64, o64 = x["do"].f64(), orc.attention_fwd(*(x[n].f64() for n in ("q", "k", "v")),
                                                 tau, causal)[0]
    bound = (np.abs(do64) * (2.0 ** -8 * np.abs(o64) + 2e-3)).sum(axis=-1)
    assert np.all(np.abs(g["D"] - ref["D"]) <= bound), np.abs(g["D"] - ref["D"]).max()


def test_bwd_workload_full():
    """Workload 5 at full size (4x16x4096x64 bf16, causal): every head element by
    element at the stated bounds, D against its bound from O's storage."""
    w = fa_inputs.WORKLOADS[5]
    x = fa_inputs.workload_inputs(w)
    import io_aware_tiled_03_amd as fa
    import torch
    q, k, v, do = (to_device(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, tau=w.tau, causal=True)
    ws = torch.empty(fa.bwd_workspace_bytes(w.B, w.H, w.N) // 4, dtype=torch.float32, device="cuda")
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, tau=w.tau, causal=True, workspace=ws)
    g = {"dq": to_f64(dq), "dk": to_f64(dk), "dv": to_f64(dv),
         "D": to_f64(ws).reshape(w.B, w.H, w.N), "o": to_f64(o)}
    qf, kf, vf, dof = (x[n].f64() for n in ("q", "k", "v", "do"))
    tag = "5: causal backward 4x16x4096x64"
    for b in range(w.B):
        for h in range(w.H):
            ref = orc.attention_bwd_head(qf[b, h], kf[b, h], vf[b, h], dof[b, h], w.tau, True)
            for name in ("dq", "dk", "dv"):
                assert_close(g[name][b, h], ref[name], "bf16", "%s[%d,%d]" % (name, b, h),
                             tag=(tag, name))
            assert_close(g["o"][b, h], ref["o"], "bf16", "O[%d,%d]" % (b, h), tag=(tag, "O (forward)"))
            # D is formed from the stored bf16 O: |D_gpu - D| <= sum_c |dO_c| |O_gpu_c - O_c|
            # plus the fp32 rounding of the length-d sum
            bound = (np.abs(dof[b, h]) * (np.abs(g["o"][b, h] - ref["o"])
                                           + 2.0 ** -17 * np.abs(g["o"][b, h]))).sum(axis=1)
            assert np.all(np.abs(g["D"][b, h] - ref["D"]) <= bound + 1e-6), (b, h)
            record(tag, "D", g["D"][b, h], ref["D"])


def test_bwd_deterministic():
    import io_aware_tiled_03_amd as fa
    import torch
    x = fa_inputs.dense_inputs(2, 2, 700, 64, "bf16", 10500, with_do=True)
    q, k, v, do = (to_device(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=True)
    a = fa.bwd(q, k, v, o, lse, do, causal=True)
    b = fa.bwd(q, k, v, o, lse, do, causal=True)
    for t1, t2 in zip(a, b):
        assert torch.equal(t1, t2)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [100, 130])
def test_bwd_very_negative_scores_ragged_tail(N, d):
    """Every score near -100 or below (Q = 8, K = -1.6 + small noise), so each
    row's LSE is below -88, where exp(-LSE) overflows float32; N is not a
    multiple of the key tile, so the tail tile holds keys past N.  Those keys
    must contribute nothing: dQ, dK, dV finite and equal to the exact
    gradients (non-causal, where no diagonal masks the tail)."""
    import io_aware_tiled_03_amd as fa
    import torch
    B, H = 1, 2
    rng = np.random.default_rng(10600 + N + d)
    q = np.full((B, H, N, d), 8.0)
    k = -1.6 + 0.05 * rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, d))
    do = rng.standard_normal((B, H, N, d))
    dev = [torch.from_numpy(a.astype(np.float32)).to("cuda", torch.bfloat16) for a in (q, k, v, do)]
    qf, kf, vf, dof = (to_f64(t) for t in dev)
    tau = 1.0 / np.sqrt(d)
    o, lse = fa.fwd(dev[0], dev[1], dev[2], tau=tau, causal=False)
    assert to_f64(lse).max() < -88.0
    dq, dk, dv = fa.bwd(dev[0], dev[1], dev[2], o, lse, dev[3], tau=tau, causal=False)
    ref = orc.attention_bwd(qf, kf, vf, dof, tau, False)
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert_close(to_f64(got), ref[name], "bf16", name)


def _bwd_f32(x, tau, causal, **kw):
    import io_aware_tiled_03_amd as fa
    q, k, v, do = (to_device(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, tau=tau, causal=causal, **kw)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, tau=tau, causal=causal, **kw)
    assert dq.dtype == q.dtype
    return {"dq": to_f64(dq), "dk": to_f64(dk), "dv": to_f64(dv)}


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 7, 63, 130, 257])
def test_bwd_f32_small(N, causal, d):
    """The fp32 backward (FA_F32) against the exact gradients at the fp32 bound."""
    x = fa_inputs.dense_inputs(1, 2, N, d, "f32", 10700 + N, with_do=True)
    tau = 1.0 / np.sqrt(d)
    g = _bwd_f32(x, tau, causal)
    ref = orc.attention_bwd(*(x[n].f64() for n in ("q", "k", "v", "do")), tau, causal)
    for name in ("dq", "dk", "dv"):
        assert_close(g[name], ref[name], "f32", name)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("w,s", [(1, 0), (16, 2), (100, 0)])
def test_bwd_f32_window(w, s, d):
    x = fa_inputs.dense_inputs(1, 2, 200, d, "f32", 10800 + w + s, with_do=True)
    tau = 1.0 / np.sqrt(d)
    g = _bwd_f32(x, tau, True, window=w, sinks=s)
    ref = orc.attention_bwd(*(x[n].f64() for n in ("q", "k", "v", "do")), tau, True, window=w,
                            sinks=s)
    for name in ("dq", "dk", "dv"):
        assert_close(g[name], ref[name], "f32", name)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_f32_dropout(causal, d):
    x = fa_inputs.dense_inputs(1, 2, 150, d, "f32", 10900 + d, with_do=True)
    tau = 1.0 / np.sqrt(d)
    g = _bwd_f32(x, tau, causal, dropout=(0.3, 77, 4))
    ref = orc.attention_bwd(*(x[n].f64() for n in ("q", "k", "v", "do")), tau, causal,
                            dropout=(77, 4, 0.3))
    for name in ("dq", "dk", "dv"):
        assert_close(g[name], ref[name], "f32", name)
