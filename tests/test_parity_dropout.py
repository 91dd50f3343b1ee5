"""GPU parity of attention dropout (fa_fwd_dropout, fa_bwd_dropout) against the
float64 oracle, including a bit-exact read-back of the mask."""
import numpy as np
import pytest

import fa_inputs
from oracle import attention as orc
from tests.util import assert_close, bwd_allowance, to_device, to_f64

pytestmark = pytest.mark.gpu


def _dev(x, dtype="bf16"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to("cuda").to(torch.bfloat16 if dtype == "bf16" else torch.float32)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("p,seed,offset", [(0.5, 1, 0), (0.1, 0xDEADBEEF12345678, 7),
                                           (0.9, 42, 1 << 31)])
@pytest.mark.parametrize("N,J0", [(128, 0), (1024, 0), (1024, 640), (4096, 4096 - 64)])
def test_dropout_mask_forward_exact(N, J0, p, seed, offset, d):
    """Q = 0 makes P uniform (1/N); V rows J0 .. J0+d-1 one-hot (others 0), so
    O_i[c] = keep(i, J0+c) / (N (1 - p)): the mask of those keys for every
    row, compared bit for bit with the oracle's Philox mask (2 heads)."""
    import io_aware_tiled_03_amd as fa
    B, H = 1, 2
    nk = min(d, N - J0)
    q = np.zeros((B, H, N, d))
    k = np.random.default_rng(1).standard_normal((B, H, N, d))
    v = np.zeros((B, H, N, d))
    v[:, :, J0 + np.arange(nk), np.arange(nk)] = 1.0
    o, _ = fa.fwd(_dev(q), _dev(k), _dev(v), causal=False, dropout=(p, seed, offset))
    o = to_f64(o)
    pe = orc.dropout_threshold(p) / 256.0
    got = np.rint(o[..., :nk] * N * (1 - pe)).astype(int)
    assert set(np.unique(got)) <= {0, 1}
    for h in range(H):
        want = orc.dropout_keep(np.arange(N), J0 + np.arange(nk), h, seed, offset, p)
        assert np.array_equal(got[0, h].astype(bool), want), (h, int((got[0, h] != want).sum()))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N,I0", [(256, 0), (1024, 384), (2048, 2048 - 64)])
def test_dropout_mask_backward_exact(N, I0, d):
    """Through dV = (P o Z)^T dO with P uniform and dO rows I0 .. I0+d-1 one-hot:
    dV_j[c] = keep(I0+c, j) / (N (1 - p)), the mask as the dK/dV kernel
    regenerates it (one lane per key), compared bit for bit."""
    import io_aware_tiled_03_amd as fa
    B, H, p, seed, offset = 1, 2, 0.25, 99, 3
    nq = min(d, N - I0)
    q = np.zeros((B, H, N, d))
    k = np.random.default_rng(2).standard_normal((B, H, N, d))
    v = np.random.default_rng(3).standard_normal((B, H, N, d))
    do = np.zeros((B, H, N, d))
    do[:, :, I0 + np.arange(nq), np.arange(nq)] = 1.0
    qd, kd, vd, dod = _dev(q), _dev(k), _dev(v), _dev(do)
    o, lse = fa.fwd(qd, kd, vd, causal=False, dropout=(p, seed, offset))
    _, _, dv = fa.bwd(qd, kd, vd, o, lse, dod, causal=False, dropout=(p, seed, offset))
    dv = to_f64(dv)
    pe = orc.dropout_threshold(p) / 256.0
    got = np.rint(dv[..., :nq] * N * (1 - pe)).astype(int)
    assert set(np.unique(got)) <= {0, 1}
    for h in range(H):
        want = orc.dropout_keep(I0 + np.arange(nq), np.arange(N), h, seed, offset, p).T
        assert np.array_equal(got[0, h].astype(bool), want), (h, int((got[0, h] != want).sum()))


def _fwd(x, tau, causal, drop):
    import io_aware_tiled_03_amd as fa
    q, k, v = (to_device(x[n]) for n in ("q", "k", "v"))
    o, lse = fa.fwd(q, k, v, tau=tau, causal=causal, dropout=drop)
    return to_f64(o), to_f64(lse)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.1, 0.5])
@pytest.mark.parametrize("N", [1, 7, 63, 130, 300])
def test_dropout_fwd_bf16_small(N, p, causal, d):
    x = fa_inputs.dense_inputs(2, 2, N, d, "bf16", 16000 + N)
    tau = 1.0 / np.sqrt(d)
    drop = (p, 2024 + N, 5)
    o, lse = _fwd(x, tau, causal, drop)
    ro, rl = orc.attention_fwd(*(x[n].f64() for n in ("q", "k", "v")), tau, causal,
                               dropout=(drop[1], drop[2], p))
    assert_close(o, ro, "bf16", "O")
    assert_close(lse, rl, "bf16", "LSE", kind="lse")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [33, 257])
def test_dropout_fwd_f32_small(N, causal, d):
    x = fa_inputs.dense_inputs(1, 2, N, d, "f32", 17000 + N)
    tau = 1.0 / np.sqrt(d)
    drop = (0.3, 77, 0)
    o, lse = _fwd(x, tau, causal, drop)
    ro, rl = orc.attention_fwd(*(x[n].f64() for n in ("q", "k", "v")), tau, causal,
                               dropout=(77, 0, 0.3))
    assert_close(o, ro, "f32", "O")
    assert_close(lse, rl, "f32", "LSE", kind="lse")


def test_dropout_zero_is_plain_forward():
    import io_aware_tiled_03_amd as fa
    import torch
    x = fa_inputs.dense_inputs(2, 2, 500, 128, "bf16", 18000)
    q, k, v = (to_device(x[n]) for n in ("q", "k", "v"))
    for causal in (False, True):
        o1, l1 = fa.fwd(q, k, v, causal=causal)
        o2, l2 = fa.fwd(q, k, v, causal=causal, dropout=(0.0, 5, 0))
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def _bwd(x, tau, causal, drop):
    import io_aware_tiled_03_amd as fa
    q, k, v, do = (to_device(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, tau=tau, causal=causal, dropout=drop)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, tau=tau, causal=causal, dropout=drop)
    return {"o": to_f64(o), "dq": to_f64(dq), "dk": to_f64(dk), "dv": to_f64(dv)}


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.1, 0.5])
@pytest.mark.parametrize("N", [7, 130, 300])
def test_dropout_bwd_small(N, p, causal, d):
    x = fa_inputs.dense_inputs(2, 2, N, d, "bf16", 19000 + N, with_do=True)
    tau = 1.0 / np.sqrt(d)
    drop = (p, 4242 + N, 11)
    g = _bwd(x, tau, causal, drop)
    qf, kf, vf, dof = (x[n].f64() for n in ("q", "k", "v", "do"))
    for b in range(2):
        for h in range(2):
            # Exact gradients; the allowance models D formed from the stored
            # bf16 O and the bf16 MFMA operands P o Z and dS: short causal
            # rows put P close to one and Z = 1/(1-p) scales dP up
            ref = orc.attention_bwd_head(qf[b, h], kf[b, h], vf[b, h], dof[b, h], tau, causal,
                                         drop=orc.head_dropout((drop[1], drop[2], p), b * 2 + h))
            extra = bwd_allowance(ref, g["o"][b, h], qf[b, h], kf[b, h], dof[b, h], tau)
            for name in ("dq", "dk", "dv"):
                assert_close(g[name][b, h], ref[name], "bf16", "%s[%d,%d]" % (name, b, h),
                             ulp_allow=True, extra=extra[name])


def test_dropout_workload_shape():
    """The backward workload's shape (4x16x4096x64 bf16, causal) with p = 0.1:
    forward O and the gradients of 2 sampled heads element by element."""
    w = fa_inputs.WORKLOADS[5]
    x = fa_inputs.workload_inputs(w)
    drop = (0.1, 123456789, 0)
    import io_aware_tiled_03_amd as fa
    q, k, v, do = (to_device(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, tau=w.tau, causal=True, dropout=drop)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, tau=w.tau, causal=True, dropout=drop)
    o, dq, dk, dv = (to_f64(t) for t in (o, dq, dk, dv))
    qf, kf, vf, dof = (x[n].f64() for n in ("q", "k", "v", "do"))
    for b, h in ((0, 1), (3, 14)):
        hd = orc.head_dropout((drop[1], drop[2], drop[0]), b * w.H + h)
        ref = orc.attention_bwd_head(qf[b, h], kf[b, h], vf[b, h], dof[b, h], w.tau, True,
                                     drop=hd)
        tag = "next 3: dropout p=0.1, causal 4x16x4096x64 (2 heads)"
        assert_close(o[b, h], ref["o"], "bf16", "O[%d,%d]" % (b, h), tag=(tag, "O"))
        for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
            assert_close(got[b, h], ref[name], "bf16", "%s[%d,%d]" % (name, b, h), tag=(tag, name))
