"""GPU parity of block-sparse attention (fa_fwd_block_sparse,
fa_bwd_block_sparse) against the float64 oracle."""
import numpy as np
import pytest

import fa_inputs
from oracle import attention as orc
from tests.util import assert_close, bwd_allowance, to_device, to_f64

pytestmark = pytest.mark.gpu


def _mask(heads, N, bq, bk, density, seed, causal):
    rng = np.random.default_rng(seed)
    nbq, nbk = -(-N // bq), -(-N // bk)
    m = (rng.random((heads, nbq, nbk)) < density).astype(np.uint8)
    m[:, 0, 0] = 1
    return m


def _lse_close(got, ref, what):
    """Equal -inf pattern (rows with no visible key), finite parts within the LSE bound."""
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), what
    live = np.isfinite(ref)
    assert_close(got[live], ref[live], "bf16", what, kind="lse")


def _run_fwd(x, tau, causal, mask, bq, bk):
    import io_aware_tiled_03_amd as fa
    import torch
    q, k, v = (to_device(x[n]) for n in ("q", "k", "v"))
    o, lse = fa.fwd(q, k, v, tau=tau, causal=causal, block_mask=torch.from_numpy(mask).cuda(),
                    block_size=(bq, bk))
    return to_f64(o), to_f64(lse)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bq,bk", [(32, 32), (64, 128), (128, 64), (256, 32)])
@pytest.mark.parametrize("N,density", [(100, 0.5), (257, 0.3), (1000, 0.6)])
def test_block_sparse_fwd_small(N, density, bq, bk, causal, d):
    B, H = 2, 2
    x = fa_inputs.dense_inputs(B, H, N, d, "bf16", 20000 + N + bq + bk)
    tau = 1.0 / np.sqrt(d)
    mask = _mask(H if bq == bk else 1, N, bq, bk, density, N + bq, causal)
    o, lse = _run_fwd(x, tau, causal, mask, bq, bk)
    ro, rl = orc.attention_fwd(*(x[n].f64() for n in ("q", "k", "v")), tau, causal,
                               block=(mask, bq, bk))
    assert_close(o, ro, "bf16", "O")
    _lse_close(lse, rl, "LSE")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_block_sparse_visibility_exact(d, causal):
    """Q = 0 gives uniform weights over the visible keys; V one-hot for keys
    J0 .. J0+d-1 makes O_i[c] > 0 exactly when key J0+c is visible to row i
    (and 0 otherwise), so the pattern of zeros is the visibility, bit for bit."""
    import io_aware_tiled_03_amd as fa
    import torch
    N, bq, bk, J0 = 768, 64, 32, 256
    mask = _mask(2, N, bq, bk, 0.4, 7, causal)
    q = torch.zeros(1, 2, N, d, dtype=torch.bfloat16, device="cuda")
    k = torch.randn(1, 2, N, d, generator=torch.Generator().manual_seed(3)).to("cuda", torch.bfloat16)
    v = torch.zeros(1, 2, N, d)
    v[:, :, J0 + torch.arange(d), torch.arange(d)] = 1.0
    o, _ = fa.fwd(q, k, v.to("cuda", torch.bfloat16), causal=causal,
                  block_mask=torch.from_numpy(mask).cuda(), block_size=(bq, bk))
    got = to_f64(o)[0] > 0
    for h in range(2):
        vis = orc.visible(np.arange(N), J0 + np.arange(d), causal, block=(mask[h], bq, bk))
        assert np.array_equal(got[h], vis), (h, int((got[h] != vis).sum()))


def test_block_sparse_all_ones_is_dense():
    import io_aware_tiled_03_amd as fa
    import torch
    x = fa_inputs.dense_inputs(2, 2, 640, 128, "bf16", 21000)
    q, k, v = (to_device(x[n]) for n in ("q", "k", "v"))
    ones = torch.ones(1, 5, 5, dtype=torch.uint8, device="cuda")
    for causal in (False, True):
        o1, l1 = fa.fwd(q, k, v, causal=causal)
        o2, l2 = fa.fwd(q, k, v, causal=causal, block_mask=ones, block_size=(128, 128))
        assert (o1.float() - o2.float()).abs().max() <= 2e-2
        assert (l1 - l2).abs().max() <= 1e-3


def test_block_sparse_long_prefill_bigbird_pattern():
    """The long prefill shape (1x32x16384x128, causal) with a band of 3 key
    blocks around the diagonal plus the first key block (global tokens),
    128 x 128 blocks: sampled rows of 4 heads against the oracle."""
    w = fa_inputs.WORKLOADS[3]
    x = fa_inputs.workload_inputs(w)
    nb = w.N // 128
    i, j = np.meshgrid(np.arange(nb), np.arange(nb), indexing="ij")
    mask = ((np.abs(i - j) <= 1) | (j == 0)).astype(np.uint8)[None]
    o, lse = _run_fwd(x, w.tau, True, mask, 128, 128)
    qf, kf, vf = (x[n].f64() for n in ("q", "k", "v"))
    rng = np.random.Generator(np.random.PCG64(35))
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 255, 256, 8191, 8192, 16383],
                                     rng.integers(0, w.N, 100)]))
    for h in (0, 11, 25, 31):
        ro, rl = orc.attention_fwd_head(qf[0, h], kf[0, h], vf[0, h], w.tau, True, rows=rows,
                                        block=(mask[0], 128, 128))
        assert_close(o[0, h, rows], ro, "bf16", "O[h=%d]" % h,
                     tag=("next 4: block-sparse band+global, 1x32x16384x128 (sampled rows)", "O"))
        _lse_close(lse[0, h, rows], rl, "LSE[h=%d]" % h)


def _run_bwd(x, tau, causal, mask, bq, bk):
    import io_aware_tiled_03_amd as fa
    import torch
    q, k, v, do = (to_device(x[n]) for n in ("q", "k", "v", "do"))
    m = torch.from_numpy(mask).cuda()
    o, lse = fa.fwd(q, k, v, tau=tau, causal=causal, block_mask=m, block_size=(bq, bk))
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, tau=tau, causal=causal, block_mask=m,
                        block_size=(bq, bk))
    return {"o": to_f64(o), "dq": to_f64(dq), "dk": to_f64(dk), "dv": to_f64(dv)}


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bq,bk", [(32, 32), (64, 128), (128, 64)])
@pytest.mark.parametrize("N,density", [(100, 0.5), (300, 0.3), (700, 0.6)])
def test_block_sparse_bwd_small(N, density, bq, bk, causal, d):
    B, H = 2, 2
    x = fa_inputs.dense_inputs(B, H, N, d, "bf16", 22000 + N + bq + bk, with_do=True)
    tau = 1.0 / np.sqrt(d)
    mask = _mask(H, N, bq, bk, density, 2 * N + bk, causal)
    g = _run_bwd(x, tau, causal, mask, bq, bk)
    qf, kf, vf, dof = (x[n].f64() for n in ("q", "k", "v", "do"))
    for b in range(B):
        for h in range(H):
            # Exact gradients; the allowance models D formed from the stored
            # bf16 O and the bf16 MFMA operands: sparse rows can have few
            # visible keys (P close to one)
            ref = orc.attention_bwd_head(qf[b, h], kf[b, h], vf[b, h], dof[b, h], tau, causal,
                                         block=(mask[h], bq, bk))
            extra = bwd_allowance(ref, g["o"][b, h], qf[b, h], kf[b, h], dof[b, h], tau)
            for name in ("dq", "dk", "dv"):
                assert_close(g[name][b, h], ref[name], "bf16", "%s[%d,%d]" % (name, b, h),
                             ulp_allow=True, extra=extra[name])


def test_block_sparse_bwd_workload_shape():
    """The backward workload's shape (4x16x4096x64 bf16, causal) with a
    random 50% mask of 128 x 128 blocks (diagonal kept), one mask per head:
    2 sampled heads element by element at the stated bounds."""
    w = fa_inputs.WORKLOADS[5]
    x = fa_inputs.workload_inputs(w)
    nb = w.N // 128
    mask = (np.random.default_rng(36).random((w.H, nb, nb)) < 0.5).astype(np.uint8)
    mask[:, np.arange(nb), np.arange(nb)] = 1
    g = _run_bwd(x, w.tau, True, mask, 128, 128)
    qf, kf, vf, dof = (x[n].f64() for n in ("q", "k", "v", "do"))
    for b, h in ((1, 2), (3, 9)):
        ref = orc.attention_bwd_head(qf[b, h], kf[b, h], vf[b, h], dof[b, h], w.tau, True,
                                     block=(mask[h], 128, 128))
        for name in ("dq", "dk", "dv"):
            assert_close(g[name][b, h], ref[name], "bf16", "%s[%d,%d]" % (name, b, h),
                         tag=("next 4: block-sparse 50% of 128x128 blocks, backward 4x16x4096x64 "
                              "(2 heads)", name))


def _global_band_mask(heads, N, blk, causal):
    """Band of +-1 blocks, the first key block global (every query block sees
    it) and, without the causal mask, the first query block global too."""
    nb = -(-N // blk)
    bi, bj = np.meshgrid(np.arange(nb), np.arange(nb), indexing="ij")
    m = (np.abs(bi - bj) <= 1) | (bj == 0)
    if not causal:
        m |= bi == 0
    return np.broadcast_to(m.astype(np.uint8), (heads, nb, nb)).copy()


def _bwd_with_workspace(x, tau, causal, mask, blk, ws_bytes):
    import io_aware_tiled_03_amd as fa
    import torch
    q, k, v, do = (to_device(x[n]) for n in ("q", "k", "v", "do"))
    m = torch.from_numpy(mask).cuda()
    o, lse = fa.fwd(q, k, v, tau=tau, causal=causal, block_mask=m, block_size=(blk, blk))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(2):   # twice: the split sum must not depend on which part ends last
        dq, dk, dv = fa.bwd(q, k, v, o, lse, do, tau=tau, causal=causal, dq=None, dk=None,
                            dv=None, workspace=ws, block_mask=m, block_size=(blk, blk))
        outs.append({"o": to_f64(o), "dq": to_f64(dq), "dk": to_f64(dk), "dv": to_f64(dv)})
    return outs


def _check_bwd_heads(x, tau, causal, mask, blk, g, label):
    qf, kf, vf, dof = (x[n].f64() for n in ("q", "k", "v", "do"))
    B, H = qf.shape[:2]
    for b in range(B):
        for h in range(H):
            ref = orc.attention_bwd_head(qf[b, h], kf[b, h], vf[b, h], dof[b, h], tau, causal,
                                         block=(mask[h], blk, blk))
            extra = bwd_allowance(ref, g["o"][b, h], qf[b, h], kf[b, h], dof[b, h], tau)
            for name in ("dq", "dk", "dv"):
                assert_close(g[name][b, h], ref[name], "bf16", "%s %s[%d,%d]" % (label, name, b, h),
                             ulp_allow=True, extra=extra[name])


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,blk", [(2048, 64), (2000, 32)])
def test_block_sparse_bwd_split_long_lists(N, blk, d, causal):
    """A global key block makes key tile 0's list of query tiles (32 of them
    at N = 2048; N = 2000 leaves a ragged last tile) several times longer than
    the others: with the split workspace its dK/dV is computed in parts by
    several workgroups and summed by the last part.  Checked against the
    oracle, bit-identical over two calls, and against the same call with a
    D-only workspace (every list walked whole), which must agree within the
    bounds."""
    import io_aware_tiled_03_amd as fa
    B, H = 1, 2
    x = fa_inputs.dense_inputs(B, H, N, d, "bf16", 23000 + N + d + causal, with_do=True)
    tau = 1.0 / np.sqrt(d)
    mask = _global_band_mask(H, N, blk, causal)
    split = _bwd_with_workspace(x, tau, causal, mask, blk, fa.bwd_block_sparse_workspace_bytes(B, H, N, d))
    for name in ("dq", "dk", "dv"):
        assert np.array_equal(split[0][name], split[1][name]), name
    _check_bwd_heads(x, tau, causal, mask, blk, split[0], "split")
    whole = _bwd_with_workspace(x, tau, causal, mask, blk, fa.bwd_workspace_bytes(B, H, N))
    _check_bwd_heads(x, tau, causal, mask, blk, whole[0], "whole")
    # dQ does not take part in the split: identical either way
    assert np.array_equal(split[0]["dq"], whole[0]["dq"])


def test_block_sparse_bwd_split_few_slots():
    """Slots for only the first long list: the first head's key tile 0 is
    split, the second head's is walked whole (the plan runs out of slots);
    both heads match the oracle."""
    import io_aware_tiled_03_amd as fa
    B, H, N, d, blk = 1, 2, 2048, 64, 64
    x = fa_inputs.dense_inputs(B, H, N, d, "bf16", 23500, with_do=True)
    tau = 1.0 / np.sqrt(d)
    mask = _global_band_mask(H, N, blk, True)
    full = fa.bwd_block_sparse_workspace_bytes(B, H, N, d)
    slot = 2 * 128 * d * 4
    fixed = full - 32 * slot        # 32 slots by default at this size
    g = _bwd_with_workspace(x, tau, True, mask, blk, fixed + 5 * slot)
    for name in ("dq", "dk", "dv"):
        assert np.array_equal(g[0][name], g[1][name]), name
    _check_bwd_heads(x, tau, True, mask, blk, g[0], "5 slots")
