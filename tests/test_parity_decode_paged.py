"""GPU parity of fa_decode_paged (grouped KV heads, paged cache) against the
float64 oracle."""
import numpy as np
import pytest

import fa_inputs
from oracle import attention as orc
from tests.util import assert_close, to_device, to_f64

pytestmark = pytest.mark.gpu


def _run(x, tau, num_splits=0):
    import io_aware_tiled_03_amd as fa
    import torch
    q, kp, vp = (to_device(x[n]) for n in ("q", "k_pages", "v_pages"))
    bt = torch.from_numpy(x["block_table"]).to("cuda")
    sl = torch.from_numpy(x["seqlens"]).to("cuda")
    o, lse = fa.decode_paged(q, kp, vp, bt, sl, tau=tau, num_splits=num_splits)
    return to_f64(o), to_f64(lse)


def _oracle(x, tau, batches=None):
    """Per-sequence oracle: gather that sequence's pages (raw bf16) first, then widen."""
    B, Hq = x["q"].raw.shape[:2]
    o = np.full((B, Hq, 1, x["q"].raw.shape[-1]), np.nan)
    lse = np.full((B, Hq), np.nan)
    P = x["k_pages"].raw.shape[2]
    for b in (range(B) if batches is None else batches):
        L = int(x["seqlens"][b])
        npg = max(1, (L + P - 1) // P)
        ids = x["block_table"][b, :npg]
        kp = fa_inputs.bf16_bits_to_f64(x["k_pages"].raw[ids])
        vp = fa_inputs.bf16_bits_to_f64(x["v_pages"].raw[ids])
        ob, lb = orc.decode_paged(x["q"].f64()[b:b + 1], kp, vp, np.arange(npg)[None, :],
                                  np.array([L]), tau)
        o[b], lse[b] = ob[0], lb[0]
    return o, lse


SEQLENS = [1, 15, 16, 17, 31, 32, 33, 300, 129]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (8, 1), (10, 2), (16, 1), (32, 1), (40, 1),
                                    (6, 3)])
@pytest.mark.parametrize("page_size", [16, 64])
def test_paged_small(page_size, Hq, Hkv, d):
    x = fa_inputs.paged_decode_inputs(len(SEQLENS), Hq, Hkv, page_size, d, "bf16",
                                      9300 + Hq + Hkv + d + page_size, SEQLENS)
    tau = 1.0 / np.sqrt(d)
    o, lse = _run(x, tau)
    ro, rl = _oracle(x, tau)
    assert_close(o, ro, "bf16", "O")
    assert_close(lse, rl, "bf16", "LSE", kind="lse")


@pytest.mark.parametrize("num_splits", [1, 2, 3, 9])
@pytest.mark.parametrize("page_size", [16, 32, 256])
def test_paged_splits_and_pages(num_splits, page_size):
    """Split boundaries (multiples of 128 keys) against page boundaries,
    ragged last blocks, and a sequence filling its whole page table."""
    seqlens = [1100, 7, 128, 129, 1024, 555]
    x = fa_inputs.paged_decode_inputs(len(seqlens), 8, 2, page_size, 128, "bf16",
                                      9400 + num_splits + page_size, seqlens)
    o, lse = _run(x, 0.088, num_splits)
    ro, rl = _oracle(x, 0.088)
    assert_close(o, ro, "bf16", "O")
    assert_close(lse, rl, "bf16", "LSE", kind="lse")


def test_paged_split_layout_edges():
    """Two splits of 1024 keys: split 0 takes the whole first chunk, the last
    split the rest.  Lengths: both splits whole (L = 2 * 1024), the last split
    empty (1024), the first split empty and the last one holding 1023 keys or
    a single key, and one key after a whole chunk (1025)."""
    import io_aware_tiled_03_amd as fa
    seqlens = [2048, 1024, 1023, 1025, 1]
    x = fa_inputs.paged_decode_inputs(len(seqlens), 8, 2, 16, 64, "bf16", 9450, seqlens)
    assert fa.decode_paged_num_splits(len(seqlens), 8, 2, 16, 2048 // 16, 64, 2) == 2
    o, lse = _run(x, 0.125, 2)
    ro, rl = _oracle(x, 0.125)
    assert_close(o, ro, "bf16", "O")
    assert_close(lse, rl, "bf16", "LSE", kind="lse")


def test_paged_empty_sequence():
    """L_b = 0: O = 0 and LSE = -inf; the other sequences are unaffected."""
    x = fa_inputs.paged_decode_inputs(3, 8, 2, 16, 128, "bf16", 9500, [0, 40, 0])
    o, lse = _run(x, 0.1)
    assert np.all(o[[0, 2]] == 0) and np.all(np.isneginf(lse[[0, 2]]))
    ro, rl = _oracle(x, 0.1, batches=[1])
    assert_close(o[1], ro[1], "bf16", "O")
    assert_close(lse[1], rl[1], "bf16", "LSE", kind="lse")


def test_paged_matches_dense_decode():
    """With Hkv = Hq and the same draws, paged decode equals the dense decode
    kernel's result within rounding (the two kernels share no code)."""
    import io_aware_tiled_03_amd as fa
    import torch
    seqlens = [700, 33, 1024]
    x = fa_inputs.paged_decode_inputs(3, 4, 4, 32, 128, "bf16", 9600, seqlens)
    dense = fa_inputs.decode_inputs(3, 4, 1024, 128, "bf16", 9600, seqlens=seqlens)
    o1, l1 = _run(x, 0.09)
    q, k, v = (to_device(dense[n]) for n in ("q", "k", "v"))
    o2, l2 = fa.decode(q, k, v, torch.from_numpy(dense["seqlens"]).cuda(), tau=0.09)
    assert np.abs(o1 - to_f64(o2)).max() <= 1e-2
    assert np.abs(l1 - to_f64(l2)).max() <= 1e-4


def test_paged_workload_full():
    """The paged workload at full size (B=64, Hq=32, Hkv=8, 16-token pages,
    d=128, the dense decode workload's key lengths U[1024, 8192]); every
    (b, h) checked against the oracle."""
    w = fa_inputs.PAGED_WORKLOAD
    x = fa_inputs.paged_workload_inputs(w)
    o, lse = _run(x, w.tau)
    ro, rl = _oracle(x, w.tau)
    tag = "next 1: paged GQA decode 64 seq, 32/8 heads, 16-token pages"
    assert_close(o, ro, "bf16", "O", tag=(tag, "O"))
    assert_close(lse, rl, "bf16", "LSE", kind="lse", tag=(tag, "LSE"))
