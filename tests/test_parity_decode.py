"""GPU parity of fa_decode (split-KV + LSE merge) against the float64 oracle."""
import numpy as np
import pytest

import fa_inputs
from oracle import attention as orc
from tests.util import assert_close, to_device, to_f64

pytestmark = pytest.mark.gpu


def _run(x, d, tau, num_splits):
    import io_aware_tiled_03_amd as fa
    import torch
    q, k, v = (to_device(x[n]) for n in ("q", "k", "v"))
    sl = torch.from_numpy(x["seqlens"]).to("cuda")
    o, lse = fa.decode(q, k, v, sl, tau=tau, num_splits=num_splits)
    return to_f64(o), to_f64(lse)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("num_splits", [0, 1, 3, 7])
def test_decode_small(num_splits, d, dtype):
    seqlens = [1, 2, 255, 300, 64, 65]
    B, H, N_max = len(seqlens), 3, 300
    x = fa_inputs.decode_inputs(B, H, N_max, d, dtype, 9000 + d + num_splits, seqlens=seqlens)
    tau = 1.0 / np.sqrt(d)
    o, lse = _run(x, d, tau, num_splits)
    ro, rl = orc.decode_fwd(x["q"].f64(), x["k"].f64(), x["v"].f64(), x["seqlens"], tau)
    assert_close(o, ro, dtype, "O")
    assert_close(lse, rl, dtype, "LSE", kind="lse")


@pytest.mark.parametrize("num_splits", [1, 2])
def test_decode_empty_sequence(num_splits):
    """L_b = 0 (clamped length): no visible key, O = 0 and LSE = -inf by definition
    of an empty sum; the other sequences are unaffected.  One split stores the
    result from the split kernel itself, two go through the merge."""
    x = fa_inputs.decode_inputs(2, 2, 128, 128, "bf16", 9100, seqlens=[0, 100])
    o, lse = _run(x, 128, 0.1, num_splits)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
    ro, rl = orc.decode_fwd(x["q"].f64(), x["k"].f64(), x["v"].f64(), x["seqlens"], 0.1,
                            batches=[1])
    assert_close(o[1], ro[1], "bf16", "O")
    assert_close(lse[1], rl[1], "bf16", "LSE", kind="lse")


def test_decode_workload_full():
    """Workload 4 at full size: B=64, H=32, N_max=8192, d=128, L_b ~ U[1024, 8192],
    NaN-poisoned padding; every (b, h) checked against the oracle."""
    w = fa_inputs.WORKLOADS[4]
    x = fa_inputs.workload_decode_inputs(w)
    o, lse = _run(x, w.d, w.tau, 0)
    qf = x["q"].f64()
    ro, rl = np.empty_like(o), np.empty_like(lse)
    for b in range(w.B):   # widen one sequence's valid rows at a time
        L = int(x["seqlens"][b])
        kb = fa_inputs.bf16_bits_to_f64(x["k"].raw[b:b + 1, :, :L])
        vb = fa_inputs.bf16_bits_to_f64(x["v"].raw[b:b + 1, :, :L])
        ob, lb = orc.decode_fwd(qf[b:b + 1], kb, vb, np.array([L]), w.tau)
        ro[b], rl[b] = ob[0], lb[0]
    tag = "4: split-KV decode 64x32, L~U[1024,8192], d=128"
    assert_close(o, ro, "bf16", "O", tag=(tag, "O"))
    assert_close(lse, rl, "bf16", "LSE", kind="lse", tag=(tag, "LSE"))


def test_decode_one_split_matches_merge_bits():
    """One split written by the split kernel directly equals, bit for bit, the
    merge of that one split (weight exp(0) = 1, ln 1 = 0), which is what two
    splits of which the second is empty (L_b <= chunk) reduce to."""
    x = fa_inputs.decode_inputs(3, 2, 256, 64, "bf16", 9300, seqlens=[64, 100, 128])
    o1, l1 = _run(x, 64, 0.125, 1)   # chunk 256: one split, no merge
    o2, l2 = _run(x, 64, 0.125, 2)   # chunk 128: the second split is empty, merged
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_decode_splits_agree():
    """Different split counts give the same answer within rounding."""
    x = fa_inputs.decode_inputs(4, 4, 2048, 128, "bf16", 9200, seqlens=[2048, 1, 1500, 777])
    outs = [_run(x, 128, 0.09, s) for s in (1, 2, 5, 32)]
    for o, lse in outs[1:]:
        assert np.abs(o - outs[0][0]).max() <= 1e-2
        assert np.abs(lse - outs[0][1]).max() <= 1e-4
