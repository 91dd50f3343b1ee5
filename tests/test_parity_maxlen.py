"""Parity at the longest sequence the library accepts: one head of N = 2^20
keys (the largest offsets into every tensor), causal.  The oracle cannot form
the N x N matrices, so it is asked for what it can compute exactly: sampled
rows of O, LSE and dQ (each from its own full score row), and dK, dV of the
last keys (under the causal mask only the last rows see them).  The split-KV
decode is checked over a cache of 2^20 keys."""
import numpy as np
import pytest

import fa_inputs
from oracle import attention as orc
from tests.util import assert_close, to_device, to_f64

pytestmark = pytest.mark.gpu

N = 1 << 20
_EDGES = [0, 1, 63, 64, 127, 128, 255, 256, 1023, 1024, 65535, 65536, 524287, 524288,
          N - 257, N - 256, N - 129, N - 128, N - 2, N - 1]


def _rows(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.unique(np.concatenate([_EDGES, rng.integers(0, N, 12)]))


def _pick(t, rows):
    """Rows of a [1, 1, N, ...] GPU tensor, widened to float64 on the host."""
    import torch
    idx = torch.from_numpy(rows).to(t.device)
    return to_f64(t[0, 0].index_select(0, idx))


@pytest.mark.parametrize("d", [64, 128])
def test_fwd_max_length(d):
    import io_aware_tiled_03_amd as fa
    x = fa_inputs.dense_inputs(1, 1, N, d, "bf16", 17000 + d)
    tau = 1.0 / np.sqrt(d)
    q, k, v = (to_device(x[n]) for n in ("q", "k", "v"))
    o, lse = fa.fwd(q, k, v, tau=tau, causal=True)
    rows = _rows(17010 + d)
    ro, rl = orc.attention_fwd_head(x["q"].f64()[0, 0], x["k"].f64()[0, 0], x["v"].f64()[0, 0],
                                    tau, True, rows=rows, chunk=16)
    assert_close(_pick(o, rows), ro, "bf16", "O")
    assert_close(to_f64(lse)[0, 0, rows], rl, "bf16", "LSE", kind="lse")
    assert bool(o.isfinite().all()) and bool(lse.isfinite().all())


def test_bwd_max_length():
    import io_aware_tiled_03_amd as fa
    d = 64
    x = fa_inputs.dense_inputs(1, 1, N, d, "bf16", 17100, with_do=True)
    nk = 64   # the last 64 keys: half of the dK/dV kernel's last 128-key tile
    last = np.arange(N - nk, N)
    # The last keys are twice their own queries (exact in bf16): each of the
    # last rows gives its own key most of its weight, so these keys' gradients
    # are of order one (with iid keys they would be of order 1/N).
    x["k"].raw[0, 0, last] = fa_inputs.bf16_bits((2.0 * x["q"].f64()[0, 0, last]).astype(np.float32))
    tau = 1.0 / np.sqrt(d)
    q, k, v, do = (to_device(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, tau=tau, causal=True)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, tau=tau, causal=True)
    qf, kf, vf, dof = (x[n].f64()[0, 0] for n in ("q", "k", "v", "do"))
    rows = _rows(17110)
    rdq, _ = orc.attention_dq_rows(qf, kf, vf, dof, tau, True, rows, chunk=16)
    assert_close(_pick(dq, rows), rdq, "bf16", "dQ")
    rdk, rdv = orc.attention_dkdv_last_keys(qf, kf, vf, dof, tau, nk)
    assert np.abs(rdk).max() > 0.1 and np.abs(rdv).max() > 0.5   # the check has teeth
    assert_close(_pick(dk, last), rdk, "bf16", "dK (last keys)")
    assert_close(_pick(dv, last), rdv, "bf16", "dV (last keys)")
    for t in (dq, dk, dv):
        assert bool(t.isfinite().all())


def test_decode_max_length():
    import io_aware_tiled_03_amd as fa
    import torch
    d = 128
    x = fa_inputs.decode_inputs(2, 1, N, d, "bf16", 17200, seqlens=[N, N - 1000])
    tau = 1.0 / np.sqrt(d)
    o, lse = fa.decode(to_device(x["q"]), to_device(x["k"]), to_device(x["v"]),
                       torch.from_numpy(x["seqlens"]).to("cuda"), tau=tau)
    o, lse = to_f64(o), to_f64(lse)
    qf = x["q"].f64()
    for b in range(2):   # widen one sequence's valid rows at a time
        L = int(x["seqlens"][b])
        kb = fa_inputs.bf16_bits_to_f64(x["k"].raw[b:b + 1, :, :L])
        vb = fa_inputs.bf16_bits_to_f64(x["v"].raw[b:b + 1, :, :L])
        ro, rl = orc.decode_fwd(qf[b:b + 1], kb, vb, np.array([L]), tau)
        assert_close(o[b], ro[0], "bf16", "O[%d]" % b)
        assert_close(lse[b], rl[0], "bf16", "LSE[%d]" % b, kind="lse")
