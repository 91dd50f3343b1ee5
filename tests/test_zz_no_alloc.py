"""fa_decode_noalloc (split partials in the library's fixed per-GPU array)
against fa_decode (caller workspace) through the C ABI: two calls in a row,
the first using nearly all of the fixed array, the second smaller, each
compared bit for bit with fa_decode on the same inputs and split count, and
the small one also with the float64 oracle at the stated bounds."""
import ctypes

import numpy as np
import pytest

import fa_inputs
from oracle import attention as orc
from tests.util import assert_close, to_device, to_f64

pytestmark = pytest.mark.gpu

SCRATCH = 16 << 20   # FA_DECODE_NOALLOC_SCRATCH_BYTES in fa.h


def _noalloc(fa, q, k, v, sl, tau, num_splits):
    import torch
    B, H, N_max, d = k.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    st = fa.lib().fa_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), sl.data_ptr(), B, H,
                                    N_max, d, tau, o.data_ptr(), lse.data_ptr(), num_splits,
                                    fa.FA_BF16, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, fa.lib().fa_status_string(st)
    return o, lse


def test_noalloc_matches_decode_two_calls():
    import io_aware_tiled_03_amd as fa
    import torch
    # 1: 32 x 32 heads, 3968-key caches (31 x 128), 31 splits of 128 keys:
    # 15.6 MiB of partials, 98% of the fixed array
    B, H, N_max, d, S = 32, 32, 3968, 128, 31
    assert fa.decode_workspace_bytes(B, H, N_max, d, S) <= SCRATCH
    assert fa.decode_workspace_bytes(B, H, N_max, d, S) > SCRATCH * 0.9
    g = torch.Generator(device="cuda")
    g.manual_seed(31000)
    q = torch.randn(B, H, 1, d, device="cuda", generator=g).to(torch.bfloat16)
    k = torch.randn(B, H, N_max, d, device="cuda", generator=g).to(torch.bfloat16)
    v = torch.randn(B, H, N_max, d, device="cuda", generator=g).to(torch.bfloat16)
    sl = torch.randint(1, N_max + 1, (B,), device="cuda", generator=g, dtype=torch.int32)
    tau = 1.0 / np.sqrt(d)
    o_ref, l_ref = fa.decode(q, k, v, sl, tau=tau, num_splits=S)
    o, lse = _noalloc(fa, q, k, v, sl, tau, S)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    del q, k, v, o_ref, o

    # 2: smaller, another head size and split count, host-recipe inputs
    lens = [1, 700, 1500, 999]
    x = fa_inputs.decode_inputs(4, 3, 1500, 64, "bf16", 31100, seqlens=lens)
    q, k, v = (to_device(x[n]) for n in ("q", "k", "v"))
    sl = torch.from_numpy(x["seqlens"]).to("cuda")
    tau = 0.125
    o_ref, l_ref = fa.decode(q, k, v, sl, tau=tau, num_splits=5)
    o2, l2 = _noalloc(fa, q, k, v, sl, tau, 5)
    torch.cuda.synchronize()
    assert torch.equal(o2, o_ref) and torch.equal(l2, l_ref)
    ro, rl = orc.decode_fwd(x["q"].f64(), x["k"].f64(), x["v"].f64(), x["seqlens"], tau)
    assert_close(to_f64(o2), ro, "bf16", "O")
    assert_close(to_f64(l2), rl, "bf16", "LSE", kind="lse")


def test_noalloc_binding_and_oversize_refusal():
    import io_aware_tiled_03_amd as fa
    import torch
    x = fa_inputs.decode_inputs(2, 2, 2100, 128, "bf16", 31200, seqlens=[2100, 5])
    q, k, v = (to_device(x[n]) for n in ("q", "k", "v"))
    sl = torch.from_numpy(x["seqlens"]).to("cuda")
    o_ref, l_ref = fa.decode(q, k, v, sl, num_splits=3)
    o, lse = fa.decode_noalloc(q, k, v, sl, num_splits=3)
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    # a split count whose partials exceed the fixed array is refused, nothing launched
    big = torch.empty(64, 32, 1, 128, dtype=torch.bfloat16, device="cuda")
    need = fa.decode_workspace_bytes(64, 32, 8192, 128, 64)
    assert need > SCRATCH
    st = fa.lib().fa_decode_noalloc(big.data_ptr(), big.data_ptr(), big.data_ptr(), sl.data_ptr(),
                                    64, 32, 8192, 128, 0.1, big.data_ptr(), lse.data_ptr(), 64,
                                    fa.FA_BF16, None)
    assert st == 8
