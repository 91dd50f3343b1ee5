"""The Python binding refuses tensors whose shape, dtype, layout or device do
not match what the kernels will address, before any call into the library.

The library receives bare pointers, so a shorter K, an fp32 O beside bf16
inputs or a small block mask would be read or written out of bounds on the
device.  These tests only build host tensors and assert the raise; a
consistent set of host tensors is refused too (the device check comes last),
so nothing here reaches a kernel."""
import pytest
import torch

import io_aware_tiled_03_amd as fa

B, H, N, D = 2, 3, 40, 64
bf = torch.bfloat16


def _t(*shape, dtype=bf):
    return torch.zeros(*shape, dtype=dtype)


def _dense():
    return [_t(B, H, N, D) for _ in range(3)]


def _raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_fwd_checks_every_tensor():
    q, k, v = _dense()
    _raises("k has shape", fa.fwd, q, _t(B, H, N - 1, D), v)
    _raises("v has dtype", fa.fwd, q, k, _t(B, H, N, D, dtype=torch.float32))
    _raises("o has dtype", fa.fwd, q, k, v, o=_t(B, H, N, D, dtype=torch.float32))
    _raises("o has shape", fa.fwd, q, k, v, o=_t(B, H, N, 2 * D))
    _raises("lse has dtype", fa.fwd, q, k, v, lse=_t(B, H, N))
    _raises("lse has shape", fa.fwd, q, k, v, lse=_t(B, H, N + 1, dtype=torch.float32))
    _raises("k must be contiguous", fa.fwd, q, _t(B, H, D, N).transpose(2, 3), v)
    _raises("q must be", fa.fwd, _t(H, N, D), k, v)
    _raises("must be a GPU tensor", fa.fwd, q, k, v)
    with pytest.raises(TypeError):
        fa.fwd(_t(B, H, N, D, dtype=torch.float16), k, v)


def test_block_mask_shape_and_heads():
    q, k, v = _dense()
    # ceil(40 / 32) = 2 query blocks, ceil(40 / 64) = 1 key block
    good = _t(1, 2, 1, dtype=torch.uint8)
    _raises("block_mask has shape", fa.fwd, q, k, v, block_mask=_t(1, 1, 1, dtype=torch.uint8),
            block_size=(32, 64))
    _raises("block_mask has 2 heads", fa.fwd, q, k, v, block_mask=_t(2, 2, 1, dtype=torch.uint8),
            block_size=(32, 64))
    _raises("uint8", fa.fwd, q, k, v, block_mask=_t(1, 2, 1), block_size=(32, 64))
    _raises("must be a GPU tensor", fa.fwd, q, k, v, block_mask=good, block_size=(32, 64))
    do = _t(B, H, N, D)
    o, lse = _t(B, H, N, D), _t(B, H, N, dtype=torch.float32)
    _raises("block_mask has shape", fa.bwd, q, k, v, o, lse, do,
            block_mask=_t(H, 3, 1, dtype=torch.uint8), block_size=(32, 64))


def test_bwd_checks_every_tensor():
    q, k, v = _dense()
    o, do = _t(B, H, N, D), _t(B, H, N, D)
    lse = _t(B, H, N, dtype=torch.float32)
    _raises("o has shape", fa.bwd, q, k, v, _t(B, H, N, D + 1), lse, do)
    _raises("do has dtype", fa.bwd, q, k, v, o, lse, _t(B, H, N, D, dtype=torch.float32))
    _raises("lse has dtype", fa.bwd, q, k, v, o, _t(B, H, N), do)
    _raises("lse has shape", fa.bwd, q, k, v, o, _t(B, H, dtype=torch.float32), do)
    _raises("dq has shape", fa.bwd, q, k, v, o, lse, do, dq=_t(B, H, N - 2, D))
    _raises("dk has dtype", fa.bwd, q, k, v, o, lse, do, dk=_t(B, H, N, D, dtype=torch.float32))
    _raises("dv has shape", fa.bwd, q, k, v, o, lse, do, dv=_t(1, H, N, D))
    _raises("workspace holds", fa.bwd, q, k, v, o, lse, do, workspace=_t(4, dtype=torch.float32))
    _raises("must be a GPU tensor", fa.bwd, q, k, v, o, lse, do)


def test_decode_checks_every_tensor():
    Nm = 96
    q = _t(B, H, 1, D)
    k, v = _t(B, H, Nm, D), _t(B, H, Nm, D)
    sl = torch.full((B,), Nm, dtype=torch.int32)
    _raises("q has shape", fa.decode, _t(B, H, 2, D), k, v, sl)
    _raises("v has shape", fa.decode, q, k, _t(B, H, Nm - 1, D), sl)
    _raises("k has dtype", fa.decode, q, _t(B, H, Nm, D, dtype=torch.float32), v, sl)
    _raises("seqlens_k has dtype", fa.decode, q, k, v, sl.long())
    _raises("seqlens_k has shape", fa.decode, q, k, v, torch.zeros(B + 1, dtype=torch.int32))
    _raises("lse has shape", fa.decode, q, k, v, sl, lse=_t(B, dtype=torch.float32))
    _raises("o has dtype", fa.decode, q, k, v, sl, o=_t(B, H, 1, D, dtype=torch.float32))
    _raises("workspace holds", fa.decode, q, k, v, sl, num_splits=4,
            workspace=_t(8, dtype=torch.uint8))
    _raises("must be a GPU tensor", fa.decode, q, k, v, sl)


def test_decode_paged_checks_every_tensor():
    Hq, Hkv, P, pages, maxp = 4, 2, 16, 10, 5
    q = _t(B, Hq, 1, D)
    kp, vp = _t(pages, Hkv, P, D), _t(pages, Hkv, P, D)
    table = torch.zeros(B, maxp, dtype=torch.int32)
    sl = torch.full((B,), 20, dtype=torch.int32)
    _raises("v_pages has shape", fa.decode_paged, q, kp, _t(pages - 1, Hkv, P, D), table, sl)
    _raises("k_pages has dtype", fa.decode_paged, q, _t(pages, Hkv, P, D, dtype=torch.float32),
            vp, table, sl)
    _raises("block_table has dtype", fa.decode_paged, q, kp, vp, table.long(), sl)
    _raises("block_table has shape", fa.decode_paged, q, kp, vp,
            torch.zeros(B + 1, maxp, dtype=torch.int32), sl)
    _raises("seqlens_k has shape", fa.decode_paged, q, kp, vp, table,
            torch.zeros(1, dtype=torch.int32))
    _raises("lse has shape", fa.decode_paged, q, kp, vp, table, sl,
            lse=_t(B, Hkv, dtype=torch.float32))
    _raises("must be a GPU tensor", fa.decode_paged, q, kp, vp, table, sl)
