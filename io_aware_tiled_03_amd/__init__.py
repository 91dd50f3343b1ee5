"""Python binding of libfa.so, the gfx950 exact-attention library.

Argument marshalling only: every call goes through the C ABI declared in
``include/fa.h`` and every step of the computation runs in the library's HIP
kernels.  PyTorch supplies device memory and the current stream.  If the
library has not been built this module raises instead of computing anything
elsewhere.

    o, lse = fwd(q, k, v, tau=None, causal=False)
    o, lse = decode(q, k, v, seqlens_k, tau=None, num_splits=0)
    o, lse = decode_paged(q, k_pages, v_pages, block_table, seqlens_k, tau=None)
    dq, dk, dv = bwd(q, k, v, o, lse, do, tau=None, causal=False)

Tensors are contiguous [B, H, N, d] on the GPU, dtype bfloat16 or float32.
"""
from __future__ import annotations

import ctypes
import math
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_F32, FA_BF16 = 0, 1
STATUS = {0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_UNSUPPORTED",
          4: "FA_ERR_WORKSPACE", 5: "FA_ERR_HIP", 6: "FA_ERR_ALIGN", 7: "FA_ERR_ARG",
          8: "FA_ERR_SCRATCH"}

# (name, restype, argtypes) of every symbol that fa.h declares.
_P, _I, _F, _Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_U64, _U32 = ctypes.c_ulonglong, ctypes.c_uint
SIGNATURES = {
    "fa_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _P]),
    "fa_fwd_window": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _I, _P]),
    "fa_fwd_dropout": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _F, _U64, _U32, _I, _P]),
    "fa_fwd_block_sparse": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _I, _I, _I, _I,
                                 _P]),
    "fa_decode_workspace_bytes": (_Z, [_I, _I, _I, _I, _I]),
    "fa_decode_num_splits": (_I, [_I, _I, _I, _I, _I]),
    "fa_decode": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _P, _I, _P, _Z, _I, _P]),
    "fa_decode_noalloc": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _P, _I, _I, _P]),
    "fa_decode_paged_num_splits": (_I, [_I, _I, _I, _I, _I, _I, _I]),
    "fa_decode_paged_workspace_bytes": (_Z, [_I, _I, _I, _I, _I, _I, _I]),
    "fa_decode_paged": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _I, _P,
                             _Z, _I, _P]),
    "fa_bwd_workspace_bytes": (_Z, [_I, _I, _I]),
    "fa_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _Z, _I, _P]),
    "fa_bwd_stage": (_I, [_I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _Z,
                          _I, _P]),
    "fa_bwd_window": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _P, _Z,
                           _I, _P]),
    "fa_bwd_dropout": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _F, _U64,
                            _U32, _P, _Z, _I, _P]),
    "fa_bwd_block_sparse_workspace_bytes": (_Z, [_I, _I, _I, _I]),
    "fa_bwd_block_sparse": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P,
                                 _I, _I, _I, _P, _Z, _I, _P]),
    "fa_status_string": (ctypes.c_char_p, [_I]),
}

# (name, restype, argtypes) of every symbol that fa_calib.h declares (measurement aid, not
# part of the attention path).
CALIB_SIGNATURES = {
    "fa_calib_mix_count": (_I, []),
    "fa_calib_mix_name": (ctypes.c_char_p, [_I]),
    "fa_calib_flops": (ctypes.c_double, [_I, _I, _I]),
    "fa_calib_mfma": (_I, [_I, _I, _I, _P, _P, _P]),
    "fa_calib_lds_count": (_I, []),
    "fa_calib_lds_name": (ctypes.c_char_p, [_I]),
    "fa_calib_lds_bytes": (ctypes.c_double, [_I, _I, _I]),
    "fa_calib_lds": (_I, [_I, _I, _I, _P, _P]),
    "fa_calib_hbm_read": (_I, [_P, _Z, _I, _P, _P]),
}

_lib = None


class FAError(RuntimeError):
    def __init__(self, fn, status, text):
        super().__init__("%s failed: %s (%s)" % (fn, STATUS.get(status, status), text))
        self.status = status


def lib():
    """Load libfa.so (once) and declare its signatures; raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libfa.so is not built at %s; run "
                               "`python -m io_aware_tiled_03_amd.build`" % LIB_PATH)
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in list(SIGNATURES.items()) + list(CALIB_SIGNATURES.items()):
            fn = getattr(handle, name)
            fn.restype, fn.argtypes = res, args
        _lib = handle
    return _lib


def check(fn, status):
    if status != 0:
        raise FAError(fn, status, lib().fa_status_string(status).decode())


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_F32
    raise TypeError("unsupported dtype %s (bfloat16 or float32)" % t.dtype)


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _expect(t, name, shape, dtype):
    """t has exactly this shape and dtype and is contiguous (ValueError otherwise).

    The library receives bare device pointers: a tensor smaller than the
    kernels assume, or of another element size, would be read or written out
    of bounds on the device, so every tensor is checked before any call."""
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _same_gpu(tensors):
    """Every tensor lives on one and the same GPU (ValueError otherwise)."""
    dev = None
    for name, t in tensors:
        if not t.is_cuda:
            raise ValueError("%s must be a GPU tensor" % name)
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("%s is on %s, the other tensors on %s" % (name, t.device, dev))


def _block_args(block_mask, block_size, H, N):
    import torch
    bq, bk = (int(x) for x in block_size)
    if bq < 1 or bk < 1:
        raise ValueError("block sizes must be positive")
    if block_mask.dtype != torch.uint8 or block_mask.dim() != 3:
        raise ValueError("block_mask must be a uint8 tensor [mask_heads, nbq, nbk]")
    heads = int(block_mask.shape[0])
    if heads not in (1, H):
        raise ValueError("block_mask has %d heads, expected 1 or %d" % (heads, H))
    _expect(block_mask, "block_mask", (heads, -(-N // bq), -(-N // bk)), torch.uint8)
    return block_mask.data_ptr(), heads, bq, bk


def _check_dense(named, lse, B, H, N, d, dt):
    """named: (name, tensor) pairs that must all be [B, H, N, d] of dtype dt."""
    import torch
    for n, t in named:
        _expect(t, n, (B, H, N, d), dt)
    _expect(lse, "lse", (B, H, N), torch.float32)


def fwd(q, k, v, tau=None, causal=False, o=None, lse=None, window=None, sinks=0, dropout=None,
        block_mask=None, block_size=(128, 128)):
    """O = softmax(tau Q K^T [+causal mask]) V and LSE, via fa_fwd.

    With window (causal only): the causal mask restricted to the `window` most
    recent keys plus the first `sinks` keys, via fa_fwd_window.
    With dropout = (p, seed, offset): dropout on P, via fa_fwd_dropout.
    With block_mask (uint8 [1 or H, ceil(N/bq), ceil(N/bk)], block_size = (bq, bk)):
    block-sparse attention, via fa_fwd_block_sparse."""
    import torch
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    _dtype_code(q)
    tau = 1.0 / math.sqrt(d) if tau is None else float(tau)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_dense((("q", q), ("k", k), ("v", v), ("o", o)), lse, B, H, N, d, q.dtype)
    devs = [("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse)]
    if block_mask is not None:
        if window is not None or dropout is not None:
            raise ValueError("block-sparse attention takes no window and no dropout")
        bargs = _block_args(block_mask, block_size, H, N)
        _same_gpu(devs + [("block_mask", block_mask)])
        st = lib().fa_fwd_block_sparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                       lse.data_ptr(), B, H, N, d, tau, int(bool(causal)),
                                       *bargs, _dtype_code(q), _stream(q))
        check("fa_fwd_block_sparse", st)
        return o, lse
    _same_gpu(devs)
    if dropout is not None:
        if window is not None:
            raise ValueError("dropout is supported with no mask or the causal mask")
        p, seed, offset = dropout
        st = lib().fa_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  lse.data_ptr(), B, H, N, d, tau, int(bool(causal)), float(p),
                                  int(seed), int(offset), _dtype_code(q), _stream(q))
        check("fa_fwd_dropout", st)
        return o, lse
    if window is not None:
        if not causal:
            raise ValueError("a sliding window applies to the causal mask")
        st = lib().fa_fwd_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                 lse.data_ptr(), B, H, N, d, tau, int(window), int(sinks),
                                 _dtype_code(q), _stream(q))
        check("fa_fwd_window", st)
        return o, lse
    st = lib().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      B, H, N, d, tau, int(bool(causal)), _dtype_code(q), _stream(q))
    check("fa_fwd", st)
    return o, lse


def decode_workspace_bytes(B, H, N_max, d, num_splits=0):
    return int(lib().fa_decode_workspace_bytes(B, H, N_max, d, num_splits))


def decode_num_splits(B, H, N_max, d, num_splits=0):
    return int(lib().fa_decode_num_splits(B, H, N_max, d, num_splits))


def _workspace(ws, need, device, name="workspace"):
    """A caller's workspace (any dtype, contiguous, at least `need` bytes, which
    the library checks again) or a new one of `need` bytes."""
    import torch
    if ws is None:
        return torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    if not ws.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if ws.numel() * ws.element_size() < need:
        raise ValueError("%s holds %d bytes, the call needs %d"
                         % (name, ws.numel() * ws.element_size(), need))
    return ws


def decode(q, k, v, seqlens_k, tau=None, num_splits=0, o=None, lse=None, workspace=None):
    """One query per (b, h) against the KV cache rows [0, seqlens_k[b]), via fa_decode.

    q [B, H, 1, d]; k, v [B, H, N_max, d] of q's dtype; seqlens_k int32 [B]."""
    import torch
    if k.dim() != 4:
        raise ValueError("k must be [B, H, N_max, d]")
    B, H, N_max, d = k.shape
    _dtype_code(q)
    tau = 1.0 / math.sqrt(d) if tau is None else float(tau)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device) if lse is None else lse
    _expect(q, "q", (B, H, 1, d), q.dtype)
    _expect(k, "k", (B, H, N_max, d), q.dtype)
    _expect(v, "v", (B, H, N_max, d), q.dtype)
    _expect(o, "o", (B, H, 1, d), q.dtype)
    _expect(lse, "lse", (B, H), torch.float32)
    _expect(seqlens_k, "seqlens_k", (B,), torch.int32)
    need = decode_workspace_bytes(B, H, N_max, d, num_splits)
    workspace = _workspace(workspace, need, q.device)
    _same_gpu([("q", q), ("k", k), ("v", v), ("seqlens_k", seqlens_k), ("o", o), ("lse", lse),
               ("workspace", workspace)])
    st = lib().fa_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), seqlens_k.data_ptr(), B, H,
                         N_max, d, tau, o.data_ptr(), lse.data_ptr(), int(num_splits),
                         workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                         _dtype_code(q), _stream(q))
    check("fa_decode", st)
    return o, lse


def decode_noalloc(q, k, v, seqlens_k, tau=None, num_splits=0, o=None, lse=None):
    """fa_decode without a workspace argument, via fa_decode_noalloc: the split
    partials live in the library's fixed per-GPU array, so the call allocates
    nothing when o and lse are given.  Arguments as for decode."""
    import torch
    if k.dim() != 4:
        raise ValueError("k must be [B, H, N_max, d]")
    B, H, N_max, d = k.shape
    _dtype_code(q)
    tau = 1.0 / math.sqrt(d) if tau is None else float(tau)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device) if lse is None else lse
    _expect(q, "q", (B, H, 1, d), q.dtype)
    _expect(k, "k", (B, H, N_max, d), q.dtype)
    _expect(v, "v", (B, H, N_max, d), q.dtype)
    _expect(o, "o", (B, H, 1, d), q.dtype)
    _expect(lse, "lse", (B, H), torch.float32)
    _expect(seqlens_k, "seqlens_k", (B,), torch.int32)
    _same_gpu([("q", q), ("k", k), ("v", v), ("seqlens_k", seqlens_k), ("o", o), ("lse", lse)])
    st = lib().fa_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), seqlens_k.data_ptr(),
                                 B, H, N_max, d, tau, o.data_ptr(), lse.data_ptr(),
                                 int(num_splits), _dtype_code(q), _stream(q))
    check("fa_decode_noalloc", st)
    return o, lse


def decode_paged_num_splits(B, Hq, Hkv, page_size, max_pages, d, num_splits=0):
    return int(lib().fa_decode_paged_num_splits(B, Hq, Hkv, page_size, max_pages, d, num_splits))


def decode_paged_workspace_bytes(B, Hq, Hkv, page_size, max_pages, d, num_splits=0):
    return int(lib().fa_decode_paged_workspace_bytes(B, Hq, Hkv, page_size, max_pages, d,
                                                     num_splits))


def decode_paged(q, k_pages, v_pages, block_table, seqlens_k, tau=None, num_splits=0, o=None,
                 lse=None, workspace=None):
    """Decode with grouped KV heads over a paged cache, via fa_decode_paged.

    q [B, Hq, 1, d]; k_pages, v_pages [num_pages, Hkv, page_size, d];
    block_table int32 [B, max_pages]; seqlens_k int32 [B]."""
    import torch
    if q.dim() != 4 or k_pages.dim() != 4 or block_table.dim() != 2:
        raise ValueError("q [B, Hq, 1, d], pages [num_pages, Hkv, page_size, d], "
                         "block_table [B, max_pages]")
    B, Hq, _, d = q.shape
    num_pages, Hkv, page_size, _ = k_pages.shape
    max_pages = block_table.shape[1]
    _dtype_code(q)
    tau = 1.0 / math.sqrt(d) if tau is None else float(tau)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if lse is None else lse
    _expect(q, "q", (B, Hq, 1, d), q.dtype)
    _expect(k_pages, "k_pages", (num_pages, Hkv, page_size, d), q.dtype)
    _expect(v_pages, "v_pages", (num_pages, Hkv, page_size, d), q.dtype)
    _expect(block_table, "block_table", (B, max_pages), torch.int32)
    _expect(seqlens_k, "seqlens_k", (B,), torch.int32)
    _expect(o, "o", (B, Hq, 1, d), q.dtype)
    _expect(lse, "lse", (B, Hq), torch.float32)
    need = decode_paged_workspace_bytes(B, Hq, Hkv, page_size, max_pages, d, num_splits)
    workspace = _workspace(workspace, need, q.device)
    _same_gpu([("q", q), ("k_pages", k_pages), ("v_pages", v_pages), ("block_table", block_table),
               ("seqlens_k", seqlens_k), ("o", o), ("lse", lse), ("workspace", workspace)])
    st = lib().fa_decode_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(),
                               block_table.data_ptr(), seqlens_k.data_ptr(), B, Hq, Hkv,
                               num_pages, page_size, max_pages, d, tau, o.data_ptr(),
                               lse.data_ptr(), int(num_splits), workspace.data_ptr(),
                               workspace.numel() * workspace.element_size(), _dtype_code(q),
                               _stream(q))
    check("fa_decode_paged", st)
    return o, lse


def bwd_workspace_bytes(B, H, N):
    return int(lib().fa_bwd_workspace_bytes(B, H, N))


def bwd_block_sparse_workspace_bytes(B, H, N, d):
    return int(lib().fa_bwd_block_sparse_workspace_bytes(B, H, N, d))


def bwd(q, k, v, o, lse, do, tau=None, causal=False, dq=None, dk=None, dv=None, workspace=None,
        stage=None, window=None, sinks=0, dropout=None, block_mask=None, block_size=(128, 128)):
    """dQ, dK, dV of fa_fwd's output given dO, via fa_bwd (workspace holds D on return).

    With stage in (0, 1) only that kernel is enqueued, via fa_bwd_stage (0: dQ
    and D, 1: dK and dV, which reads D).  With
    window (causal only): the backward of the sliding-window forward, via fa_bwd_window.
    With dropout = (p, seed, offset): the backward of fa_fwd_dropout, via fa_bwd_dropout.
    With block_mask: the backward of fa_fwd_block_sparse, via fa_bwd_block_sparse; the
    default workspace there is bwd_block_sparse_workspace_bytes, with which long key-tile
    lists are split over several workgroups (a D-sized one walks each list whole)."""
    import torch
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    _dtype_code(q)
    tau = 1.0 / math.sqrt(d) if tau is None else float(tau)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_dense((("q", q), ("k", k), ("v", v), ("o", o), ("do", do), ("dq", dq), ("dk", dk),
                  ("dv", dv)), lse, B, H, N, d, q.dtype)
    bargs = None
    if block_mask is not None:
        bargs = _block_args(block_mask, block_size, H, N)
    # a block-sparse call splits long key-tile lists when given the larger
    # workspace (allocated here by default); D alone is enough otherwise
    want = (bwd_block_sparse_workspace_bytes(B, H, N, d) if block_mask is not None and workspace is None
            else bwd_workspace_bytes(B, H, N))
    workspace = _workspace(workspace, want, q.device)
    _same_gpu([("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("do", do), ("dq", dq),
               ("dk", dk), ("dv", dv), ("workspace", workspace)]
              + ([("block_mask", block_mask)] if block_mask is not None else []))
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
            do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, tau,
            int(bool(causal)), workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), _dtype_code(q), _stream(q))
    if block_mask is not None:
        if window is not None or dropout is not None or stage is not None:
            raise ValueError("block-sparse backward: no window, no dropout, whole backward only")
        check("fa_bwd_block_sparse", lib().fa_bwd_block_sparse(*(args[:15] + bargs + args[15:])))
    elif dropout is not None:
        if window is not None or stage is not None:
            raise ValueError("dropout backward: no window, whole backward only")
        p, seed, offset = dropout
        dargs = args[:15] + (float(p), int(seed), int(offset)) + args[15:]
        check("fa_bwd_dropout", lib().fa_bwd_dropout(*dargs))
    elif window is not None:
        if not causal or stage is not None:
            raise ValueError("a sliding window applies to the causal mask, whole backward only")
        wargs = args[:14] + (int(window), int(sinks)) + args[15:]
        check("fa_bwd_window", lib().fa_bwd_window(*wargs))
    elif stage is None:
        check("fa_bwd", lib().fa_bwd(*args))
    else:
        check("fa_bwd_stage", lib().fa_bwd_stage(int(stage), *args))
    return dq, dk, dv


CALIB_SEED_BYTES = 65536


def calib_mixes():
    """Descriptions of the synthetic matrix-core mixes (fa_calib.h), by id."""
    L = lib()
    return [L.fa_calib_mix_name(i).decode() for i in range(L.fa_calib_mix_count())]


def calib_flops(mix, grid, iters):
    return lib().fa_calib_flops(int(mix), int(grid), int(iters))


def calib_mfma(mix, grid, iters, seed, out):
    """One launch of synthetic mix `mix` on the current stream (fa_calib_mfma).

    seed: a device tensor of at least 64 KB (any bf16 values); out: a float32
    device tensor of grid * 256 elements."""
    import torch
    if seed.numel() * seed.element_size() < CALIB_SEED_BYTES or not seed.is_contiguous():
        raise ValueError("seed must be a contiguous tensor of at least %d bytes" % CALIB_SEED_BYTES)
    _expect(out, "out", (int(grid) * 256,), torch.float32)
    _same_gpu([("seed", seed), ("out", out)])
    check("fa_calib_mfma", lib().fa_calib_mfma(int(mix), int(grid), int(iters), seed.data_ptr(),
                                               out.data_ptr(), _stream(out)))
    return out


def calib_lds_patterns():
    """Descriptions of the LDS read patterns (fa_calib.h), by id."""
    L = lib()
    return [L.fa_calib_lds_name(i).decode() for i in range(L.fa_calib_lds_count())]


def calib_lds_bytes(pattern, grid, iters):
    return lib().fa_calib_lds_bytes(int(pattern), int(grid), int(iters))


def calib_lds(pattern, grid, iters, out):
    """One launch of LDS read pattern `pattern` on the current stream (fa_calib_lds);
    out: an int32 device tensor of grid * 512 elements."""
    import torch
    _expect(out, "out", (int(grid) * 512,), torch.int32)
    _same_gpu([("out", out)])
    check("fa_calib_lds", lib().fa_calib_lds(int(pattern), int(grid), int(iters), out.data_ptr(),
                                             _stream(out)))
    return out


def calib_hbm_read(buf, grid, out):
    """One streaming read of the whole of `buf` (a contiguous device tensor whose size in bytes
    is a multiple of 16) on the current stream (fa_calib_hbm_read); out: an int32 device tensor of
    grid * 256 elements."""
    import torch
    nbytes = buf.numel() * buf.element_size()
    if not buf.is_contiguous() or nbytes % 16:
        raise ValueError("buf must be contiguous and a multiple of 16 bytes")
    _expect(out, "out", (int(grid) * 256,), torch.int32)
    _same_gpu([("buf", buf), ("out", out)])
    check("fa_calib_hbm_read", lib().fa_calib_hbm_read(buf.data_ptr(), nbytes, int(grid),
                                                       out.data_ptr(), _stream(out)))
    return out
