"""Host-side checks of libfa.so: it loads, exports every symbol fa.h declares, and
rejects invalid arguments with the documented status before launching anything.
None of these calls reaches a kernel, so they run without a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    import io_aware_tiled_03_amd as fa
    if not os.path.exists(fa.LIB_PATH):
        pytest.skip("libfa.so not built")
    return fa, fa.lib()


def _declared(header="fa.h"):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    import io_aware_tiled_03_amd as fa
    assert _declared() == sorted(fa.SIGNATURES)
    assert _declared("fa_calib.h") == sorted(fa.CALIB_SIGNATURES)


def test_every_header_is_covered():
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == ["fa.h", "fa_calib.h"]


def test_library_exports_every_declared_symbol():
    fa, lib = _lib()
    for name in _declared() + _declared("fa_calib.h"):
        assert hasattr(lib, name), name


def test_calib_host_checks():
    """The synthetic-mix entry point validates its arguments before launching."""
    fa, lib = _lib()
    n = lib.fa_calib_mix_count()
    assert n >= 2
    assert all(lib.fa_calib_mix_name(i) for i in range(n))
    assert lib.fa_calib_mix_name(n) is None and lib.fa_calib_mix_name(-1) is None
    # mix 0: one wave per SIMD, 8 chains; 4 waves x iters x 8 x 32768 per workgroup
    assert lib.fa_calib_flops(0, 2, 10) == 2 * 4 * 10 * 8 * 32768.0
    assert lib.fa_calib_flops(n, 2, 10) == 0.0
    assert lib.fa_calib_mfma(0, 1, 2, None, P, None) == 1
    assert lib.fa_calib_mfma(0, 1, 2, P + 8, P, None) == 6
    assert lib.fa_calib_mfma(n, 1, 2, P, P, None) == 7
    assert lib.fa_calib_mfma(0, 0, 2, P, P, None) == 7
    assert lib.fa_calib_mfma(0, 65537, 2, P, P, None) == 7
    assert lib.fa_calib_mfma(0, 1, 3, P, P, None) == 7
    assert lib.fa_calib_mfma(0, 1, 0, P, P, None) == 7
    m = lib.fa_calib_lds_count()
    assert m >= 2 and all(lib.fa_calib_lds_name(i) for i in range(m))
    assert lib.fa_calib_lds_name(m) is None
    # pattern 0: row reads, 1 KB per wave read; 8 waves x 8 reads per step
    assert lib.fa_calib_lds_bytes(0, 3, 5) == 3 * 8 * 5 * 8 * 1024.0
    assert lib.fa_calib_lds(0, 1, 1, None, None) == 1
    assert lib.fa_calib_lds(0, 1, 1, P + 4, None) == 6
    assert lib.fa_calib_lds(m, 1, 1, P, None) == 7
    assert lib.fa_calib_lds(0, 0, 1, P, None) == 7
    assert lib.fa_calib_lds(0, 1, 0, P, None) == 7
    assert lib.fa_calib_hbm_read(None, 16, 1, P, None) == 1
    assert lib.fa_calib_hbm_read(P + 8, 16, 1, P, None) == 6
    assert lib.fa_calib_hbm_read(P, 0, 1, P, None) == 7
    assert lib.fa_calib_hbm_read(P, 24, 1, P, None) == 7
    assert lib.fa_calib_hbm_read(P, 16, 0, P, None) == 7


def test_status_strings():
    fa, lib = _lib()
    for code in range(9):
        assert lib.fa_status_string(code)
    assert lib.fa_status_string(99) == b"unknown status"


P = 4096  # a fake, 16-byte aligned non-null address: never dereferenced on failure paths


def _fwd(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=16, d=64, tau=0.125, causal=0, dtype=1)
    a.update(kw)
    return lib.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                      a["tau"], a["causal"], a["dtype"], None)


def test_fwd_rejects_bad_arguments():
    fa, lib = _lib()
    assert _fwd(lib, q=None) == 1
    assert _fwd(lib, lse=None) == 1
    assert _fwd(lib, N=0) == 2
    assert _fwd(lib, B=-1) == 2
    assert _fwd(lib, N=(1 << 20) + 1) == 2
    assert _fwd(lib, d=96) == 3
    assert _fwd(lib, dtype=7) == 3
    assert _fwd(lib, causal=2) == 3
    assert _fwd(lib, tau=0.0) == 7
    assert _fwd(lib, tau=float("nan")) == 7
    assert _fwd(lib, tau=float("inf")) == 7
    assert _fwd(lib, q=P + 8) == 6
    assert _fwd(lib, lse=P + 2) == 6


def test_fwd_window_rejects_bad_arguments():
    fa, lib = _lib()
    args = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=16, d=64, tau=0.125, w=4, s=0, dtype=1)
    def call(**kw):
        a = dict(args); a.update(kw)
        return lib.fa_fwd_window(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"],
                                 a["d"], a["tau"], a["w"], a["s"], a["dtype"], None)
    assert call(v=None) == 1
    assert call(N=0) == 2
    assert call(d=32) == 3
    assert call(w=0) == 7
    assert call(s=-1) == 7
    assert call(tau=-0.5) == 7
    assert call(o=P + 4) == 6


def test_dropout_rejects_bad_arguments():
    fa, lib = _lib()
    f = [P, P, P, P, P, 1, 1, 16, 64, 0.125, 1, 0.1, 5, 0, 1, None]
    bad = list(f); bad[11] = -0.1
    assert lib.fa_fwd_dropout(*bad) == 7
    bad = list(f); bad[11] = 0.999
    assert lib.fa_fwd_dropout(*bad) == 7
    bad = list(f); bad[11] = float("nan")
    assert lib.fa_fwd_dropout(*bad) == 7
    bad = list(f); bad[10] = 3
    assert lib.fa_fwd_dropout(*bad) == 3
    bad = list(f); bad[0] = None
    assert lib.fa_fwd_dropout(*bad) == 1
    b = [P, P, P, P, P, P, P, P, P, 1, 2, 64, 64, 0.125, 1, 0.1, 5, 0, P, 1 << 20, 1, None]
    bad = list(b); bad[15] = 1.0
    assert lib.fa_bwd_dropout(*bad) == 7
    bad = list(b); bad[20] = 9
    assert lib.fa_bwd_dropout(*bad) == 3    # unknown dtype
    bad = list(b); bad[18] = None
    assert lib.fa_bwd_dropout(*bad) == 4


def test_block_sparse_rejects_bad_arguments():
    fa, lib = _lib()
    f = [P, P, P, P, P, 1, 2, 256, 64, 0.125, 1, P, 1, 64, 64, 1, None]
    bad = list(f); bad[11] = None
    assert lib.fa_fwd_block_sparse(*bad) == 1
    bad = list(f); bad[13] = 48
    assert lib.fa_fwd_block_sparse(*bad) == 7     # not a power of two
    bad = list(f); bad[14] = 16
    assert lib.fa_fwd_block_sparse(*bad) == 7     # below 32
    bad = list(f); bad[12] = 3
    assert lib.fa_fwd_block_sparse(*bad) == 2     # mask heads neither 1 nor H
    bad = list(f); bad[7] = 262145
    assert lib.fa_fwd_block_sparse(*bad) == 2     # tile lists would overflow LDS
    bad = list(f); bad[15] = 0
    assert lib.fa_fwd_block_sparse(*bad) == 3     # bf16 only
    b = [P, P, P, P, P, P, P, P, P, 1, 2, 256, 64, 0.125, 1, P, 1, 64, 64, P, 1 << 20, 1, None]
    bad = list(b); bad[17] = 2048
    assert lib.fa_bwd_block_sparse(*bad) == 7
    bad = list(b); bad[19] = None
    assert lib.fa_bwd_block_sparse(*bad) == 4


def _dec(lib, **kw):
    a = dict(q=P, k=P, v=P, sl=P, B=2, H=2, N=100, d=128, tau=0.1, o=P, lse=P, ns=0, ws=P,
             wsb=1 << 30, dtype=1)
    a.update(kw)
    return lib.fa_decode(a["q"], a["k"], a["v"], a["sl"], a["B"], a["H"], a["N"], a["d"],
                         a["tau"], a["o"], a["lse"], a["ns"], a["ws"], a["wsb"], a["dtype"], None)


def test_decode_rejects_bad_arguments():
    fa, lib = _lib()
    assert _dec(lib, sl=None) == 1
    assert _dec(lib, N=0) == 2
    assert _dec(lib, d=32) == 3
    assert _dec(lib, ns=-1) == 7
    assert _dec(lib, ns=5000) == 7
    assert _dec(lib, ws=None) == 4
    need = lib.fa_decode_workspace_bytes(2, 2, 100, 128, 0)
    assert need > 0
    assert _dec(lib, wsb=need - 1) == 4
    assert _dec(lib, ws=P + 4) == 6


def test_decode_split_rule():
    fa, lib = _lib()
    # automatic splits: one when N_max <= 1024, else >= 256 keys per split
    # unless that would exceed 16384 workgroups
    assert lib.fa_decode_num_splits(8, 16, 1024, 64, 0) == 1
    assert lib.fa_decode_num_splits(8, 16, 2048, 64, 0) == 8
    assert lib.fa_decode_num_splits(1, 1, 8192, 128, 0) == 32
    assert lib.fa_decode_num_splits(64, 32, 8192, 128, 0) == 8
    assert lib.fa_decode_num_splits(1, 1, 100, 128, 0) == 1
    # explicit counts use equal chunks rounded up to 64 keys
    assert lib.fa_decode_num_splits(1, 1, 300, 64, 7) == 5
    assert lib.fa_decode_num_splits(1, 1, 300, 64, 1) == 1
    s = lib.fa_decode_num_splits(64, 32, 8192, 128, 0)
    assert lib.fa_decode_workspace_bytes(64, 32, 8192, 128, 0) == s * 64 * 32 * 129 * 4
    assert lib.fa_decode_workspace_bytes(1, 1, 100, 96, 0) == 0


def _paged(lib, **kw):
    a = dict(q=P, kp=P, vp=P, bt=P, sl=P, B=2, Hq=8, Hkv=2, npages=10, ps=16, mp=8, d=128,
             tau=0.1, o=P, lse=P, ns=0, ws=P, wsb=1 << 30, dtype=1)
    a.update(kw)
    return lib.fa_decode_paged(a["q"], a["kp"], a["vp"], a["bt"], a["sl"], a["B"], a["Hq"],
                               a["Hkv"], a["npages"], a["ps"], a["mp"], a["d"], a["tau"], a["o"],
                               a["lse"], a["ns"], a["ws"], a["wsb"], a["dtype"], None)


def test_decode_paged_rejects_bad_arguments():
    fa, lib = _lib()
    assert _paged(lib, bt=None) == 1
    assert _paged(lib, sl=None) == 1
    assert _paged(lib, Hq=7) == 2          # not a multiple of Hkv
    assert _paged(lib, Hkv=0) == 2
    assert _paged(lib, ps=24) == 2         # not a power of two
    assert _paged(lib, ps=8) == 2          # below 16
    assert _paged(lib, mp=0) == 2
    assert _paged(lib, ps=1 << 16, mp=32) == 2   # more than 2^20 keys
    assert _paged(lib, npages=0) == 2
    assert _paged(lib, d=96) == 3
    assert _paged(lib, dtype=0) == 3       # bf16 only
    assert _paged(lib, tau=-1.0) == 7
    assert _paged(lib, ns=2000) == 7
    assert _paged(lib, ws=None) == 4
    need = lib.fa_decode_paged_workspace_bytes(2, 8, 2, 16, 8, 128, 0)
    assert need > 0
    assert _paged(lib, wsb=need - 1) == 4
    assert _paged(lib, kp=P + 8) == 6
    assert _paged(lib, bt=P + 2) == 6


def test_decode_paged_split_rule():
    fa, lib = _lib()
    # automatic: chunks of >= 512 keys, doubled while the grid would exceed
    # 4096 workgroups; (b, kv head, group of 16 query heads) units
    assert lib.fa_decode_paged_num_splits(64, 32, 8, 16, 512, 128, 0) == 8
    assert lib.fa_decode_paged_num_splits(1, 32, 8, 16, 512, 128, 0) == 16
    assert lib.fa_decode_paged_num_splits(1, 8, 8, 16, 4, 128, 0) == 1
    # explicit counts: equal chunks rounded up to 128 keys
    assert lib.fa_decode_paged_num_splits(1, 8, 8, 16, 20, 128, 7) == 3   # 320 keys, chunk 128
    s = lib.fa_decode_paged_num_splits(64, 32, 8, 16, 512, 128, 0)
    assert lib.fa_decode_paged_workspace_bytes(64, 32, 8, 16, 512, 128, 0) == s * 64 * 32 * 129 * 4
    assert lib.fa_decode_paged_workspace_bytes(1, 8, 3, 16, 4, 128, 0) == 0


def _bwd(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, H=2, N=64, d=64, tau=0.125,
             causal=1, ws=P, wsb=1 << 20, dtype=1)
    a.update(kw)
    return lib.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                      a["dv"], a["B"], a["H"], a["N"], a["d"], a["tau"], a["causal"], a["ws"],
                      a["wsb"], a["dtype"], None)


def test_bwd_rejects_bad_arguments():
    fa, lib = _lib()
    assert _bwd(lib, dv=None) == 1
    assert _bwd(lib, N=0) == 2
    assert _bwd(lib, d=80) == 3
    assert _bwd(lib, dtype=9) == 3
    assert _bwd(lib, ws=None) == 4
    assert _bwd(lib, wsb=1 * 2 * 64 * 4 - 1) == 4
    assert _bwd(lib, dq=P + 2) == 6
    assert lib.fa_bwd_workspace_bytes(1, 2, 64) == 512


def test_bwd_window_rejects_bad_arguments():
    fa, lib = _lib()
    # every call below fails a host-side check, so nothing is launched on the fake pointers
    args = [P, P, P, P, P, P, P, P, P, 1, 2, 64, 64, 0.125, 16, 0, P, 1 << 20, 1, None]
    bad = list(args); bad[14] = 0
    assert lib.fa_bwd_window(*bad) == 7
    bad = list(args); bad[15] = -2
    assert lib.fa_bwd_window(*bad) == 7
    bad = list(args); bad[18] = 9
    assert lib.fa_bwd_window(*bad) == 3    # unknown dtype
    bad = list(args); bad[16] = None
    assert lib.fa_bwd_window(*bad) == 4


def test_bwd_stage_rejects_bad_arguments():
    fa, lib = _lib()
    args = (P, P, P, P, P, P, P, P, P, 1, 2, 64, 64, 0.125, 1, P, 1 << 20, 1, None)
    assert lib.fa_bwd_stage(2, *args) == 7
    assert lib.fa_bwd_stage(3, *args) == 7
    assert lib.fa_bwd_stage(-1, *args) == 7
    bad = list(args); bad[10] = 0
    assert lib.fa_bwd_stage(1, *bad) == 2


def test_binding_refuses_cpu_tensors():
    fa, lib = _lib()
    import torch
    x = torch.zeros(1, 1, 8, 64)
    with pytest.raises(ValueError):
        fa.fwd(x, x, x)
