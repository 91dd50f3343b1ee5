"""The calls run asynchronously on the caller's stream and allocate nothing, so
a caller may issue them on any stream and capture them in a HIP graph.

The tests compare against eager results on the default stream bit for bit:
the kernels are deterministic (no atomic accumulation; the block-sparse
backward's split parts are summed in a fixed order), so the same inputs give
the same bits whichever stream or graph launches them."""
import numpy as np
import pytest

import fa_inputs
from tests.util import to_device

pytestmark = pytest.mark.gpu

B, H, N, D = 2, 3, 300, 64
TAU = 0.125


def _inputs(seed):
    import torch
    x = fa_inputs.dense_inputs(B, H, N, D, "bf16", seed, with_do=True)
    t = {n: to_device(x[n]) for n in ("q", "k", "v", "do")}
    t["seq"] = torch.tensor([N, 17], dtype=torch.int32, device="cuda")
    t["qd"] = t["q"][:, :, -1:, :].contiguous()
    return t


def _buffers(fa, t):
    import torch
    q = t["q"]
    return {
        "o": torch.empty_like(q), "lse": torch.empty(B, H, N, device="cuda"),
        "dq": torch.empty_like(q), "dk": torch.empty_like(q), "dv": torch.empty_like(q),
        "ws": torch.empty(fa.bwd_workspace_bytes(B, H, N) // 4, device="cuda"),
        "od": torch.empty_like(t["qd"]), "lsed": torch.empty(B, H, device="cuda"),
        "wsd": torch.empty(fa.decode_workspace_bytes(B, H, N, D), dtype=torch.uint8,
                           device="cuda"),
    }


def _path(fa, t, b):
    """Forward (causal), backward, decode into preallocated buffers."""
    fa.fwd(t["q"], t["k"], t["v"], TAU, True, b["o"], b["lse"])
    fa.bwd(t["q"], t["k"], t["v"], b["o"], b["lse"], t["do"], TAU, True, b["dq"], b["dk"],
           b["dv"], b["ws"])
    fa.decode(t["qd"], t["k"], t["v"], t["seq"], TAU, 0, b["od"], b["lsed"], b["wsd"])


NAMES = ("o", "lse", "dq", "dk", "dv", "od", "lsed")


def test_calls_follow_the_given_stream():
    import torch
    import io_aware_tiled_03_amd as fa
    t = _inputs(16000)
    ref = _buffers(fa, t)
    _path(fa, t, ref)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    got = _buffers(fa, t)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _path(fa, t, got)
        done = torch.cuda.Event()
        done.record(side)
    done.synchronize()   # waits for the side stream's work only
    for n in NAMES:
        assert torch.equal(got[n], ref[n]), n


def test_graph_capture_replays_match_eager():
    import torch
    import io_aware_tiled_03_amd as fa
    t = _inputs(16100)
    ref = _buffers(fa, t)
    _path(fa, t, ref)
    torch.cuda.synchronize()

    b = _buffers(fa, t)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up launch outside the capture
        _path(fa, t, b)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _path(fa, t, b)
    other = _inputs(16200)
    for rep in range(3):
        for n in NAMES:
            b[n].zero_()                   # cleared eagerly, outside the graph
        _path(fa, other, _buffers(fa, other))   # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in NAMES:
            assert torch.equal(b[n], ref[n]), (rep, n)
    assert np.isfinite(b["lse"].cpu().numpy()).all()


def test_block_sparse_split_backward_in_a_graph():
    """The block-sparse backward with the split workspace enqueues its count
    and plan passes and the helper grid; captured in a graph and replayed
    between unrelated eager calls, it gives the eager bits each time (the
    plan is rewritten by every replay, so nothing carries over)."""
    import torch
    import io_aware_tiled_03_amd as fa
    Bs, Hs, Ns, Ds, blk = 1, 2, 2048, 64, 64
    nb = Ns // blk
    bi, bj = np.meshgrid(np.arange(nb), np.arange(nb), indexing="ij")
    mask = torch.from_numpy(np.broadcast_to(((np.abs(bi - bj) <= 1) | (bj == 0)).astype(np.uint8),
                                            (Hs, nb, nb)).copy()).cuda()
    x = fa_inputs.dense_inputs(Bs, Hs, Ns, Ds, "bf16", 16300, with_do=True)
    q, k, v, do = (to_device(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, TAU, True, block_mask=mask, block_size=(blk, blk))
    ws = torch.empty(fa.bwd_block_sparse_workspace_bytes(Bs, Hs, Ns, Ds), dtype=torch.uint8,
                     device="cuda")
    outs = [torch.empty_like(q) for _ in range(3)]

    def run():
        fa.bwd(q, k, v, o, lse, do, TAU, True, outs[0], outs[1], outs[2], ws, block_mask=mask,
               block_size=(blk, blk))

    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up launch outside the capture
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    other = _inputs(16400)
    for rep in range(3):
        for t in outs:
            t.zero_()
        _path(fa, other, _buffers(fa, other))   # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("dq", "dk", "dv"), outs, ref):
            assert torch.equal(got, want), (rep, name)
