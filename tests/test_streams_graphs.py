"""The calls run asynchronously on the caller's stream and allocate nothing, so
a caller may issue them on any stream and capture them in a HIP graph.

Both tests compare against eager results on the default stream bit for bit:
the kernels are deterministic (no atomics), so the same inputs give the same
bits whichever stream or graph launches them."""
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
