"""Throughput of the exact-attention path on one MI355X.

One step = one pass of the whole path over the GPT-2-medium-shaped batch
(B=8, H=16, N=1024, d=64, bf16, tau=1/8):
    fa_fwd non-causal, fa_fwd causal, fa_bwd causal (its two kernels enqueued
    one by one through fa_bwd_stage), and fa_decode with one query per sequence
    against the same K/V as the cache (L_b = N for every b).
value = algorithmic TFLOP/s of the step (forward 4*B*H*N^2*d, halved when
causal; backward 10*B*H*N^2*d halved when causal; decode 4*B*H*N*d), from the
wall clock around exactly --steps steps bracketed by device synchronisation.

The line also carries, measured in the same run:
  * "kernels": every call of the step timed with HIP events on the stream the
    library launches on, with TFLOP/s and GB/s of algorithmic work;
  * "roofline": the kernel with the largest share of the step against its
    peak (MFMA bf16 2.5 PFLOP/s; HBM 8 TB/s), with the HBM traffic read from
    the committed rocprofv3 counter summary when it matches the sources;
  * "also_measured": the long causal prefill (1x32x16384x128), the same
    prefill as a sliding-window (local) layer with a 4096-key window and as a
    block-sparse layer (band plus global blocks), the split-KV
    decode (64x32, L_b ~ U[1024, 8192], d=128), the paged decode with grouped
    KV heads (64 sequences, 32 query / 8 KV heads, 16-token pages, the same
    key lengths), the causal backward (4x16x4096x64) and the same shape with
    dropout p = 0.1 (forward and backward) at full size, each against its
    roofline (skip: --no-extra);
  * "cpu_baseline": the float64 oracle on the host over a bounded sample of
    the same step (whole heads, about 10 s of CPU work).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_BF16 = 2.5e15     # dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12           # HBM3E, B/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def src_digest():
    h = hashlib.sha256()
    d = os.path.join(ROOT, "io_aware_tiled_03_amd", "csrc")
    for name in sorted(os.listdir(d)):
        with open(os.path.join(d, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


class Timer:
    """HIP events recorded on the given stream around every call of one kind."""

    def __init__(self, stream):
        self.stream = stream
        self.pairs = {}

    def run(self, name, fn):
        import torch
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(self.stream)
        fn()
        b.record(self.stream)
        self.pairs.setdefault(name, []).append((a, b))

    def mean_ms(self, name):
        p = self.pairs[name]
        return sum(a.elapsed_time(b) for a, b in p) / len(p)


def fwd_flops(B, H, N, d, causal):
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def make_step(fa, x, B, H, N, d, tau, timer=None):
    """Returns a closure running one step; tensors are preallocated (no allocation inside)."""
    import torch
    q, k, v, do = x["q"], x["k"], x["v"], x["do"]
    o_nc, lse_nc = torch.empty_like(q), torch.empty(B, H, N, device=q.device)
    o_c, lse_c = torch.empty_like(q), torch.empty(B, H, N, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.bwd_workspace_bytes(B, H, N) // 4, device=q.device)
    qd = q[:, :, -1:, :].contiguous()
    od, lsed = torch.empty_like(qd), torch.empty(B, H, device=q.device)
    seq = torch.full((B,), N, dtype=torch.int32, device=q.device)
    wsd = torch.empty(fa.decode_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=q.device)

    calls = [
        ("fwd_noncausal", lambda: fa.fwd(q, k, v, tau, False, o_nc, lse_nc)),
        ("fwd_causal", lambda: fa.fwd(q, k, v, tau, True, o_c, lse_c)),
        ("bwd_dq", lambda: fa.bwd(q, k, v, o_c, lse_c, do, tau, True, dq, dk, dv, ws, stage=0)),
        ("bwd_dkdv", lambda: fa.bwd(q, k, v, o_c, lse_c, do, tau, True, dq, dk, dv, ws, stage=1)),
        ("decode", lambda: fa.decode(qd, k, v, seq, tau, 0, od, lsed, wsd)),
    ]

    def step():
        for name, fn in calls:
            if timer is None:
                fn()
            else:
                timer.run(name, fn)
    return step


def window_pairs(N, window, sinks):
    """Visible (query, key) pairs of one head under the causal mask with a
    sliding window and sinks: sum_i min(i+1, window) + max(0, min(sinks, i-window+1))."""
    i = np.arange(N, dtype=np.int64)
    return float((np.minimum(i + 1, window) + np.maximum(0, np.minimum(sinks, i - window + 1))).sum())


def step_work(B, H, N, d):
    """Algorithmic FLOPs and HBM bytes per call of the step (bf16 = 2 bytes)."""
    e = 2
    t = B * H * N * d * e          # one [B,H,N,d] bf16 tensor
    lse = B * H * N * 4
    n2 = B * H * N * N * d
    return {
        "fwd_noncausal": (4.0 * n2, 3 * t + t + lse),
        "fwd_causal": (2.0 * n2, 3 * t + t + lse),
        # dQ kernel: D = rowsum(dO o O) for its rows, then the dQ product (1 of
        # the 5 backward GEMMs; its own S and dP recompute is not counted);
        # reads Q, K, V, dO, O, LSE, writes dQ and D
        "bwd_dq": (1.0 * n2 + 2.0 * B * H * N * d, 5 * t + 2 * lse + t),
        # dK/dV kernel: S, dP, dV, dK products (4 of the 5 backward GEMMs), causal half
        "bwd_dkdv": (4.0 * n2, 4 * t + 2 * lse + 2 * t),
        "decode": (4.0 * B * H * N * d, 2 * t + 2 * B * H * d * e + B * H * 4),
    }


def algorithmic_step_flops(B, H, N, d):
    """fwd nc 4BHN^2d + fwd causal 2BHN^2d + bwd causal 5BHN^2d + decode 4BHNd."""
    n2 = B * H * N * N * d
    return 4.0 * n2 + 2.0 * n2 + 5.0 * n2 + 4.0 * B * H * N * d


def load_traffic(kernel):
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get("kernels", {}).get(kernel)
    if not e or t.get("src_digest") != src_digest():
        return None
    return e.get("bytes_per_launch")


# The step's kernels as rocprofv3 names them (a decode with more than one
# split also launches the merge; the step's decode has one split).
STEP_KERNELS = {
    "fwd_noncausal": ["fwd_bf16_kernel<64, 0, 64, 4, false>"],
    "fwd_causal": ["fwd_bf16_kernel<64, 1, 64, 4, false>"],
    "bwd_dq": ["bwd_dq_kernel<64, 1, false>"],
    "bwd_dkdv": ["bwd_dkdv_kernel<64, 1, false>"],
    "decode": ["decode_split_kernel<unsigned short, 64>", "decode_merge_kernel<unsigned short, 64>"],
}


def _counter_means(run_dir, counter):
    """Mean value of `counter` per dispatch, by kernel name, over the
    *counter_collection.csv files rocprofv3 wrote under run_dir."""
    import csv
    import glob
    per = {}
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % run_dir)
    for fn in files:
        with open(fn) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                key = (fn, row["Dispatch_Id"])
                name = row["Kernel_Name"]
                per.setdefault(name, {}).setdefault(key, 0.0)
                per[name][key] += float(row["Counter_Value"])
    return {name: sum(d.values()) / len(d) for name, d in per.items()}


def summarize_counters(fetch_step, fetch_copy, write_step, write_copy, copy_mib, commands):
    """Writes profiles/traffic.json: HBM bytes per launch of the step's kernels
    from FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by what the
    same counter reads per byte of the plain device copy (--calibrate-copy)."""
    copy_bytes = float(copy_mib << 20)
    out = {"about": "HBM bytes per launch of the step's kernels (8x16x1024x64 bf16) from two "
                    "rocprofv3 counter runs, FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each "
                    "divided by what the same counter reads per byte of a plain %d MiB device "
                    "copy (bench.py --calibrate-copy %d) run the same way." % (copy_mib, copy_mib),
           "commands": commands, "copy_counter_per_byte": {}, "src_digest": src_digest(),
           "kernels": {}}
    vals = {}
    for counter, step_dir, copy_dir in (("FETCH_SIZE", fetch_step, fetch_copy),
                                        ("WRITE_SIZE", write_step, write_copy)):
        cm = _counter_means(copy_dir, counter)
        copy_kib = max(cm.values())   # the copy is the largest dispatch of that run
        out["copy_counter_per_byte"][counter] = copy_kib * 1024.0 / copy_bytes
        vals[counter] = _counter_means(step_dir, counter)
    for bench_name, names in STEP_KERNELS.items():
        e = {}
        for counter, key in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
            kib = 0.0
            for i, n in enumerate(names):
                hits = [v for k, v in vals[counter].items() if n in k]
                if not hits and i == 0:
                    raise SystemExit("kernel %s not in the %s run" % (n, counter))
                kib += hits[0] if hits else 0.0
            e[counter + "_KiB"] = round(kib, 1)
            e[key + "_bytes"] = round(kib * 1024.0 / out["copy_counter_per_byte"][counter], 1)
        e["bytes_per_launch"] = int(round(e["fetch_bytes"] + e["write_bytes"]))
        out["kernels"][bench_name] = e
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out["kernels"]))


def cpu_baseline(xh, B, H, N, d, tau, budget_s=10.0):
    """The float64 oracle over whole heads of the same step until ~budget_s seconds."""
    import numpy as np
    from oracle import attention as orc
    threads = None
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max((i.get("num_threads") or 0) for i in info) if info else None
    except Exception:
        pass
    qf, kf, vf, dof = (xh[n].f64() for n in ("q", "k", "v", "do"))
    heads, flops = 0, 0.0
    t0 = time.perf_counter()
    per_head = algorithmic_step_flops(1, 1, N, d)
    for it in range(1 << 30):
        b, h = divmod(it % (B * H), H)
        orc.attention_fwd_head(qf[b, h], kf[b, h], vf[b, h], tau, False)
        orc.attention_fwd_head(qf[b, h], kf[b, h], vf[b, h], tau, True)
        orc.attention_bwd_head(qf[b, h], kf[b, h], vf[b, h], dof[b, h], tau, True)
        orc.decode_fwd(qf[b:b + 1, h:h + 1, -1:], kf[b:b + 1, h:h + 1], vf[b:b + 1, h:h + 1],
                       np.array([N]), tau)
        heads += 1
        flops += per_head
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": threads or os.cpu_count(), "kind": "oracle",
            "sample": "%d (b,h) heads (cycling over the %d of the batch) of the step: fwd "
                      "non-causal, fwd causal, bwd causal, decode; float64 NumPy, %.1f s"
                      % (heads, B * H, dt)}


def bench_extra(fa, reps=50):
    """Full-size long-prefill, decode and backward workloads, each vs its roofline."""
    import torch
    out = {}
    dev = "cuda"
    g = torch.Generator(device=dev)
    stream = torch.cuda.current_stream()

    def time_it(fn, reps):
        """Median of reps HIP-event pairs on the stream, after 10 warm-up calls."""
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) for a, b in ev)
        return ts[len(ts) // 2]

    # long causal prefill: 1 x 32 x 16384 x 128, bf16
    B, H, N, d = 1, 32, 16384, 128
    g.manual_seed(1003)
    q, k, v = (torch.randn(B, H, N, d, device=dev, generator=g).to(torch.bfloat16) for _ in range(3))
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, device=dev)
    tau = 1 / math.sqrt(d)
    ms = time_it(lambda: fa.fwd(q, k, v, tau, True, o, lse), reps)
    fl = fwd_flops(B, H, N, d, True)
    out["long_causal_prefill"] = {"shape": [B, H, N, d], "causal": True, "ms": round(ms, 4),
                                  "TFLOP/s": round(fl / ms / 1e9, 2),
                                  "frac_mfma_bf16": round(fl / ms / 1e-3 / PEAK_MFMA_BF16, 4)}
    del q, k, v, o, lse

    # the same prefill as a local (sliding-window) layer: window 4096, no sinks
    B, H, N, d, wnd = 1, 32, 16384, 128, 4096
    g.manual_seed(1003)
    q, k, v = (torch.randn(B, H, N, d, device=dev, generator=g).to(torch.bfloat16) for _ in range(3))
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, device=dev)
    ms = time_it(lambda: fa.fwd(q, k, v, 1 / math.sqrt(d), True, o, lse, window=wnd), reps)
    fl = 4.0 * B * H * d * window_pairs(N, wnd, 0)
    out["window_prefill"] = {"shape": [B, H, N, d], "window": wnd, "sinks": 0, "ms": round(ms, 4),
                             "TFLOP/s": round(fl / ms / 1e9, 2),
                             "frac_mfma_bf16": round(fl / ms / 1e-3 / PEAK_MFMA_BF16, 4)}
    del q, k, v, o, lse

    # the same prefill block-sparse: 128 x 128 blocks, a band of 3 blocks
    # around the diagonal plus the first key block (global tokens), causal
    B, H, N, d, bs = 1, 32, 16384, 128, 128
    nb = N // bs
    bi, bj = np.meshgrid(np.arange(nb), np.arange(nb), indexing="ij")
    mask_np = ((np.abs(bi - bj) <= 1) | (bj == 0)).astype(np.uint8)
    # visible pairs: whole blocks below the diagonal, half (with it) on it
    pairs = float(((mask_np == 1) & (bi > bj)).sum()) * bs * bs + nb * bs * (bs + 1) / 2
    g.manual_seed(1003)
    q, k, v = (torch.randn(B, H, N, d, device=dev, generator=g).to(torch.bfloat16) for _ in range(3))
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, device=dev)
    bm = torch.from_numpy(mask_np[None]).to(dev)
    ms = time_it(lambda: fa.fwd(q, k, v, 1 / math.sqrt(d), True, o, lse, block_mask=bm,
                                block_size=(bs, bs)), reps)
    fl = 4.0 * B * H * d * pairs
    out["block_sparse_prefill"] = {"shape": [B, H, N, d], "block": [bs, bs],
                                   "pattern": "band +-1 block and global first key block, causal",
                                   "density": round(pairs / (N * (N + 1) / 2), 4),
                                   "ms": round(ms, 4), "TFLOP/s": round(fl / ms / 1e9, 2),
                                   "frac_mfma_bf16": round(fl / ms / 1e-3 / PEAK_MFMA_BF16, 4)}
    del q, k, v, o, lse

    # decode: 64 x 32 x 8192 x 128, L_b ~ U[1024, 8192]
    B, H, N, d = 64, 32, 8192, 128
    import fa_inputs
    seqlens = fa_inputs.decode_seqlens(B, 1024, 8192, 1004 + 400)
    g.manual_seed(1004)
    q = torch.randn(B, H, 1, d, device=dev, generator=g).to(torch.bfloat16)
    k = torch.empty(B, H, N, d, device=dev, dtype=torch.bfloat16)
    v = torch.empty_like(k)
    for b in range(B):   # one sequence at a time keeps each draw far below 2^31 elements
        k[b] = torch.randn(H, N, d, device=dev, generator=g).to(torch.bfloat16)
        v[b] = torch.randn(H, N, d, device=dev, generator=g).to(torch.bfloat16)
    sl = torch.from_numpy(seqlens).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(B, H, device=dev)
    ws = torch.empty(fa.decode_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
    ms = time_it(lambda: fa.decode(q, k, v, sl, 1 / math.sqrt(d), 0, o, lse, ws), reps * 2)
    if not bool(torch.isfinite(o.float()).all()):
        raise RuntimeError("decode produced non-finite output")
    nbytes = float(seqlens.astype("int64").sum()) * H * d * 2 * 2 + 2 * B * H * d * 2 + B * H * 4
    out["decode_splitkv"] = {"shape": [B, H, N, d], "seqlens_sum": int(seqlens.sum()),
                             "num_splits": fa.decode_num_splits(B, H, N, d),
                             "ms": round(ms, 4), "GB/s": round(nbytes / ms / 1e6, 1),
                             "frac_hbm": round(nbytes / ms / 1e-3 / PEAK_HBM, 4)}
    del q, k, v, o, lse, ws

    # paged decode with grouped KV heads: B=64, Hq=32, Hkv=8, 16-token pages,
    # d=128, the dense decode's key lengths; pages assigned in a seeded random order
    import fa_inputs
    w = fa_inputs.PAGED_WORKLOAD
    B, Hq, Hkv, P, d = w.B, w.Hq, w.Hkv, w.page_size, w.d
    seqlens = fa_inputs.decode_seqlens(B, w.lmin, w.lmax, w.seqlens_seed)
    npb = (seqlens.astype("int64") + P - 1) // P
    npages, maxp = int(npb.sum()), w.max_pages
    perm = torch.randperm(npages, generator=torch.Generator().manual_seed(w.seed)).to(torch.int32)
    table = torch.zeros(B, maxp, dtype=torch.int32)
    nxt = 0
    for b in range(B):
        table[b, :npb[b]] = perm[nxt:nxt + npb[b]]
        nxt += int(npb[b])
    table = table.to(dev)
    g.manual_seed(w.seed)
    q = torch.randn(B, Hq, 1, d, device=dev, generator=g).to(torch.bfloat16)
    kp = torch.empty(npages, Hkv, P, d, device=dev, dtype=torch.bfloat16)
    vp = torch.empty_like(kp)
    for i in range(0, npages, 4096):
        n = min(4096, npages - i)
        kp[i:i + n] = torch.randn(n, Hkv, P, d, device=dev, generator=g).to(torch.bfloat16)
        vp[i:i + n] = torch.randn(n, Hkv, P, d, device=dev, generator=g).to(torch.bfloat16)
    sl = torch.from_numpy(seqlens).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, device=dev)
    ws = torch.empty(fa.decode_paged_workspace_bytes(B, Hq, Hkv, P, maxp, d), dtype=torch.uint8,
                     device=dev)
    ms = time_it(lambda: fa.decode_paged(q, kp, vp, table, sl, 1 / math.sqrt(d), 0, o, lse, ws),
                 reps * 2)
    if not bool(torch.isfinite(o.float()).all()):
        raise RuntimeError("paged decode produced non-finite output")
    nbytes = (float(seqlens.astype("int64").sum()) * Hkv * d * 2 * 2 + 2 * B * Hq * d * 2
              + B * Hq * 4 + int(npb.sum()) * 4)
    out["decode_paged_gqa"] = {"shape": {"B": B, "Hq": Hq, "Hkv": Hkv, "page_size": P, "d": d},
                               "seqlens_sum": int(seqlens.sum()),
                               "num_splits": fa.decode_paged_num_splits(B, Hq, Hkv, P, maxp, d),
                               "ms": round(ms, 4), "GB/s": round(nbytes / ms / 1e6, 1),
                               "frac_hbm": round(nbytes / ms / 1e-3 / PEAK_HBM, 4)}
    del q, kp, vp, o, lse, ws, table

    # backward: 4 x 16 x 4096 x 64, causal
    B, H, N, d = 4, 16, 4096, 64
    g.manual_seed(1005)
    q, k, v, do = (torch.randn(B, H, N, d, device=dev, generator=g).to(torch.bfloat16)
                   for _ in range(4))
    tau = 1 / math.sqrt(d)
    o, lse = fa.fwd(q, k, v, tau, True)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(B * H * N, device=dev)
    ms = time_it(lambda: fa.bwd(q, k, v, o, lse, do, tau, True, dq, dk, dv, ws), reps)
    fl = 10.0 * B * H * N * N * d / 2
    out["bwd_recompute"] = {"shape": [B, H, N, d], "causal": True, "ms": round(ms, 4),
                            "TFLOP/s": round(fl / ms / 1e9, 2),
                            "frac_mfma_bf16": round(fl / ms / 1e-3 / PEAK_MFMA_BF16, 4)}

    # the same shape with dropout p = 0.1 (Philox mask regenerated in the backward)
    drop = (0.1, 1005, 0)
    ms_f = time_it(lambda: fa.fwd(q, k, v, tau, True, o, lse, dropout=drop), reps)
    ms_b = time_it(lambda: fa.bwd(q, k, v, o, lse, do, tau, True, dq, dk, dv, ws, dropout=drop),
                   reps)
    ffl = 4.0 * B * H * N * N * d / 2
    out["dropout"] = {"shape": [B, H, N, d], "causal": True, "p": 0.1,
                      "fwd_ms": round(ms_f, 4), "fwd_TFLOP/s": round(ffl / ms_f / 1e9, 2),
                      "bwd_ms": round(ms_b, 4), "bwd_TFLOP/s": round(fl / ms_b / 1e9, 2)}
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB five times "
                         "(scales the HBM byte counters of a profiler run) and exit")
    ap.add_argument("--summarize-counters", nargs=4, default=None,
                    metavar=("FETCH_STEP", "FETCH_COPY", "WRITE_STEP", "WRITE_COPY"),
                    help="write profiles/traffic.json from four rocprofv3 --pmc output "
                         "directories (FETCH_SIZE and WRITE_SIZE, each over a step run and a "
                         "--calibrate-copy 1024 run) and exit; runs on the host, no GPU")
    args = ap.parse_args(argv)
    if args.summarize_counters:
        d = args.summarize_counters
        cmds = ["rocprofv3 --pmc %s --output-format csv -d %s -o %s -- python -u bench.py %s"
                % (c, r, o, a) for c, r, o, a in (
                    ("FETCH_SIZE", d[0], "step", "--steps 3 --warmup 1 --no-extra --no-cpu"),
                    ("FETCH_SIZE", d[1], "copy", "--calibrate-copy 1024"),
                    ("WRITE_SIZE", d[2], "step", "--steps 3 --warmup 1 --no-extra --no-cpu"),
                    ("WRITE_SIZE", d[3], "copy", "--calibrate-copy 1024"))]
        summarize_counters(d[0], d[1], d[2], d[3], 1024, cmds)
        return 0
    if args.gpus != 1:
        print("bench.py: this attention path runs on one GPU; --gpus %d is not supported "
              "(sharding over (batch, head) is described in the design notes, not built)"
              % args.gpus, file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import fa_inputs
    import io_aware_tiled_03_amd as fa
    fa.lib()   # fails loudly if the library is not built
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 5}))
        return 0

    w = fa_inputs.WORKLOADS[2]
    B, H, N, d, tau = w.B, w.H, w.N, w.d, w.tau
    xh = fa_inputs.dense_inputs(B, H, N, d, "bf16", w.seed, with_do=True)
    x = {n: torch.from_numpy(np.ascontiguousarray(xh[n].raw).view(np.int16)).view(
        torch.bfloat16).cuda() for n in ("q", "k", "v", "do")}

    plain = make_step(fa, x, B, H, N, d, tau)
    for _ in range(args.warmup):
        plain()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        plain()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / args.steps * 1e3
    step_flops = algorithmic_step_flops(B, H, N, d)
    value = step_flops / (wall / args.steps) / 1e12

    # per-call HIP events over a second timed pass of the same steps
    stream = torch.cuda.current_stream()
    timer = Timer(stream)
    timed = make_step(fa, x, B, H, N, d, tau, timer)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        timed()
    torch.cuda.synchronize()
    work = step_work(B, H, N, d)
    kernels = {}
    for name in work:
        ms = timer.mean_ms(name)
        fl, by = work[name]
        kernels[name] = {"ms": round(ms, 5), "TFLOP/s": round(fl / ms / 1e9, 2),
                         "GB/s": round(by / ms / 1e6, 1)}
    dom = max(kernels, key=lambda n: kernels[n]["ms"])
    fl, by = work[dom]
    dms = timer.mean_ms(dom)
    if fl / by > 300:
        roof = {"bound": "mfma", "achieved": round(fl / dms / 1e9, 2), "peak": PEAK_MFMA_BF16 / 1e12,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(by / dms / 1e6, 1), "peak": PEAK_HBM / 1e9,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["kernel"] = dom
    roof["traffic"] = load_traffic(dom)

    line = {
        "metric": "attention fwd/bwd TFLOP/s and % MFMA peak (bf16, d=64/128); decode HBM GB/s",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "gpt2-medium-shaped attention step: fwd non-causal + fwd causal "
                               "+ bwd causal + decode (L_b=N)", "B": B, "H": H, "N": N, "d": d,
                   "tau": tau, "parallelism": "single GPU"},
        "frac_of_mfma_peak": round(value * 1e12 / PEAK_MFMA_BF16, 4),
        "kernels": kernels,
        "roofline": roof,
    }
    if not args.no_extra:
        line["also_measured"] = bench_extra(fa)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(xh, B, H, N, d, tau)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
