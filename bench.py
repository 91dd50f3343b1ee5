"""Throughput of the exact-attention path on one MI355X.

Headline step: the long-context causal prefill forward, fa_fwd on
B=1, H=32, N=16384, d=128, bf16 Q/K/V drawn N(0,1) from the seeded recipe of
fa_inputs (seeds 1003/1103/1203), causal, tau = 1/sqrt(128).  A materialised
N x N score matrix of this shape would hold 512 MiB per head in fp16 ("Atenção
eficiente — FlashAttention, sparse e híbrida", table of section "Por que isso
importa"); the kernel never writes it.
value = algorithmic TFLOP/s (4*B*H*N^2*d, halved for the causal mask) from the
wall clock around exactly --steps calls bracketed by device synchronisation,
inputs resident in HBM.

The JSON line also carries, from the same run:
  * "timing": every timed call bracketed by HIP events on the stream the
    library launches on (median, p10, p90, mean);
  * "roofline": the forward kernel against the dense bf16 MFMA peak
    (algorithmic flops / mean event time) and its HBM traffic per launch from
    the committed rocprofv3 counter summary when it matches the sources;
  * "sclk_mhz": the shader clock level read from sysfs while the kernel runs
    back to back (null where the file is not readable);
  * "bytes_avoided": the HBM traffic standard attention would spend on S and
    P at this shape;
  * "pages_context": the pages' own figures, quoted with their hardware;
  * "also_measured" (skip: --no-extra): the GPT-2-medium-shaped step (fwd
    non-causal, fwd causal, bwd causal, decode), the tiny fp32 forward, the
    split-KV decode, the paged grouped-head decode, the 4k causal backward,
    the prefill as a sliding-window and as a block-sparse layer (forward and
    backward), and dropout,
    each against its roofline (the decodes alternate between two copies of
    their caches, so that no call is served from the caches by the previous);
  * "cpu_baseline" (skip: --no-cpu): the float64 oracle on the host over two
    whole heads of the headline workload, with the GPU output of those heads
    compared against it, plus the oracle's wall time on the other workloads.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import itertools
import json
import math
import os
import subprocess
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_BF16 = 2.5e15     # dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12           # HBM3E, B/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
METRIC = "attention fwd/bwd TFLOP/s and % MFMA peak (bf16, d=64/128); decode HBM GB/s"

# The headline kernel as rocprofv3 names it.
HEADLINE_KERNELS = {"long_causal_prefill": ["fwd_bf16_kernel<128, 1, 128, 8, false>"]}

# The pages' own figures that touch this path, quoted with their hardware.
PAGES_CONTEXT = [
    {"figure": "2-4x faster than standard attention (inference and training)",
     "hardware": "not stated", "source": "FlashAttention: O Que É e Como Acelera LLMs na "
                                         "Prática, section 'O Que É e Por Que Ela Muda o Jogo'"},
    {"figure": "up to 10x less memory and about 3x faster at a 32k-token context, where "
               "standard attention runs out of memory",
     "hardware": "A100", "source": "FlashAttention: O Que É e Como Acelera LLMs na Prática, "
                                   "section 'Exemplo Prático'"},
    {"figure": "standard attention at GPT-2 medium, sequence 1024: 40.3 GB of HBM traffic "
               "against 66.6 GFLOPs (memory-bound)",
     "hardware": "A100 (HBM 1.5-2.0 TB/s)", "source": "flash-attention encyclopedia page, "
                                                      "section 'o problema'"},
]


# The sources the headline kernel is built from: its HBM traffic record stays
# valid while these are unchanged.
HEADLINE_SOURCES = ("fa_fwd.hip", "fa_device.hpp", "fa_internal.h")


def src_digest(names=None):
    """Digest of the named sources under csrc/ (default: all of them)."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "io_aware_tiled_03_amd", "csrc")
    for name in sorted(os.listdir(d) if names is None else names):
        with open(os.path.join(d, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def git_head():
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "--short=12", "HEAD"],
                           stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True, timeout=10)
        return r.stdout.strip() or None
    except (OSError, subprocess.SubprocessError):
        return None


def fwd_flops(B, H, N, d, causal):
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def window_pairs(N, window, sinks):
    """Visible (query, key) pairs of one head under the causal mask with a
    sliding window and sinks: sum_i min(i+1, window) + max(0, min(sinks, i-window+1))."""
    i = np.arange(N, dtype=np.int64)
    return float((np.minimum(i + 1, window) + np.maximum(0, np.minimum(sinks, i - window + 1))).sum())


def bytes_avoided(B, H, N):
    """HBM bytes standard attention moves for S and P at this shape: the N x N
    fp16 score matrix per head ("Por que isso importa" table: 512 MiB per head
    at N = 16384) written as S, read back, written as P and read by P V
    ("flash-attention" page, "o problema")."""
    per_head = N * N * 2
    return {"per_head_MiB": per_head / 2 ** 20, "passes": 4,
            "total_GiB": B * H * per_head * 4 / 2 ** 30,
            "note": "S = Q K^T written, read for the softmax, P written, read for P V; fp16"}


def stats_ms(ts):
    ts = sorted(ts)
    q = lambda f: ts[min(len(ts) - 1, int(round(f * (len(ts) - 1))))]
    return {"median": round(q(0.5), 5), "p10": round(q(0.1), 5), "p90": round(q(0.9), 5),
            "mean": round(sum(ts) / len(ts), 5), "n": len(ts)}


def load_traffic(kernel):
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get("kernels", {}).get(kernel)
    if not e or t.get("src_digest") != src_digest(HEADLINE_SOURCES):
        return None
    return e.get("bytes_per_launch")


def _counter_means(run_dir, counter):
    """Mean value of `counter` per dispatch, by kernel name, over the
    *counter_collection.csv files rocprofv3 wrote under run_dir."""
    import csv
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


def summarize_counters(fetch_run, fetch_copy, write_run, write_copy, copy_mib, commands,
                       kernels=None):
    """Writes profiles/traffic.json: HBM bytes per launch of the given kernels
    from FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by what the
    same counter reads per byte of the plain device copy (--calibrate-copy)."""
    kernels = HEADLINE_KERNELS if kernels is None else kernels
    copy_bytes = float(copy_mib << 20)
    out = {"about": "HBM bytes per launch of the headline kernel (long causal prefill, "
                    "1x32x16384x128 bf16) from two rocprofv3 counter runs, FETCH_SIZE and "
                    "WRITE_SIZE (KiB per dispatch), each divided by what the same counter reads "
                    "per byte of a plain %d MiB device copy (bench.py --calibrate-copy %d) run "
                    "the same way." % (copy_mib, copy_mib),
           "commands": commands, "copy_counter_per_byte": {},
           "src_digest": src_digest(HEADLINE_SOURCES), "sources": list(HEADLINE_SOURCES),
           "kernels": {}}
    vals = {}
    for counter, run_dir, copy_dir in (("FETCH_SIZE", fetch_run, fetch_copy),
                                       ("WRITE_SIZE", write_run, write_copy)):
        cm = _counter_means(copy_dir, counter)
        copy_kib = max(cm.values())   # the copy is the largest dispatch of that run
        out["copy_counter_per_byte"][counter] = copy_kib * 1024.0 / copy_bytes
        vals[counter] = _counter_means(run_dir, counter)
    for bench_name, names in kernels.items():
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


def read_sclk_mhz():
    """The active shader clock level of the first GPU from sysfs, or None."""
    for fn in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(fn) as f:
                for line in f:
                    if "*" in line:
                        tok = line.split(":")[-1].replace("*", "").strip().lower()
                        return float(tok.replace("mhz", "").strip())
        except (OSError, ValueError):
            continue
    return None


def sample_clock(run, seconds=0.5):
    """Runs `run` back to back for about `seconds` while sampling the sclk level."""
    import torch
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            v = read_sclk_mhz()
            if v is not None:
                samples.append(v)
            time.sleep(0.01)
    t = threading.Thread(target=sampler, daemon=True)
    t.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            run()
        torch.cuda.synchronize()
    stop.set()
    t.join()
    if not samples:
        return None
    s = sorted(samples)
    return {"median": s[len(s) // 2], "min": s[0], "max": s[-1], "samples": len(s),
            "source": "pp_dpm_sclk active level while the headline kernel runs back to back"}


def alternating(items):
    """An endless iterator over items in turn."""
    return itertools.cycle(items)


def time_events(fn, reps, warmup=10):
    """Per-call HIP event times (ms) on the current stream, after warm-up calls."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def rate_under_load(run, flops, seconds=1.2):
    """TFLOP/s of `run` called back to back for about `seconds` (the second half timed with
    HIP events, after the first half brought the clock to its level under this load), with
    the sclk level sampled throughout."""
    import torch
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            v = read_sclk_mhz()
            if v is not None:
                samples.append(v)
            time.sleep(0.01)
    t = threading.Thread(target=sampler, daemon=True)
    t.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds / 2:
        run()
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 0
    e0.record(stream)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds / 2:
        run()
        n += 1
        torch.cuda.synchronize()
    e1.record(stream)
    torch.cuda.synchronize()
    stop.set()
    t.join()
    ms = e0.elapsed_time(e1) / n
    s = sorted(samples)
    return {"TFLOP/s": round(flops / ms / 1e9, 1), "frac_of_nominal": round(flops / ms / 1e-3 / PEAK_MFMA_BF16, 4),
            "ms_per_call": round(ms, 4), "sclk_mhz_median": s[len(s) // 2] if s else None}


def ceilings(fa, headline_tflops, seconds=1.2):
    """Rates this part reaches on synthetic matrix-core loops with a given mix of work per
    bf16 product (fa_calib.h), and on the vendor library's bf16 GEMM, each timed under its
    own load; the headline kernel's rate as a fraction of each."""
    import torch
    g = torch.Generator().manual_seed(7)
    seed = (torch.randn(fa.CALIB_SEED_BYTES // 2, generator=g) * 0.5).to(torch.bfloat16).cuda()
    grid, iters = 2048, 2000
    out = torch.empty(grid * 256, device="cuda")
    res = {"note": "synthetic loops (no HBM traffic, barriers or masking): what the part reaches "
                   "for each mix of work per 32x32x16 bf16 product; the headline's kernel issues "
                   "one 1 KB LDS operand read, one exp2 and about four other vector "
                   "instructions per product",
           "mixes": []}
    for mix, name in enumerate(fa.calib_mixes()):
        r = rate_under_load(lambda: fa.calib_mfma(mix, grid, iters, seed, out),
                            fa.calib_flops(mix, grid, iters), seconds)
        r = {"mix": name, **r, "headline_fraction_of_this": round(headline_tflops / r["TFLOP/s"], 4)}
        res["mixes"].append(r)
    del seed, out
    n = 8192
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    r = rate_under_load(lambda: torch.matmul(a, b, out=c), 2.0 * n ** 3, seconds)
    res["library_gemm"] = {"op": "torch.matmul bf16 8192 x 8192 x 8192 (vendor BLAS)", **r,
                           "headline_fraction_of_this": round(headline_tflops / r["TFLOP/s"], 4)}
    del a, b, c
    # HBM: a streaming read of 4 GiB (non-temporal 16-byte loads, as the decode kernels issue),
    # at a few grid sizes; the best rate is the ceiling the decode kernels are read against
    buf = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    best = None
    for grid in (256, 512, 1024, 2048, 4096, 8192):
        chk = torch.empty(grid * 256, dtype=torch.int32, device="cuda")
        r = rate_under_load(lambda: fa.calib_hbm_read(buf, grid, chk), float(buf.numel()), seconds)
        gbs = round(buf.numel() / (r["ms_per_call"] * 1e-3) / 1e9, 1)
        if best is None or gbs > best["GB/s"]:
            best = {"op": "streaming read of 4 GiB, non-temporal 16-byte loads (fa_calib_hbm_read)",
                    "grid": grid, "GB/s": gbs, "frac_of_8TB/s": round(gbs / (PEAK_HBM / 1e9), 4),
                    "ms_per_call": r["ms_per_call"], "sclk_mhz_median": r["sclk_mhz_median"]}
    res["hbm_stream_read"] = best
    del buf
    torch.cuda.empty_cache()
    return res


def lds_patterns(fa, seconds=0.6):
    """LDS read patterns of the kernels' operand reads, each alone (fa_calib.h): bytes per clock
    per CU at the sampled sclk."""
    import torch
    grid, iters = 1024, 4000
    out = torch.empty(grid * 512, dtype=torch.int32, device="cuda")
    res = []
    for pat, name in enumerate(fa.calib_lds_patterns()):
        nbytes = fa.calib_lds_bytes(pat, grid, iters)
        r = rate_under_load(lambda: fa.calib_lds(pat, grid, iters, out), nbytes, seconds)
        ms, mhz = r["ms_per_call"], r["sclk_mhz_median"] or 2400.0
        res.append({"pattern": name, "ms_per_call": ms, "sclk_mhz_median": mhz,
                    "B_per_clk_per_CU": round(nbytes / (ms * 1e-3) / (mhz * 1e6) / 256, 1)})
    return res


def upload(ht, dev="cuda"):
    """HostTensor -> GPU tensor with exactly the same bits."""
    import torch
    if ht.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(ht.raw).view(np.int16)).view(
            torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(ht.raw)).to(dev)


# --- the GPT-2-medium-shaped step (also measured) ---------------------------

def gpt2m_step_work(B, H, N, d):
    """Algorithmic FLOPs and HBM bytes per call of the step (bf16 = 2 bytes)."""
    e = 2
    t = B * H * N * d * e          # one [B,H,N,d] bf16 tensor
    lse = B * H * N * 4
    n2 = B * H * N * N * d
    return {
        "fwd_noncausal": (4.0 * n2, 3 * t + t + lse),
        "fwd_causal": (2.0 * n2, 3 * t + t + lse),
        # dQ kernel: D = rowsum(dO o O) for its rows, then the dQ product (1 of
        # the 5 backward products; its own S and dP recompute is not counted)
        "bwd_dq": (1.0 * n2 + 2.0 * B * H * N * d, 5 * t + 2 * lse + t),
        # dK/dV kernel: S, dP, dV, dK products (4 of the 5 backward products), causal half
        "bwd_dkdv": (4.0 * n2, 4 * t + 2 * lse + 2 * t),
        "decode": (4.0 * B * H * N * d, 2 * t + 2 * B * H * d * e + B * H * 4),
    }


def gpt2m_step(fa, x, B, H, N, d, tau, reps):
    """One step = fwd non-causal + fwd causal + bwd causal (its two kernels
    enqueued one by one) + decode with one query per sequence against the same
    K/V (L_b = N); each call timed with HIP events, and the step as a whole."""
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
        for _, fn in calls:
            fn()
    step_ms = stats_ms(time_events(step, reps))
    work = gpt2m_step_work(B, H, N, d)
    kernels = {}
    for name, fn in calls:
        ms = stats_ms(time_events(fn, reps))["median"]
        fl, by = work[name]
        kernels[name] = {"ms": ms, "TFLOP/s": round(fl / ms / 1e9, 2),
                         "GB/s": round(by / ms / 1e6, 1),
                         "frac_mfma_bf16": round(fl / ms / 1e-3 / PEAK_MFMA_BF16, 4)}
    n2 = B * H * N * N * d
    flops = 4.0 * n2 + 2.0 * n2 + 5.0 * n2 + 4.0 * B * H * N * d
    out = {"shape": [B, H, N, d], "tau": tau, "step_ms": step_ms,
           "TFLOP/s": round(flops / step_ms["median"] / 1e9, 2),
           "frac_mfma_bf16": round(flops / step_ms["median"] / 1e-3 / PEAK_MFMA_BF16, 4),
           "kernels": kernels}
    return out, {"o_nc": o_nc, "lse_nc": lse_nc, "o_c": o_c, "lse_c": lse_c}


def bench_extra(fa, reps=50):
    """The other workloads at full size, each against its roofline."""
    import torch

    import fa_inputs
    out, gpu_out = {}, {}
    dev = "cuda"
    g = torch.Generator(device=dev)

    def med(fn, n=reps):
        return stats_ms(time_events(fn, n))["median"]

    # GPT-2-medium-shaped step on the host recipe's inputs (8x16x1024x64 bf16)
    w = fa_inputs.WORKLOADS[2]
    xh = fa_inputs.dense_inputs(w.B, w.H, w.N, w.d, "bf16", w.seed, with_do=True)
    x = {n: upload(xh[n]) for n in ("q", "k", "v", "do")}
    out["gpt2m_step"], gpu_out["gpt2m"] = gpt2m_step(fa, x, w.B, w.H, w.N, w.d, w.tau, reps)
    del x

    # tiny fp32 forward (1x1x256x64, non-causal)
    w = fa_inputs.WORKLOADS[1]
    xh = fa_inputs.workload_inputs(w)
    q, k, v = (upload(xh[n]) for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty(1, 1, w.N, device=dev)
    ms = med(lambda: fa.fwd(q, k, v, w.tau, False, o, lse))
    out["tiny_fp32_fwd"] = {"shape": [w.B, w.H, w.N, w.d], "dtype": "f32", "ms": ms,
                            "note": "latency-bound (32 workgroups of 8 waves, each wave reading "
                                    "its 32 key rows one after another); checked for parity, "
                                    "no roofline"}
    del q, k, v, o, lse

    # the prefill as a local (sliding-window) layer: window 4096, no sinks
    B, H, N, d, wnd = 1, 32, 16384, 128, 4096
    g.manual_seed(1003)
    q, k, v = (torch.randn(B, H, N, d, device=dev, generator=g).to(torch.bfloat16) for _ in range(3))
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, device=dev)
    ms = med(lambda: fa.fwd(q, k, v, 1 / math.sqrt(d), True, o, lse, window=wnd))
    fl = 4.0 * B * H * d * window_pairs(N, wnd, 0)
    out["window_prefill"] = {"shape": [B, H, N, d], "window": wnd, "sinks": 0, "ms": ms,
                             "TFLOP/s": round(fl / ms / 1e9, 2),
                             "frac_mfma_bf16": round(fl / ms / 1e-3 / PEAK_MFMA_BF16, 4)}
    # its backward (dQ, then dK and dV), 5 products over the visible pairs
    do = torch.randn(B, H, N, d, device=dev, generator=g).to(torch.bfloat16)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    bws = torch.empty(fa.bwd_workspace_bytes(B, H, N), dtype=torch.uint8, device=dev)
    ms = med(lambda: fa.bwd(q, k, v, o, lse, do, 1 / math.sqrt(d), True, dq, dk, dv, bws,
                            window=wnd), reps // 2)
    out["window_prefill"].update({"bwd_ms": ms, "bwd_TFLOP/s": round(2.5 * fl / ms / 1e9, 2),
                                  "bwd_frac_mfma_bf16": round(2.5 * fl / ms / 1e-3 / PEAK_MFMA_BF16, 4)})

    # the same prefill block-sparse: 128 x 128 blocks, a band of 3 blocks
    # around the diagonal plus the first key block (global tokens), causal
    bs = 128
    nb = N // bs
    bi, bj = np.meshgrid(np.arange(nb), np.arange(nb), indexing="ij")
    mask_np = ((np.abs(bi - bj) <= 1) | (bj == 0)).astype(np.uint8)
    pairs = float(((mask_np == 1) & (bi > bj)).sum()) * bs * bs + nb * bs * (bs + 1) / 2
    bm = torch.from_numpy(mask_np[None]).to(dev)
    ms = med(lambda: fa.fwd(q, k, v, 1 / math.sqrt(d), True, o, lse, block_mask=bm,
                            block_size=(bs, bs)))
    fl = 4.0 * B * H * d * pairs
    # at this density the binding roofline is HBM: Q, K, V read and O, LSE written once
    # (538 MB, 67 us at 8 TB/s) outweigh the products (86 GFLOP, 34 us at 2.5 PFLOP/s)
    nbytes = 4.0 * B * H * N * d * 2 + B * H * N * 4
    out["block_sparse_prefill"] = {"shape": [B, H, N, d], "block": [bs, bs],
                                   "pattern": "band +-1 block and global first key block, causal",
                                   "density": round(pairs / (N * (N + 1) / 2), 4), "ms": ms,
                                   "TFLOP/s": round(fl / ms / 1e9, 2),
                                   "frac_mfma_bf16": round(fl / ms / 1e-3 / PEAK_MFMA_BF16, 4),
                                   "GB/s": round(nbytes / ms / 1e6, 1),
                                   "frac_hbm": round(nbytes / ms / 1e-3 / PEAK_HBM, 4)}
    # its backward, with the workspace that lets the global key block's long
    # list of query tiles be split over several workgroups
    sws = torch.empty(fa.bwd_block_sparse_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
    ms = med(lambda: fa.bwd(q, k, v, o, lse, do, 1 / math.sqrt(d), True, dq, dk, dv, sws,
                            block_mask=bm, block_size=(bs, bs)), reps // 2)
    out["block_sparse_prefill"].update({
        "bwd_ms": ms, "bwd_TFLOP/s": round(2.5 * fl / ms / 1e9, 2),
        "bwd_frac_mfma_bf16": round(2.5 * fl / ms / 1e-3 / PEAK_MFMA_BF16, 4),
        "bwd_workspace_MiB": round(sws.numel() / 2 ** 20, 1)})
    del q, k, v, o, lse, bm, do, dq, dk, dv, bws, sws

    # split-KV decode: 64 x 32 x 8192 x 128, L_b ~ U[1024, 8192]
    w = fa_inputs.WORKLOADS[4]
    B, H, N, d = w.B, w.H, w.N, w.d
    seqlens = fa_inputs.decode_seqlens(B, w.lmin, w.lmax, w.seed + fa_inputs.SEED_OFFSET["seqlens"])
    g.manual_seed(w.seed)
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
    # successive calls alternate between the cache and a copy of it at other
    # addresses, so no call finds the previous call's rows in the caches
    kv = alternating([(k, v), (k.clone(), v.clone())])
    ms = med(lambda: fa.decode(q, *next(kv), sl, w.tau, 0, o, lse, ws), 2 * reps)
    if not bool(torch.isfinite(o.float()).all()):
        raise RuntimeError("decode produced non-finite output")
    nbytes = float(seqlens.astype("int64").sum()) * H * d * 2 * 2 + 2 * B * H * d * 2 + B * H * 4
    out["decode_splitkv"] = {"shape": [B, H, N, d], "seqlens_sum": int(seqlens.sum()),
                             "num_splits": fa.decode_num_splits(B, H, N, d),
                             "input_copies": 2, "ms": ms, "GB/s": round(nbytes / ms / 1e6, 1),
                             "frac_hbm": round(nbytes / ms / 1e-3 / PEAK_HBM, 4)}
    del q, k, v, o, lse, ws, kv

    # paged decode with grouped KV heads: B=64, Hq=32, Hkv=8, 16-token pages,
    # d=128, the dense decode's key lengths; pages assigned in a seeded random order
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
    kv = alternating([(kp, vp), (kp.clone(), vp.clone())])   # as for the dense decode
    ms = med(lambda: fa.decode_paged(q, *next(kv), table, sl, w.tau, 0, o, lse, ws), 2 * reps)
    if not bool(torch.isfinite(o.float()).all()):
        raise RuntimeError("paged decode produced non-finite output")
    nbytes = (float(seqlens.astype("int64").sum()) * Hkv * d * 2 * 2 + 2 * B * Hq * d * 2
              + B * Hq * 4 + int(npb.sum()) * 4)
    out["decode_paged_gqa"] = {"shape": {"B": B, "Hq": Hq, "Hkv": Hkv, "page_size": P, "d": d},
                               "seqlens_sum": int(seqlens.sum()),
                               "num_splits": fa.decode_paged_num_splits(B, Hq, Hkv, P, maxp, d),
                               "input_copies": 2, "ms": ms, "GB/s": round(nbytes / ms / 1e6, 1),
                               "frac_hbm": round(nbytes / ms / 1e-3 / PEAK_HBM, 4)}
    del q, kp, vp, o, lse, ws, table, kv

    # backward: 4 x 16 x 4096 x 64, causal
    w = fa_inputs.WORKLOADS[5]
    B, H, N, d = w.B, w.H, w.N, w.d
    g.manual_seed(w.seed)
    q, k, v, do = (torch.randn(B, H, N, d, device=dev, generator=g).to(torch.bfloat16)
                   for _ in range(4))
    o, lse = fa.fwd(q, k, v, w.tau, True)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(B * H * N, device=dev)
    ms = med(lambda: fa.bwd(q, k, v, o, lse, do, w.tau, True, dq, dk, dv, ws))
    ms_dq = med(lambda: fa.bwd(q, k, v, o, lse, do, w.tau, True, dq, dk, dv, ws, stage=0))
    ms_dkdv = med(lambda: fa.bwd(q, k, v, o, lse, do, w.tau, True, dq, dk, dv, ws, stage=1))
    fl = 10.0 * B * H * N * N * d / 2
    out["bwd_recompute"] = {"shape": [B, H, N, d], "causal": True, "ms": ms,
                            "TFLOP/s": round(fl / ms / 1e9, 2),
                            "frac_mfma_bf16": round(fl / ms / 1e-3 / PEAK_MFMA_BF16, 4),
                            "dq_kernel_ms": ms_dq, "dkdv_kernel_ms": ms_dkdv,
                            "flops_convention": "10*B*H*N^2*d/2 (5 products incl. the S "
                                                "recompute, causal half)"}

    # the same shape with dropout p = 0.1 (Philox mask regenerated in the backward)
    drop = (0.1, 1005, 0)
    ms_f = med(lambda: fa.fwd(q, k, v, w.tau, True, o, lse, dropout=drop))
    ms_b = med(lambda: fa.bwd(q, k, v, o, lse, do, w.tau, True, dq, dk, dv, ws, dropout=drop))
    ffl = 4.0 * B * H * N * N * d / 2
    out["dropout"] = {"shape": [B, H, N, d], "causal": True, "p": 0.1,
                      "fwd_ms": ms_f, "fwd_TFLOP/s": round(ffl / ms_f / 1e9, 2),
                      "bwd_ms": ms_b, "bwd_TFLOP/s": round(fl / ms_b / 1e9, 2)}
    return out, gpu_out


def _blas_threads():
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        return max((i.get("num_threads") or 0) for i in info) if info else None
    except Exception:
        return None


def cpu_baseline(xh3, o3, lse3, gpu_extra=None):
    """The float64 oracle on the host.

    Headline: two whole heads of the long causal prefill (every row), timed;
    the rate in TFLOP/s is that of the oracle on those heads, and the GPU's O
    and LSE of the same heads are compared with it.  Also: the oracle's wall
    time on the other workloads (whole, or a stated sample extrapolated)."""
    from oracle import attention as orc

    import fa_inputs
    w = fa_inputs.WORKLOADS[3]
    qf, kf, vf = (xh3[n].f64() for n in ("q", "k", "v"))
    heads = (0, 31)
    t0 = time.perf_counter()
    ref = [orc.attention_fwd_head(qf[0, h], kf[0, h], vf[0, h], w.tau, True) for h in heads]
    dt = time.perf_counter() - t0
    fl = fwd_flops(1, len(heads), w.N, w.d, True)
    err_o = np.concatenate([np.abs(o3[0, h] - r[0]).ravel() for h, r in zip(heads, ref)])
    err_l = np.concatenate([np.abs(lse3[0, h] - r[1]).ravel() for h, r in zip(heads, ref)])
    out = {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s",
           "cores": _blas_threads() or os.cpu_count(), "kind": "oracle",
           "sample": "heads %s of the long causal prefill (1x32x16384x128, every row), float64 "
                     "NumPy with explicit score rows, %.1f s; the full 32-head job extrapolates "
                     "to %.0f s" % (list(heads), dt, dt * 16),
           "parity_sampled_heads": {"O_max_abs": float(err_o.max()), "O_mean_abs": float(err_o.mean()),
                                    "LSE_max_abs": float(err_l.max()),
                                    "bounds": "O max 2e-2, mean 2e-3; LSE 1e-3"}}
    other = {}
    # tiny fp32 forward: whole
    w1 = fa_inputs.WORKLOADS[1]
    x1 = fa_inputs.workload_inputs(w1)
    t0 = time.perf_counter()
    orc.attention_fwd(*(x1[n].f64() for n in ("q", "k", "v")), w1.tau, False)
    other["tiny_fp32_fwd"] = {"wall_s": round(time.perf_counter() - t0, 4), "sample": "whole"}
    # GPT-2-medium shape: both masks, whole; GPU outputs compared when given
    w2 = fa_inputs.WORKLOADS[2]
    x2 = fa_inputs.workload_inputs(w2)
    q2, k2, v2 = (x2[n].f64() for n in ("q", "k", "v"))
    t0 = time.perf_counter()
    r_nc = orc.attention_fwd(q2, k2, v2, w2.tau, False)
    r_c = orc.attention_fwd(q2, k2, v2, w2.tau, True)
    e = {"wall_s": round(time.perf_counter() - t0, 3), "sample": "whole, non-causal and causal"}
    if gpu_extra and "gpt2m" in gpu_extra:
        gm = gpu_extra["gpt2m"]
        for tag, key, r in (("noncausal", "o_nc", r_nc), ("causal", "o_c", r_c)):
            d = np.abs(gm[key] - r[0])
            e["O_%s_max_abs" % tag] = float(d.max())
            e["O_%s_mean_abs" % tag] = float(d.mean())
    other["gpt2m_fwd"] = e
    # backward workload: 4 of 64 heads, extrapolated x16
    w5 = fa_inputs.WORKLOADS[5]
    x5 = fa_inputs.workload_inputs(w5)
    q5, k5, v5, d5 = (x5[n].f64() for n in ("q", "k", "v", "do"))
    t0 = time.perf_counter()
    for b, h in ((0, 0), (1, 5), (2, 10), (3, 15)):
        orc.attention_bwd_head(q5[b, h], k5[b, h], v5[b, h], d5[b, h], w5.tau, True)
    t = time.perf_counter() - t0
    other["bwd_recompute"] = {"wall_s": round(t * 16, 2),
                              "sample": "4 of 64 heads (forward and gradients), extrapolated x16"}
    # split-KV decode: 8 of 64 sequences, extrapolated by their key count
    w4 = fa_inputs.WORKLOADS[4]
    sl = fa_inputs.decode_seqlens(w4.B, w4.lmin, w4.lmax, w4.seed + fa_inputs.SEED_OFFSET["seqlens"])
    x4 = fa_inputs.decode_inputs(8, w4.H, w4.N, w4.d, "bf16", w4.seed, sl[:8])
    t0 = time.perf_counter()
    orc.decode_fwd(x4["q"].f64(), x4["k"].f64(), x4["v"].f64(), x4["seqlens"], w4.tau)
    t = time.perf_counter() - t0
    other["decode_splitkv"] = {"wall_s": round(t * float(sl.sum()) / float(sl[:8].sum()), 2),
                               "sample": "8 of 64 sequences, extrapolated by key count"}
    out["other_workloads"] = other
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the synthetic matrix-core ceilings and the library GEMM")
    ap.add_argument("--lds-patterns", action="store_true",
                    help="only time the kernels' LDS read patterns alone (fa_calib.h), print one "
                         "JSON line and exit")
    ap.add_argument("--ceiling-seconds", type=float, default=1.2,
                    help="run time of each ceiling measurement (half of it timed)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB five times "
                         "(scales the HBM byte counters of a profiler run) and exit")
    ap.add_argument("--summarize-counters", nargs=4, default=None,
                    metavar=("FETCH_RUN", "FETCH_COPY", "WRITE_RUN", "WRITE_COPY"),
                    help="write profiles/traffic.json from four rocprofv3 --pmc output "
                         "directories (FETCH_SIZE and WRITE_SIZE, each over a headline run and a "
                         "--calibrate-copy 1024 run) and exit; runs on the host, no GPU")
    args = ap.parse_args(argv)
    if args.summarize_counters:
        d = args.summarize_counters
        cmds = ["rocprofv3 --pmc %s --output-format csv -d %s -o %s -- python -u bench.py %s"
                % (c, r, o, a) for c, r, o, a in (
                    ("FETCH_SIZE", d[0], "run", "--steps 5 --warmup 1 --no-extra --no-cpu --no-ceilings"),
                    ("FETCH_SIZE", d[1], "copy", "--calibrate-copy 1024"),
                    ("WRITE_SIZE", d[2], "run", "--steps 5 --warmup 1 --no-extra --no-cpu --no-ceilings"),
                    ("WRITE_SIZE", d[3], "copy", "--calibrate-copy 1024"))]
        summarize_counters(d[0], d[1], d[2], d[3], 1024, cmds)
        return 0
    if args.gpus != 1:
        print("bench.py: this attention path runs on one GPU; --gpus %d is not supported "
              "(sharding over (batch, head) is described in the design notes, not built)"
              % args.gpus, file=sys.stderr)
        return 2

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

    if args.lds_patterns:
        print(json.dumps({"lds_patterns": lds_patterns(fa)}))
        return 0

    w = fa_inputs.WORKLOADS[3]
    B, H, N, d, tau = w.B, w.H, w.N, w.d, w.tau
    xh = fa_inputs.workload_inputs(w)
    q, k, v = (upload(xh[n]) for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, device="cuda")
    run = lambda: fa.fwd(q, k, v, tau, True, o, lse)
    flops = fwd_flops(B, H, N, d, True)

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = [a.elapsed_time(b) for a, b in ev]
    timing = stats_ms(ev_ms)
    ms_step = wall / args.steps * 1e3
    value = flops / (wall / args.steps) / 1e12
    achieved = flops / timing["mean"] / 1e9
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_MFMA_BF16 / 1e12,
            "unit": "TFLOP/s", "frac": round(achieved * 1e12 / PEAK_MFMA_BF16, 4),
            "kernel": HEADLINE_KERNELS["long_causal_prefill"][0],
            "algorithmic_flops_per_launch": flops,
            "traffic": load_traffic("long_causal_prefill"),
            "algorithmic_bytes_per_launch": 4 * B * H * N * d * 2 + B * H * N * 4}
    o_host = o.float().cpu().numpy().astype(np.float64)
    lse_host = lse.cpu().numpy().astype(np.float64)
    if not (np.isfinite(o_host).all() and np.isfinite(lse_host).all()):
        raise RuntimeError("the headline forward produced non-finite output")
    clock = sample_clock(run)

    line = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: fp32 N(0,1) draws from PCG64 rounded to bf16 (seeds 1003, 1103, 1203)",
        "config": {"workload": "long-context causal prefill forward: B=1, H=32, N=16384, d=128, "
                               "bf16, causal, tau=1/sqrt(128)",
                   "B": B, "H": H, "N": N, "d": d, "tau": tau, "causal": True,
                   "seeds": {"q": w.seed, "k": w.seed + 100, "v": w.seed + 200},
                   "parallelism": "single GPU"},
        "frac_of_mfma_peak": round(value * 1e12 / PEAK_MFMA_BF16, 4),
        "timing_ms": timing,
        "roofline": roof,
        "sclk_mhz": clock,
        "bytes_avoided": bytes_avoided(B, H, N),
        "pages_context": PAGES_CONTEXT,
        "git": git_head(),
        "src_digest": src_digest(),
    }
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    if not args.no_ceilings:
        line["ceilings"] = ceilings(fa, achieved, args.ceiling_seconds)
    gpu_extra = None
    if not args.no_extra:
        line["also_measured"], gpu_extra = bench_extra(fa)
        if gpu_extra:
            gm = gpu_extra["gpt2m"]
            gpu_extra = {"gpt2m": {"o_nc": gm["o_nc"].float().cpu().numpy().astype(np.float64),
                                   "o_c": gm["o_c"].float().cpu().numpy().astype(np.float64)}}
    if "ceilings" in line and "also_measured" in line:
        hb = line["ceilings"]["hbm_stream_read"]["GB/s"]
        for key in ("decode_splitkv", "decode_paged_gqa"):
            if key in line["also_measured"]:
                am = line["also_measured"][key]
                am["fraction_of_hbm_stream_read"] = round(am["GB/s"] / hb, 4)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(xh, o_host, lse_host, gpu_extra)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
