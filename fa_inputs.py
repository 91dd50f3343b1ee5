"""Seeded synthetic inputs for the attention workloads.

This module is shared by the HIP path's tests and benchmark and by the
oracle's tests.  It holds no attention arithmetic: only random draws, the
round-to-nearest-even conversion of those draws to bfloat16, and the table of
workload shapes.  Everything is deterministic in the seed.

Recipe
------
* Draws are IEEE fp32 standard normals from ``numpy.random.Generator(PCG64)``.
* bf16 tensors are those fp32 draws rounded to nearest-even to bfloat16; the
  device receives exactly those 16-bit patterns and the oracle receives the
  same values widened exactly to float64.
* Seeds: ``1000 + c`` for Q, ``+100`` for K, ``+200`` for V, ``+300`` for dO
  and ``+400`` for the decode key lengths, where ``c`` is the workload number
  (1..5) in ``WORKLOADS``.
* Decode K/V caches are drawn per batch entry from ``PCG64([seed, b])`` with
  shape ``[H, L_b, d]`` so that a single sequence can be regenerated alone;
  rows at and beyond ``L_b`` (the padding up to ``N_max``) hold NaN.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

BF16_NAN = np.uint16(0x7FC0)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention workload: shapes, dtype, scale and mask flag."""
    number: int
    name: str
    B: int
    H: int
    N: int          # query length (fwd/bwd) or N_max of the KV cache (decode)
    d: int
    dtype: str      # "f32" or "bf16"
    causal: tuple   # causal flags to run (the GPT-2-medium shape runs both)
    kind: str       # "fwd", "decode" or "bwd"
    lmin: int = 0   # decode only: key lengths drawn uniformly in [lmin, lmax]
    lmax: int = 0

    @property
    def tau(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def seed(self) -> int:
        return 1000 + self.number


WORKLOADS = {
    1: Workload(1, "tiny-fp32-fwd", 1, 1, 256, 64, "f32", (False,), "fwd"),
    2: Workload(2, "gpt2-medium-fwd", 8, 16, 1024, 64, "bf16", (False, True), "fwd"),
    3: Workload(3, "long-causal-prefill", 1, 32, 16384, 128, "bf16", (True,), "fwd"),
    4: Workload(4, "decode-splitkv", 64, 32, 8192, 128, "bf16", (False,), "decode",
                lmin=1024, lmax=8192),
    5: Workload(5, "bwd-recompute", 4, 16, 4096, 64, "bf16", (True,), "bwd"),
}

SEED_OFFSET = {"q": 0, "k": 100, "v": 200, "do": 300, "seqlens": 400}


@dataclasses.dataclass(frozen=True)
class PagedWorkload:
    """Decode over a paged cache with grouped KV heads: Hq query heads share
    Hkv KV heads; key lengths are those of the dense decode workload."""
    name: str
    B: int
    Hq: int
    Hkv: int
    page_size: int
    d: int
    lmin: int
    lmax: int
    seed: int
    seqlens_seed: int

    @property
    def tau(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def max_pages(self) -> int:
        return (self.lmax + self.page_size - 1) // self.page_size


# Llama-style grouping (4 query heads per KV head), 16-token pages, the dense
# decode workload's batch, head count, head size and key lengths.
PAGED_WORKLOAD = PagedWorkload("decode-paged-gqa", 64, 32, 8, 16, 128, 1024, 8192, 1006,
                               1004 + 400)


def normal_f32(shape, seed) -> np.ndarray:
    """fp32 standard normal draws from PCG64(seed)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal(size=shape, dtype=np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16, nearest-even; returns the uint16 patterns.

    NaN stays a quiet NaN.  Finite draws never overflow here.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = BF16_NAN
    return r


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of bfloat16 bit patterns."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


@dataclasses.dataclass
class HostTensor:
    """A tensor as the device sees it (``raw``) and its exact float64 value."""
    raw: np.ndarray      # float32 array or uint16 bf16 bit patterns
    dtype: str           # "f32" or "bf16"

    def f64(self) -> np.ndarray:
        if self.dtype == "bf16":
            return bf16_bits_to_f64(self.raw)
        return self.raw.astype(np.float64)


def draw(shape, seed, dtype) -> HostTensor:
    x = normal_f32(shape, seed)
    if dtype == "bf16":
        return HostTensor(bf16_bits(x), "bf16")
    return HostTensor(x, "f32")


def dense_inputs(B, H, N, d, dtype, seed, with_do=False) -> dict:
    """Q, K, V (and dO) of shape [B, H, N, d] drawn from the seed recipe."""
    shape = (B, H, N, d)
    out = {name: draw(shape, seed + SEED_OFFSET[name], dtype) for name in ("q", "k", "v")}
    if with_do:
        out["do"] = draw(shape, seed + SEED_OFFSET["do"], dtype)
    return out


def workload_inputs(w: Workload, scale_n=None) -> dict:
    """Dense inputs of a forward/backward workload (optionally with N replaced)."""
    N = w.N if scale_n is None else scale_n
    return dense_inputs(w.B, w.H, N, w.d, w.dtype, w.seed, with_do=(w.kind == "bwd"))


def decode_seqlens(B, lmin, lmax, seed) -> np.ndarray:
    """Per-sequence KV lengths, uniform on the integers [lmin, lmax]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(lmin, lmax, size=B, endpoint=True).astype(np.int32)


def decode_cache_rows(seed, b, H, L, d, dtype) -> HostTensor:
    """The valid rows [H, L, d] of sequence b's cache, from PCG64([seed, b])."""
    rng = np.random.Generator(np.random.PCG64([seed, b]))
    x = rng.standard_normal(size=(H, L, d), dtype=np.float32)
    return HostTensor(bf16_bits(x) if dtype == "bf16" else x, dtype)


def decode_inputs(B, H, N_max, d, dtype, seed, seqlens=None) -> dict:
    """Q [B,H,1,d] and NaN-padded K, V caches [B,H,N_max,d] plus seqlens_k."""
    if seqlens is None:
        raise ValueError("seqlens required")
    seqlens = np.asarray(seqlens, dtype=np.int32)
    q = draw((B, H, 1, d), seed + SEED_OFFSET["q"], dtype)
    caches = {}
    for name in ("k", "v"):
        if dtype == "bf16":
            arr = np.full((B, H, N_max, d), BF16_NAN, dtype=np.uint16)
        else:
            arr = np.full((B, H, N_max, d), np.nan, dtype=np.float32)
        for b in range(B):
            L = int(seqlens[b])
            arr[b, :, :L, :] = decode_cache_rows(seed + SEED_OFFSET[name], b, H, L, d, dtype).raw
        caches[name] = HostTensor(arr, dtype)
    return {"q": q, "k": caches["k"], "v": caches["v"], "seqlens": seqlens}


def workload_decode_inputs(w: Workload, B=None) -> dict:
    """Decode inputs of a decode workload (optionally only the first B sequences)."""
    Bn = w.B if B is None else B
    seqlens = decode_seqlens(w.B, w.lmin, w.lmax, w.seed + SEED_OFFSET["seqlens"])[:Bn]
    return decode_inputs(Bn, w.H, w.N, w.d, w.dtype, w.seed, seqlens)


def paged_workload_inputs(w: PagedWorkload = PAGED_WORKLOAD, B=None) -> dict:
    """Inputs of a paged workload (optionally only the first B sequences)."""
    Bn = w.B if B is None else B
    seqlens = decode_seqlens(w.B, w.lmin, w.lmax, w.seqlens_seed)[:Bn]
    return paged_decode_inputs(Bn, w.Hq, w.Hkv, w.page_size, w.d, "bf16", w.seed, seqlens,
                               max_pages=w.max_pages)


def paged_decode_inputs(B, Hq, Hkv, page_size, d, dtype, seed, seqlens, max_pages=None):
    """Q [B,Hq,1,d] and a paged KV cache for sequences of the given lengths.

    Pages: [num_pages, Hkv, page_size, d]; each sequence gets ceil(L_b /
    page_size) pages, the page table assigns them a random permutation of the
    page indices (seeded), and rows past L_b in a sequence's last page are NaN.
    Values: the same per-sequence draws as the dense decode recipe,
    decode_cache_rows(seed + offset, b, Hkv, L_b, d), scattered into pages.
    Returns dict(q, k_pages, v_pages, block_table [B, max_pages] int32, seqlens).
    """
    seqlens = np.asarray(seqlens, dtype=np.int32)
    npb = [(int(L) + page_size - 1) // page_size for L in seqlens]
    max_pages = max(1, max(npb)) if max_pages is None else max_pages
    num_pages = max(1, sum(npb))
    rng = np.random.Generator(np.random.PCG64(seed + 500))
    perm = rng.permutation(num_pages).astype(np.int32)
    table = np.zeros((B, max_pages), dtype=np.int32)
    nan = BF16_NAN if dtype == "bf16" else np.float32(np.nan)
    store = np.uint16 if dtype == "bf16" else np.float32
    pages = {n: np.full((num_pages, Hkv, page_size, d), nan, dtype=store) for n in ("k", "v")}
    nxt = 0
    for b in range(B):
        L = int(seqlens[b])
        ids = perm[nxt:nxt + npb[b]]
        nxt += npb[b]
        table[b, :len(ids)] = ids
        for n in ("k", "v"):
            rows = decode_cache_rows(seed + SEED_OFFSET[n], b, Hkv, L, d, dtype).raw
            for pi, pid in enumerate(ids):
                a, e = pi * page_size, min(L, (pi + 1) * page_size)
                pages[n][pid, :, :e - a] = rows[:, a:e]
    q = draw((B, Hq, 1, d), seed + SEED_OFFSET["q"], dtype)
    return {"q": q, "k_pages": HostTensor(pages["k"], dtype), "v_pages": HostTensor(pages["v"], dtype),
            "block_table": table, "seqlens": seqlens}
