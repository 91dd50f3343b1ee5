"""Plain float64 CPU oracle for exact attention.  TEST INFRASTRUCTURE ONLY.

Only the tests, the package's ``smoke()`` entry and the benchmark's CPU
baseline leg may import this module.  It shares no code with the HIP path and
imports nothing from it.

Notation and sources (the pages are cited by title and section):

* "flash-attention" encyclopedia page (tonho.wtf), section "o problema":
  standard attention computes S = Q K^T, P = softmax(S), O = P V, with S and P
  held in full.  The oracle does exactly that, in float64, per (batch, head).
* same page, section "como funciona": the scores carry a scale tau
  (S = tau * Q_i K_j^T), the softmax is decomposed with a running row maximum m
  and a running row sum l, and the backward keeps only O and (m, l) and uses
  D_i = P_i . dP_i = dO_i . O_i.
* "Atenção eficiente — FlashAttention, sparse e híbrida" (josenaldo.com.br),
  section "FlashAttention não acelera o decode": decode is one query row per
  sequence against the whole KV cache.

Readings where the pages are silent (each listed in the design notes):

* causal mask: key j is visible to query i iff j <= i (diagonal included),
  with as many queries as keys; decode sees every valid key of its sequence.
* the saved statistic is LSE = m + ln(l), natural log, of the tau-scaled
  scores; it replaces the pair (m, l).
* sliding window with sink tokens ("Atenção eficiente — FlashAttention, sparse
  e híbrida", sections "Atenção híbrida: local + global intercalados" — local
  layers attend to a window of w recent tokens — and "Attention sinks — o
  paradoxo do primeiro token" — StreamingLLM keeps the first few tokens and
  slides the window over the rest): on top of the causal mask, key j is
  visible to query i iff i - j < window or j < sinks.
* block-sparse attention ("flash-attention" page, "o que isso custou": the
  paper's answer to long sequences is block-sparse FlashAttention, an
  approximation): a block mask over (query block, key block) pairs of sizes
  bq x bk; key j is visible to query i only if block (i // bq, j // bk) is
  set (and j <= i under the causal mask).  A row with no visible key has the
  empty sum: O = 0 and LSE = -inf.
* dropout ("flash-attention" page, "o problema" lists dropout among the
  memory-bound steps of standard attention; "como funciona": the backward keeps
  the pseudo-random generator's state and regenerates the mask): after the
  softmax, P_ij is kept with probability 1 - p and scaled by 1/(1 - p), else
  zeroed; the row statistics (m, l, LSE) are those of the undropped P.  The
  mask comes from the counter-based generator Philox4x32-10 (Salmon et al.,
  "Parallel random numbers: as easy as 1, 2, 3", SC11), written here from its
  published definition: one generator call per 4 x 4 block of (query, key)
  pairs, counter (j/4, i/4, b*H + h, offset), key = the 64-bit seed; word i%4,
  byte j%4 is compared with round(256 p) (p is used as that multiple of 1/256).
* the gradients are derived by hand from O = softmax(tau Q K^T) V:
  dV = P^T dO, dP = dO V^T, D = rowsum(P o dP), dS = P o (dP - D),
  dQ = tau dS K, dK = tau dS^T Q.

Every function here is pinned by the tests in ``tests/test_oracle.py``
against closed forms, invariants, a hand-worked example, a library softmax
and central finite differences; none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "scores", "probs", "attention_fwd_head", "attention_fwd", "attention_bwd_head",
    "attention_bwd", "decode_fwd", "tiled_fwd_partials", "merge_partials", "split_kv_decode",
    "gather_pages", "decode_paged", "visible", "philox4x32_10",
    "dropout_threshold", "dropout_keep", "head_dropout", "head_block",
]


def visible(row_idx, key_idx, causal, window=None, sinks=0, block=None):
    """Boolean [rows, keys]: which keys each query row may attend to.

    causal: key j <= query i.  window (causal only): additionally i - j < window
    or j < sinks (a sliding window of the `window` most recent keys, the query's
    own included, plus the first `sinks` keys).  block = (mask, bq, bk): also
    mask[i // bq, j // bk] must be set (block-sparse attention)."""
    i = np.asarray(row_idx)[:, None]
    j = np.asarray(key_idx)[None, :]
    vis = np.ones((i.shape[0], j.shape[1]), dtype=bool)
    if causal:
        vis &= j <= i
    if window is not None:
        vis &= ((i - j) < window) | (j < sinks)
    if block is not None:
        mask, bq, bk = block
        vis &= np.asarray(mask, dtype=bool)[i // bq, j // bk]
    return vis


def scores(q_rows, k, tau, row_idx, causal, window=None, sinks=0, block=None):
    """S[r, j] = tau * q_rows[r] . k[j], with -inf where key j is not visible to
    query row_idx[r] ("o problema": S = Q K^T; "como funciona": the scale tau)."""
    s = tau * (np.asarray(q_rows, dtype=np.float64) @ np.asarray(k, dtype=np.float64).T)
    if causal or window is not None or block is not None:
        s = np.where(visible(row_idx, np.arange(k.shape[0]), causal, window, sinks, block), s,
                     -np.inf)
    return s


def probs(s):
    """Row softmax of a full score block: P = exp(S - m) / l, m = rowmax, l = rowsum.

    A row with no visible key (all -inf) has the empty sum: P = 0, m = -inf,
    l = 0 (so its LSE = m + ln l is -inf).  Returns (P, m, l)."""
    m = s.max(axis=1)
    live = np.isfinite(m)
    e = np.zeros_like(s)
    e[live] = np.exp(s[live] - m[live, None])
    l = e.sum(axis=1)
    p = np.zeros_like(s)
    p[live] = e[live] / l[live, None]
    return p, m, l


def _lse(m, l):
    with np.errstate(divide="ignore"):
        return m + np.log(l)


PHILOX_M = (0xD2511F53, 0xCD9E8D57)   # round multipliers
PHILOX_W = (0x9E3779B9, 0xBB67AE85)   # key increments between rounds


def philox4x32_10(ctr, key):
    """Philox4x32 with 10 rounds on arrays of counters.

    ctr: uint32-valued array [..., 4]; key: (k0, k1).  Each round multiplies
    words 0 and 2 by the two constants (64-bit products split into high and
    low halves) and outputs (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the key
    is advanced by the two Weyl constants before every round after the first.
    Returns the four output words as a uint32 array [..., 4]."""
    c = np.asarray(ctr, dtype=np.uint64) & np.uint64(0xFFFFFFFF)
    c0, c1, c2, c3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0, k1 = int(key[0]) & 0xFFFFFFFF, int(key[1]) & 0xFFFFFFFF
    mask = np.uint64(0xFFFFFFFF)
    for r in range(10):
        if r:
            k0 = (k0 + PHILOX_W[0]) & 0xFFFFFFFF
            k1 = (k1 + PHILOX_W[1]) & 0xFFFFFFFF
        p0 = np.uint64(PHILOX_M[0]) * c0
        p1 = np.uint64(PHILOX_M[1]) * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & mask
        hi1, lo1 = p1 >> np.uint64(32), p1 & mask
        c0, c1, c2, c3 = hi1 ^ c1 ^ np.uint64(k0), lo1, hi0 ^ c3 ^ np.uint64(k1), lo0
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def dropout_threshold(p):
    """The byte threshold t = round(256 p) (0..255); a pair is kept iff its
    byte >= t, so the drop probability used is t / 256."""
    t = int(round(float(p) * 256.0))
    if not (0 <= t <= 255):
        raise ValueError("dropout probability must round to at most 255/256")
    return t


def dropout_keep(rows, keys, bh, seed, offset, p):
    """Boolean [len(rows), len(keys)]: which (query, key) pairs of head bh
    (= b*H + h) survive dropout with probability p, for the given seed/offset."""
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    t = dropout_threshold(p)
    i = rows[:, None]
    j = keys[None, :]
    shape = (len(rows), len(keys))
    ctr = np.stack([np.broadcast_to(j // 4, shape), np.broadcast_to(i // 4, shape),
                    np.full(shape, bh), np.full(shape, int(offset) & 0xFFFFFFFF)], axis=-1)
    words = philox4x32_10(ctr, (int(seed) & 0xFFFFFFFF, (int(seed) >> 32) & 0xFFFFFFFF))
    word = np.take_along_axis(words, np.broadcast_to(i % 4, shape)[..., None], axis=-1)[..., 0]
    byte = (word >> (8 * np.broadcast_to(j % 4, shape)).astype(np.uint32)) & np.uint32(0xFF)
    return byte >= t


def _check_window(causal, window, sinks):
    if window is not None and (not causal or window < 1 or sinks < 0):
        raise ValueError("a window needs the causal mask, window >= 1 and sinks >= 0")


def attention_fwd_head(q, k, v, tau, causal, rows=None, chunk=1024, window=None, sinks=0,
                       drop=None, block=None):
    """Standard attention for one (batch, head): O[r] and LSE[r] for the requested rows.

    q: [Nq, d], k/v: [Nk, d].  The score rows are materialised whole, in chunks
    of at most ``chunk`` rows; under the causal mask a chunk computes scores only
    against keys up to its last query (the rest are masked, so exp gives 0).
    drop = (keep, p): dropout with the boolean mask keep(row_indices, key_indices)
    and probability p: O = (P o keep / (1 - p)) V; LSE is that of the undropped P.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if causal and q.shape[0] != k.shape[0]:
        raise ValueError("causal attention needs as many queries as keys")
    _check_window(causal, window, sinks)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.empty((len(rows), v.shape[1]))
    lse = np.empty(len(rows))
    for a in range(0, len(rows), chunk):
        r = rows[a:a + chunk]
        kmax = (int(r.max()) + 1) if causal else k.shape[0]
        s = scores(q[r], k[:kmax], tau, r, causal, window, sinks, block)
        p, m, l = probs(s)
        if drop is not None:
            keep, pd = drop
            p = p * keep(r, np.arange(kmax)) / (1.0 - pd)
        o[a:a + len(r)] = p @ v[:kmax]
        lse[a:a + len(r)] = _lse(m, l)
    return o, lse


def head_dropout(dropout, bh):
    """(keep, p) of head bh for dropout = (seed, offset, p), or None."""
    if dropout is None:
        return None
    seed, offset, p = dropout
    pe = dropout_threshold(p) / 256.0
    return (lambda rows, keys: dropout_keep(rows, keys, bh, seed, offset, p)), pe


def head_block(block, h):
    """(mask, bq, bk) of head h for block = (masks [1 or H, nbq, nbk], bq, bk), or None."""
    if block is None:
        return None
    masks, bq, bk = block
    masks = np.asarray(masks)
    return masks[h if masks.shape[0] > 1 else 0], bq, bk


def attention_fwd(q, k, v, tau, causal, window=None, sinks=0, dropout=None, block=None):
    """Standard attention over [B, H, N, d] tensors: returns O [B,H,N,d], LSE [B,H,N].
    dropout = (seed, offset, p): the dropout of head b*H + h as in head_dropout.
    block = (masks [1 or H, nbq, nbk], bq, bk): block-sparse (masks shared by
    every batch entry; one per head or one for all heads)."""
    B, H, N, d = q.shape
    o = np.empty((B, H, N, v.shape[-1]))
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = attention_fwd_head(q[b, h], k[b, h], v[b, h], tau, causal,
                                                    window=window, sinks=sinks,
                                                    drop=head_dropout(dropout, b * H + h),
                                                    block=head_block(block, h))
    return o, lse


def attention_bwd_head(q, k, v, do, tau, causal, window=None, sinks=0, drop=None, block=None):
    """Hand-derived gradients of O = softmax(tau Q K^T [+mask]) V for one head.

    With the loss's gradient dO:
      dV = P^T dO;  dP = dO V^T;  D_i = sum_j P_ij dP_ij;
      dS = P o (dP - D)  (zero on masked entries, where P = 0);
      dQ = tau dS K;  dK = tau dS^T Q.
    The identity D_i = dO_i . O_i ("como funciona", backward paragraph) is
    returned as a second form of D for the tests to compare.
    drop = (keep, p): dropout as in attention_fwd_head.  With Z = keep / (1 - p):
    O = (P o Z) V, dV = (P o Z)^T dO, dS = P o (Z o dP - D) with dP = dO V^T and
    D_i = sum_j P_ij Z_ij dP_ij = dO_i . O_i.
    Returns dict(dq, dk, dv, o, lse, D, D_from_o, p, pz (= P o Z), ds).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    _check_window(causal, window, sinks)
    n = q.shape[0]
    s = scores(q, k, tau, np.arange(n), causal, window, sinks, block)
    p, m, l = probs(s)
    z = 1.0 if drop is None else drop[0](np.arange(n), np.arange(k.shape[0])) / (1.0 - drop[1])
    o = (p * z) @ v
    dv = (p * z).T @ do
    dp = z * (do @ v.T)
    D = (p * dp).sum(axis=1)
    ds = p * (dp - D[:, None])
    dq = tau * (ds @ k)
    dk = tau * (ds.T @ q)
    return {"dq": dq, "dk": dk, "dv": dv, "o": o, "lse": _lse(m, l),
            "D": D, "D_from_o": (do * o).sum(axis=1), "p": p, "pz": p * z, "ds": ds}


def attention_bwd(q, k, v, do, tau, causal, window=None, sinks=0, dropout=None, block=None):
    """attention_bwd_head over [B, H, N, d]; returns dq, dk, dv, D as arrays."""
    B, H, N, d = q.shape
    out = {name: np.empty((B, H, N, d)) for name in ("dq", "dk", "dv")}
    out["D"] = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            g = attention_bwd_head(q[b, h], k[b, h], v[b, h], do[b, h], tau, causal, window, sinks,
                                   drop=head_dropout(dropout, b * H + h), block=head_block(block, h))
            for name in ("dq", "dk", "dv", "D"):
                out[name][b, h] = g[name]
    return out


def attention_dq_rows(q, k, v, do, tau, causal, rows, chunk=64):
    """dQ and D of the requested rows of one head, without the full N x N matrices.

    The same hand-derived gradient as attention_bwd_head, restricted to rows:
    for each row i, P_i over its visible keys, dP_i = dO_i V^T,
    D_i = sum_j P_ij dP_ij, dS_i = P_i o (dP_i - D_i), dQ_i = tau dS_i K.
    Score rows are formed in chunks of ``chunk`` rows (under the causal mask
    only against keys up to the chunk's last row).  Returns (dq, D)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    dq = np.empty((len(rows), k.shape[1]))
    D = np.empty(len(rows))
    for a in range(0, len(rows), chunk):
        r = rows[a:a + chunk]
        kmax = (int(r.max()) + 1) if causal else k.shape[0]
        p = probs(scores(q[r], k[:kmax], tau, r, causal))[0]
        dp = do[r] @ v[:kmax].T
        Dr = (p * dp).sum(axis=1)
        dq[a:a + len(r)] = tau * ((p * (dp - Dr[:, None])) @ k[:kmax])
        D[a:a + len(r)] = Dr
    return dq, D


def attention_dkdv_last_keys(q, k, v, do, tau, nk):
    """dK and dV of the last nk keys of one head under the causal mask.

    Key j is visible only to queries i >= j, so the last nk keys receive
    gradient only from the last nk query rows: their full score rows give P,
    dP = dO V^T, D and dS = P o (dP - D) (as attention_bwd_head), and then
    dV_j = sum_i P_ij dO_i and dK_j = tau sum_i dS_ij Q_i over those rows.
    Returns (dk, dv) of shape [nk, d]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    n = q.shape[0]
    r = np.arange(n - nk, n)
    p = probs(scores(q[r], k, tau, r, True))[0]
    dp = do[r] @ v.T
    ds = p * (dp - (p * dp).sum(axis=1)[:, None])
    dv = p[:, n - nk:].T @ do[r]
    dk = tau * (ds[:, n - nk:].T @ q[r])
    return dk, dv


def decode_fwd(q, k, v, seqlens, tau, heads=None, batches=None):
    """One query per (b, h) against keys [0, L_b) of the cache; no mask inside.

    q: [B,H,1,d]; k, v: [B,H,N_max,d] (rows at and beyond L_b are never read);
    seqlens: [B].  Returns O [B,H,1,d] and LSE [B,H] (entries outside the
    selected batches/heads are NaN).
    """
    B, H = q.shape[0], q.shape[1]
    batches = range(B) if batches is None else batches
    heads = range(H) if heads is None else heads
    o = np.full((B, H, 1, v.shape[-1]), np.nan)
    lse = np.full((B, H), np.nan)
    for b in batches:
        L = int(seqlens[b])
        for h in heads:
            oo, ll = attention_fwd_head(q[b, h], k[b, h, :L], v[b, h, :L], tau, False)
            o[b, h] = oo
            lse[b, h] = ll[0]
    return o, lse


def merge_partials(a, b):
    """Combine the softmax partials of two disjoint key sets.

    A partial over a key set J is (m, l, u): m = max_{j in J} S_j, l =
    sum_{j in J} exp(S_j - m) and u = sum_{j in J} exp(S_j - m) V_j (not
    normalised), per query row.  For the union of the two sets the reference
    becomes the larger maximum and each side is rescaled to it by exp(m_side -
    m) ("como funciona": the running maximum and sum are rescaled whenever a
    block is merged).  A side with no visible key (m = -inf) contributes
    nothing.  Arrays: m, l [rows], u [rows, d]."""
    (ma, la, ua), (mb, lb, ub) = a, b
    m = np.maximum(ma, mb)
    fa = np.zeros_like(m)
    fb = np.zeros_like(m)
    live = np.isfinite(m)
    fa[live] = np.exp(ma[live] - m[live])
    fb[live] = np.exp(mb[live] - m[live])
    return m, la * fa + lb * fb, ua * fa[:, None] + ub * fb[:, None]


def tiled_fwd_partials(q, k, v, tau, causal, Br, Bc, window=None, sinks=0, block=None):
    """Self-check of the block decomposition of the softmax, for one head.

    For each block of Br query rows and each block of Bc keys this forms the
    block's own partial (m, l, u) from its scores alone (the key block's
    maximum as reference), then combines the partials of a query block with
    merge_partials as a balanced binary tree (pairs of neighbouring key
    blocks, then pairs of pairs, ...), so the blocks are merged in a different
    order from any left-to-right sweep.  The pages claim the blocked result is
    the exact softmax, not an approximation ("flash-attention" page, "a
    ideia"): O = u / l and LSE = m + ln l must equal standard attention.
    A row that sees no key keeps m = -inf, l = 0: O = 0, LSE = -inf.
    Returns O [N, d] and LSE [N]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, nk = q.shape[0], k.shape[0]
    o = np.zeros((nq, v.shape[1]))
    lse = np.full(nq, -np.inf)
    masked = causal or window is not None or block is not None
    for i0 in range(0, nq, Br):
        rows = np.arange(i0, min(i0 + Br, nq))
        parts = []
        for j0 in range(0, nk, Bc):
            keys = np.arange(j0, min(j0 + Bc, nk))
            s = tau * (q[rows] @ k[keys].T)
            if masked:
                s = np.where(visible(rows, keys, causal, window, sinks, block), s, -np.inf)
            m = s.max(axis=1)
            e = np.zeros_like(s)
            live = np.isfinite(m)
            e[live] = np.exp(s[live] - m[live, None])
            parts.append((m, e.sum(axis=1), e @ v[keys]))
        while len(parts) > 1:
            nxt = [merge_partials(parts[t], parts[t + 1]) for t in range(0, len(parts) - 1, 2)]
            if len(parts) % 2:
                nxt.append(parts[-1])
            parts = nxt
        m, l, u = parts[0]
        live = l > 0
        o[rows[live]] = u[live] / l[live, None]
        lse[rows[live]] = m[live] + np.log(l[live])
    return o, lse


def split_kv_decode(q, k, v, tau, bounds):
    """Self-check of the split-KV decode for one (b, h): q [1,d], k/v [L,d].

    Each split s covers keys [bounds[s], bounds[s+1]) and yields its own
    normalised output o_s and lse_s = m_s + ln l_s (standard attention on the
    split).  The splits are merged by their log-sum-exp ("como funciona": the
    partial results of key blocks are combined through their row statistics):
    LSE = ln sum_s exp(lse_s), taken after subtracting max_s lse_s, and
    O = sum_s exp(lse_s - LSE) o_s.
    Returns O [1,d], LSE scalar.
    """
    parts = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        if b > a:
            parts.append(attention_fwd_head(q, k[a:b], v[a:b], tau, False))
    lses = np.array([p[1][0] for p in parts])
    mx = lses.max()
    lse = mx + np.log(np.exp(lses - mx).sum())
    o = sum(np.exp(ls - lse) * p[0] for ls, p in zip(lses, parts))
    return o, lse


def gather_pages(pages, block_table_row, kv_head, length, page_size):
    """Rows [0, length) of one sequence's cache for one KV head, read through
    its page table: key t lives in page block_table_row[t // page_size], row
    t % page_size.  pages: [num_pages, Hkv, page_size, d]."""
    idx = np.arange(length)
    page = np.asarray(block_table_row)[idx // page_size]
    return pages[page, kv_head, idx % page_size]


def decode_paged(q, k_pages, v_pages, block_table, seqlens, tau):
    """Decode with grouped KV heads over a paged cache.

    "Atenção eficiente — FlashAttention, sparse e híbrida": section
    "FlashAttention não acelera o decode token a token" (decode is bound by
    reading the KV cache, which MQA/GQA shrink; see also the page's "Veja
    também" list) and the table of section "Sparse e híbrida" (Paged Attention
    keeps the KV cache in memory pages).  Readings: query head h of Hq uses KV
    head h // (Hq / Hkv); key t of sequence b sits in page
    block_table[b, t // page_size] at row t % page_size.  Each (b, h) is then
    plain decode: one query against its L_b keys.
    q: [B, Hq, 1, d]; k_pages, v_pages: [num_pages, Hkv, page_size, d];
    block_table: [B, max_pages]; seqlens: [B].  Returns O [B,Hq,1,d], LSE [B,Hq].
    """
    B, Hq = q.shape[0], q.shape[1]
    Hkv, page_size = k_pages.shape[1], k_pages.shape[2]
    G = Hq // Hkv
    o = np.empty((B, Hq, 1, v_pages.shape[-1]))
    lse = np.empty((B, Hq))
    for b in range(B):
        L = int(seqlens[b])
        for h in range(Hq):
            kk = gather_pages(k_pages, block_table[b], h // G, L, page_size)
            vv = gather_pages(v_pages, block_table[b], h // G, L, page_size)
            oo, ll = attention_fwd_head(q[b, h], kk, vv, tau, False)
            o[b, h], lse[b, h] = oo, ll[0]
    return o, lse
