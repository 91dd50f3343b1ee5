"""Pins of the float64 oracle against facts fixed by the pages and by mathematics.

Each test names what it pins.  None of them compares the oracle with itself:
they use closed forms, invariants, a hand-worked example, an independent
library softmax, the literal tiled recurrence and central finite differences.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import fa_inputs
from oracle import attention as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_example.json")


def _ev(expr):
    return eval(expr, {"__builtins__": {}}, {"ln": math.log})  # fixture written by hand


def _arr(x):
    if isinstance(x, str):
        return _ev(x)
    return np.array([[_ev(e) for e in row] if isinstance(row, list) else _ev(row) for row in x],
                    dtype=np.float64)


def _rand(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


# --- hand-worked example --------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_hand_example_forward_and_backward(causal):
    """Pins S = tau Q K^T (not K Q^T), the scale, the LSE base, the causal
    diagonal and every gradient formula against values worked by hand."""
    g = json.load(open(GOLDEN))
    tau = _ev(g["tau"])
    q, k, v, do = (_arr(g[n]) for n in ("q", "k", "v", "do"))
    exp = g["causal" if causal else "noncausal"]
    o, lse = orc.attention_fwd_head(q, k, v, tau, causal)
    np.testing.assert_allclose(o, _arr(exp["o"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, np.array([_ev(e) for e in exp["lse"]]), rtol=0, atol=1e-14)
    gr = orc.attention_bwd_head(q, k, v, do, tau, causal)
    for name in ("dv", "dq", "dk"):
        np.testing.assert_allclose(gr[name], _arr(exp[name]), rtol=0, atol=1e-14, err_msg=name)
    np.testing.assert_allclose(gr["D"], [_ev(e) for e in exp["D"]], rtol=0, atol=1e-14)
    np.testing.assert_allclose(gr["D_from_o"], [_ev(e) for e in exp["D"]], rtol=0, atol=1e-14)


def test_hand_example_decode():
    g = json.load(open(GOLDEN))
    tau = _ev(g["tau"])
    q, k, v = (_arr(g[n]) for n in ("q", "k", "v"))
    qd = q[1].reshape(1, 1, 1, 2)
    kk = np.full((1, 1, 4, 2), np.nan)
    vv = np.full((1, 1, 4, 2), np.nan)
    kk[0, 0, :2], vv[0, 0, :2] = k, v
    for L in (1, 2):
        o, lse = orc.decode_fwd(qd, kk, vv, np.array([L]), tau)
        e = g["decode"]["L%d" % L]
        np.testing.assert_allclose(o[0, 0, 0], [_ev(x) for x in e["o"]], atol=1e-14)
        assert abs(lse[0, 0] - _ev(e["lse"])) < 1e-14


# --- softmax normalisation and closed forms -------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows_sum_to_one(causal):
    """Softmax weights of every query sum to 1 (attention-sinks section of the
    "Atenção eficiente" page); so V = 1 gives O = 1."""
    n, d = 37, 8
    q, k = _rand((n, d), 1) * 3, _rand((n, d), 2) * 3
    s = orc.scores(q, k, 0.7, np.arange(n), causal)
    p, _, _ = orc.probs(s)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    if causal:
        assert np.all(p[np.triu_indices(n, 1)] == 0.0)
    o, _ = orc.attention_fwd_head(q, k, np.ones((n, 5)), 0.7, causal)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_is_uniform_average(causal):
    """Q = 0: all visible scores are 0, so P is uniform: O_i = mean of visible V
    and LSE_i = ln(#visible) (ln N, or ln(i+1) under the causal mask)."""
    n, d = 50, 16
    k, v = _rand((n, d), 3), _rand((n, d), 4)
    o, lse = orc.attention_fwd_head(np.zeros((n, d)), k, v, 0.25, causal)
    if causal:
        cnt = np.arange(1, n + 1)
        np.testing.assert_allclose(o, np.cumsum(v, axis=0) / cnt[:, None], atol=1e-13)
        np.testing.assert_allclose(lse, np.log(cnt), atol=1e-13)
    else:
        np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), atol=1e-13)
        np.testing.assert_allclose(lse, np.log(n), atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_average_values(causal):
    """All keys equal: every visible score of a row is the same, O = mean of V,
    and LSE_i = tau q_i.k + ln(#visible)."""
    n, d, tau = 33, 8, 0.3
    q, v = _rand((n, d), 5), _rand((n, d), 6)
    kvec = _rand((d,), 7)
    k = np.tile(kvec, (n, 1))
    o, lse = orc.attention_fwd_head(q, k, v, tau, causal)
    cnt = np.arange(1, n + 1) if causal else np.full(n, n)
    mean = np.cumsum(v, axis=0) / cnt[:, None] if causal else np.broadcast_to(v.mean(0), v.shape)
    np.testing.assert_allclose(o, mean, atol=1e-13)
    np.testing.assert_allclose(lse, tau * q @ kvec + np.log(cnt), atol=1e-12)


def test_dominant_score_selects_value_row():
    """One score larger than the others by >= 40 picks its V row, and huge
    scores (~1e4) neither overflow nor lose the row (max-shift stability)."""
    n, d = 20, 8
    rng = np.random.Generator(np.random.PCG64(8))
    q = rng.standard_normal((n, d))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    k = rng.standard_normal((n, d)) * 0.1
    v = rng.standard_normal((n, d))
    star = rng.permutation(n)
    for scale in (60.0, 1e4):
        # query i gets one dominant key, star[i], aligned with q_i; the other
        # keys are small, so the gap in scores is about `scale`.
        out = []
        for i in range(n):
            k2 = k.copy()
            k2[star[i]] = scale * q[i]
            o, lse = orc.attention_fwd_head(q[i:i + 1], k2, v, 1.0, False)
            out.append(o[0])
            assert np.isfinite(lse[0])
            assert abs(lse[0] - scale) < 1e-6 * scale
        np.testing.assert_allclose(np.array(out), v[star], atol=1e-12)


def test_softmax_matches_library_routine():
    """Row softmax and LSE agree with scipy.special.softmax/logsumexp."""
    n, d, tau = 40, 16, 0.2
    q, k = _rand((n, d), 9) * 4, _rand((n, d), 10) * 4
    s = orc.scores(q, k, tau, np.arange(n), False)
    p, _, _ = orc.probs(s)
    np.testing.assert_allclose(p, scipy.special.softmax(tau * q @ k.T, axis=1), atol=1e-14)
    _, lse = orc.attention_fwd_head(q, k, _rand((n, 3), 11), tau, False)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(tau * q @ k.T, axis=1), atol=1e-12)


def test_joint_key_value_permutation_invariance():
    """Non-causal attention does not depend on the order of the (key, value) pairs."""
    n, d = 29, 8
    q, k, v = _rand((n, d), 12), _rand((n, d), 13), _rand((n, d), 14)
    perm = np.random.Generator(np.random.PCG64(15)).permutation(n)
    o1, l1 = orc.attention_fwd_head(q, k, v, 0.4, False)
    o2, l2 = orc.attention_fwd_head(q, k[perm], v[perm], 0.4, False)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


def test_row_subset_and_chunking_agree_with_full():
    n, d = 300, 8
    q, k, v = _rand((n, d), 16), _rand((n, d), 17), _rand((n, d), 18)
    for causal in (False, True):
        o, lse = orc.attention_fwd_head(q, k, v, 0.3, causal)
        rows = np.array([0, 1, 63, 64, 150, 299])
        o2, l2 = orc.attention_fwd_head(q, k, v, 0.3, causal, rows=rows, chunk=4)
        np.testing.assert_allclose(o2, o[rows], atol=1e-13)
        np.testing.assert_allclose(l2, lse[rows], atol=1e-13)


# --- the tiled recurrence and the split-KV merge --------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("br,bc", [(16, 16), (7, 13), (13, 7), (1, 64), (64, 5), (100, 100)])
def test_tiled_recurrence_equals_standard(causal, br, bc):
    """Key-block partials (m, l, u) merged through their row statistics ("como
    funciona") give exactly standard attention ("a ideia": exact, not an
    approximation), whatever the block shapes and the merge order."""
    n, d = 61, 8
    q, k, v = _rand((n, d), 19) * 2, _rand((n, d), 20) * 2, _rand((n, d), 21)
    o, lse = orc.attention_fwd_head(q, k, v, 0.5, causal)
    ot, lt = orc.tiled_fwd_partials(q, k, v, 0.5, causal, br, bc)
    np.testing.assert_allclose(ot, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lt, lse, rtol=0, atol=1e-12)


def test_tiled_recurrence_catches_a_dropped_rescale():
    """The tiled check is sensitive: a merge that adds the partials of two key
    blocks without bringing them to a common reference maximum (a plausible
    kernel bug) moves the result far from standard attention, while the
    oracle's merge of the same two partials reproduces it."""
    n, d = 40, 8
    q, k, v = _rand((n, d), 22) * 3, _rand((n, d), 23) * 3, _rand((n, d), 24)
    o, _ = orc.attention_fwd_head(q, k, v, 0.5, False)

    def partial(keys):
        s = 0.5 * q @ k[keys].T
        m = s.max(axis=1)
        e = np.exp(s - m[:, None])
        return m, e.sum(axis=1), e @ v[keys]

    a, b = partial(np.arange(0, 17)), partial(np.arange(17, n))
    m, l, u = orc.merge_partials(a, b)
    np.testing.assert_allclose(u / l[:, None], o, atol=1e-12)
    bad = (a[2] + b[2]) / (a[1] + b[1])[:, None]
    assert np.abs(bad - o).max() > 1e-3


def test_merge_with_an_empty_side_keeps_the_other():
    """A key block with no visible key (m = -inf, l = 0, u = 0) leaves the
    other partial unchanged, in either order."""
    rng = np.random.default_rng(25)
    a = (rng.standard_normal(5), rng.random(5) + 0.5, rng.standard_normal((5, 3)))
    empty = (np.full(5, -np.inf), np.zeros(5), np.zeros((5, 3)))
    for x, y in ((a, empty), (empty, a)):
        m, l, u = orc.merge_partials(x, y)
        np.testing.assert_array_equal(m, a[0])
        np.testing.assert_array_equal(l, a[1])
        np.testing.assert_array_equal(u, a[2])


def test_split_kv_merge_equals_unsplit():
    """Merging split-KV partials by their LSE reproduces single-pass decode."""
    d, L = 16, 517
    q = _rand((1, d), 25)
    k, v = _rand((L, d), 26) * 2, _rand((L, d), 27)
    o, lse = orc.attention_fwd_head(q, k, v, 0.25, False)
    for bounds in ([0, L], [0, 100, L], [0, 1, 2, 300, 301, L], list(range(0, L, 64)) + [L]):
        o2, l2 = orc.split_kv_decode(q, k, v, 0.25, bounds)
        np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
        assert abs(l2 - lse[0]) < 1e-12


def test_decode_is_last_row_of_causal_attention():
    """A decode step is the newest query of causal attention: it sees every key."""
    n, d = 45, 8
    q, k, v = _rand((n, d), 28), _rand((n, d), 29), _rand((n, d), 30)
    o, lse = orc.attention_fwd_head(q, k, v, 0.35, True)
    kk = np.full((1, 1, 64, d), np.nan); vv = np.full((1, 1, 64, d), np.nan)
    kk[0, 0, :n], vv[0, 0, :n] = k, v
    od, ld = orc.decode_fwd(q[-1].reshape(1, 1, 1, d), kk, vv, np.array([n]), 0.35)
    np.testing.assert_allclose(od[0, 0, 0], o[-1], atol=1e-13)
    assert abs(ld[0, 0] - lse[-1]) < 1e-13


# --- backward --------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_backward_D_identity(causal):
    """D_i = P_i . dP_i equals dO_i . O_i ("como funciona", backward)."""
    n, d = 40, 8
    q, k, v, do = (_rand((n, d), s) for s in (31, 32, 33, 34))
    g = orc.attention_bwd_head(q, k, v, do, 0.5, causal)
    np.testing.assert_allclose(g["D"], g["D_from_o"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_column_sum_invariants(causal):
    """Rows of P sum to 1, so sum_j dS_ij = 0: sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i."""
    n, d = 48, 8
    q, k, v, do = (_rand((n, d), s) for s in (35, 36, 37, 38))
    g = orc.attention_bwd_head(q, k, v, do, 0.4, causal)
    np.testing.assert_allclose(g["dk"].sum(axis=0), 0.0, atol=1e-12)
    np.testing.assert_allclose(g["dv"].sum(axis=0), do.sum(axis=0), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_dq_rows_match_finite_differences_and_full_backward(causal):
    """attention_dq_rows (the row-sampled dQ for heads too long for the full
    matrices): central differences of L = sum(O o dO) with respect to the
    sampled rows of Q (rel <= 1e-6), and the full-head backward's rows, with
    chunks that split the sampled rows unevenly."""
    n, d, tau, h = 11, 4, 0.7, 1e-6
    rng = np.random.Generator(np.random.PCG64(140 + causal))
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    rows = np.array([0, 3, 4, 10])
    dq, D = orc.attention_dq_rows(q, k, v, do, tau, causal, rows, chunk=3)

    def loss(qq):
        o, _ = orc.attention_fwd_head(qq, k, v, tau, causal)
        return float((o * do).sum())

    num = np.empty((len(rows), d))
    for a, i in enumerate(rows):
        for j in range(d):
            qp, qm = q.copy(), q.copy()
            qp[i, j] += h
            qm[i, j] -= h
            num[a, j] = (loss(qp) - loss(qm)) / (2 * h)
    np.testing.assert_allclose(dq, num, rtol=1e-6, atol=1e-8)
    g = orc.attention_bwd_head(q, k, v, do, tau, causal)
    np.testing.assert_allclose(dq, g["dq"][rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(D, g["D"][rows], rtol=0, atol=1e-12)


@pytest.mark.parametrize("nk", [1, 3, 7])
def test_dkdv_last_keys_match_finite_differences_and_full_backward(nk):
    """attention_dkdv_last_keys: central differences of L = sum(O o dO) with
    respect to the last keys and values (rel <= 1e-6), and the full-head causal
    backward's last rows."""
    n, d, tau, h = 10, 3, 0.8, 1e-6
    rng = np.random.Generator(np.random.PCG64(150 + nk))
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    dk, dv = orc.attention_dkdv_last_keys(q, k, v, do, tau, nk)

    def loss(kk, vv):
        o, _ = orc.attention_fwd_head(q, kk, vv, tau, True)
        return float((o * do).sum())

    for got, idx in ((dk, 0), (dv, 1)):
        num = np.empty((nk, d))
        for a, i in enumerate(range(n - nk, n)):
            for j in range(d):
                plus, minus = [k.copy(), v.copy()], [k.copy(), v.copy()]
                plus[idx][i, j] += h
                minus[idx][i, j] -= h
                num[a, j] = (loss(*plus) - loss(*minus)) / (2 * h)
        np.testing.assert_allclose(got, num, rtol=1e-6, atol=1e-8)
    g = orc.attention_bwd_head(q, k, v, do, tau, True)
    np.testing.assert_allclose(dk, g["dk"][n - nk:], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, g["dv"][n - nk:], rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(5, 3), (9, 4), (16, 8)])
def test_backward_matches_finite_differences(causal, n, d):
    """Central differences of L = sum(O o dO) match dQ, dK and dV (rel <= 1e-6)."""
    tau, h = 0.6, 1e-6
    rng = np.random.Generator(np.random.PCG64(100 + n))
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    g = orc.attention_bwd_head(q, k, v, do, tau, causal)

    def loss(qq, kk, vv):
        o, _ = orc.attention_fwd_head(qq, kk, vv, tau, causal)
        return float((o * do).sum())

    for name, idx in (("dq", 0), ("dk", 1), ("dv", 2)):
        base = [q, k, v]
        num = np.empty((n, d))
        for i in range(n):
            for j in range(d):
                plus = [x.copy() for x in base]
                minus = [x.copy() for x in base]
                plus[idx][i, j] += h
                minus[idx][i, j] -= h
                num[i, j] = (loss(*plus) - loss(*minus)) / (2 * h)
        err = np.abs(num - g[name]).max() / max(np.abs(num).max(), 1e-30)
        assert err <= 1e-6, (name, err)


def test_batched_wrappers_match_per_head():
    B, H, n, d = 2, 3, 17, 4
    rng = np.random.Generator(np.random.PCG64(40))
    q, k, v, do = (rng.standard_normal((B, H, n, d)) for _ in range(4))
    o, lse = orc.attention_fwd(q, k, v, 0.5, True)
    g = orc.attention_bwd(q, k, v, do, 0.5, True)
    for b in range(B):
        for hh in range(H):
            o1, l1 = orc.attention_fwd_head(q[b, hh], k[b, hh], v[b, hh], 0.5, True)
            g1 = orc.attention_bwd_head(q[b, hh], k[b, hh], v[b, hh], do[b, hh], 0.5, True)
            np.testing.assert_allclose(o[b, hh], o1, atol=0)
            np.testing.assert_allclose(lse[b, hh], l1, atol=0)
            for name in ("dq", "dk", "dv"):
                np.testing.assert_allclose(g[name][b, hh], g1[name], atol=0)


# --- the shared input generator --------------------------------------------

def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5, 3.0e38, 1e-40, np.nan],
                 dtype=np.float32)
    bits = fa_inputs.bf16_bits(x)
    back = fa_inputs.bf16_bits_to_f64(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins;
    # 1 + 3*2^-8 ties between 1+2^-7 and 1+2^-6: 1 + 2^-6 has the even mantissa.
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == 1.0 + 2**-6
    assert back[3] == 1.0 and back[4] == -2.5
    assert np.isfinite(back[5]) and abs(back[5] - 3.0e38) / 3.0e38 < 2**-8
    assert np.isnan(back[7])
    r = fa_inputs.normal_f32((1000,), 1)
    rb = fa_inputs.bf16_bits_to_f64(fa_inputs.bf16_bits(r))
    assert np.all(np.abs(rb - r) <= np.abs(r) * 2**-8 + 1e-45)


def test_decode_inputs_poison_padding():
    d = fa_inputs.decode_inputs(3, 2, 40, 8, "bf16", 5, seqlens=[1, 39, 40])
    kf = d["k"].f64()
    assert np.all(np.isnan(kf[0, :, 1:])) and np.all(np.isfinite(kf[0, :, :1]))
    assert np.all(np.isnan(kf[1, :, 39:])) and np.all(np.isfinite(kf[2]))
    s = fa_inputs.decode_seqlens(64, 1024, 8192, 1404)
    assert s.min() >= 1024 and s.max() <= 8192


# --- grouped KV heads and the paged cache ---------------------------------

def test_paged_decode_equals_dense_decode_of_the_gathered_cache():
    """Reading through the page table gives the same keys as a dense cache:
    with one KV head per query head (G = 1) paged decode is dense decode."""
    seqlens = [1, 17, 40, 64]
    x = fa_inputs.paged_decode_inputs(4, 2, 2, 16, 8, "f32", 77, seqlens)
    dense = fa_inputs.decode_inputs(4, 2, 64, 8, "f32", 77, seqlens=seqlens)
    o1, l1 = orc.decode_paged(x["q"].f64(), x["k_pages"].f64(), x["v_pages"].f64(),
                              x["block_table"], x["seqlens"], 0.3)
    o2, l2 = orc.decode_fwd(dense["q"].f64(), dense["k"].f64(), dense["v"].f64(), seqlens, 0.3)
    np.testing.assert_allclose(o1, o2, atol=0)
    np.testing.assert_allclose(l1, l2, atol=0)


def test_grouped_heads_share_kv_and_mqa_matches_repeated_heads():
    """Query heads of one group see the same keys: with all query heads equal
    inside a group the outputs coincide, and MQA (one KV head) equals MHA with
    that KV head repeated for every query head."""
    seqlens = [30, 5]
    x = fa_inputs.paged_decode_inputs(2, 4, 1, 16, 8, "f32", 78, seqlens)
    q = x["q"].f64()
    kp, vp = x["k_pages"].f64(), x["v_pages"].f64()
    o, l = orc.decode_paged(q, kp, vp, x["block_table"], x["seqlens"], 0.5)
    rep_k = np.repeat(kp, 4, axis=1)
    rep_v = np.repeat(vp, 4, axis=1)
    o2, l2 = orc.decode_paged(q, rep_k, rep_v, x["block_table"], x["seqlens"], 0.5)
    np.testing.assert_allclose(o, o2, atol=0)
    q_same = np.repeat(q[:, :1], 4, axis=1)
    o3, _ = orc.decode_paged(q_same, kp, vp, x["block_table"], x["seqlens"], 0.5)
    for h in range(1, 4):
        np.testing.assert_allclose(o3[:, h], o3[:, 0], atol=0)
    # hand check of the grouping rule h -> h // G with two KV heads
    x2 = fa_inputs.paged_decode_inputs(1, 4, 2, 16, 8, "f32", 79, [9])
    o4, _ = orc.decode_paged(x2["q"].f64(), x2["k_pages"].f64(), x2["v_pages"].f64(),
                             x2["block_table"], x2["seqlens"], 0.5)
    for h in range(4):
        kk = x2["k_pages"].f64()[x2["block_table"][0, 0], h // 2, :9]
        vv = x2["v_pages"].f64()[x2["block_table"][0, 0], h // 2, :9]
        oo, _ = orc.attention_fwd_head(x2["q"].f64()[0, h], kk, vv, 0.5, False)
        np.testing.assert_allclose(o4[0, h], oo, atol=1e-14)


def test_paged_inputs_poison_unused_rows():
    x = fa_inputs.paged_decode_inputs(2, 2, 1, 16, 8, "bf16", 80, [20, 16])
    kp = x["k_pages"].f64()
    t = x["block_table"]
    assert np.all(np.isfinite(kp[t[0, 0]])) and np.all(np.isfinite(kp[t[0, 1], :, :4]))
    assert np.all(np.isnan(kp[t[0, 1], :, 4:]))
    assert sorted(t[0, :2].tolist() + t[1, :1].tolist()) == [0, 1, 2]


# --- sliding window with sink tokens ---------------------------------------

def _qkv(n, d, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((n, d)), rng.standard_normal((n, d)), rng.standard_normal((n, d))


def test_window_covering_everything_is_causal():
    q, k, v = _qkv(40, 8, 501)
    o1, l1 = orc.attention_fwd_head(q, k, v, 0.3, True)
    for w, s in ((40, 0), (1000, 0), (1, 40), (5, 64)):
        o2, l2 = orc.attention_fwd_head(q, k, v, 0.3, True, window=w, sinks=s)
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)


def test_window_one_sees_only_itself():
    """window = 1, no sinks: every query attends to its own key only, so
    O_i = V_i and LSE_i = tau q_i . k_i."""
    q, k, v = _qkv(17, 6, 502)
    o, l = orc.attention_fwd_head(q, k, v, 0.7, True, window=1)
    np.testing.assert_allclose(o, v, atol=1e-15)
    np.testing.assert_allclose(l, 0.7 * np.einsum("id,id->i", q, k), atol=1e-13)


@pytest.mark.parametrize("w,s", [(1, 1), (3, 0), (3, 2), (7, 4), (20, 3)])
def test_window_uniform_weights_closed_form(w, s):
    """Q = 0: uniform weights over the visible set {max(0, i-w+1) .. i} plus
    the sinks {0 .. min(s, i+1)-1} below it; O_i is that set's mean of V and
    LSE_i = ln |set|, |set| = min(i+1, w) + max(0, min(s, i-w+1))."""
    n, d = 30, 5
    _, k, v = _qkv(n, d, 503)
    q = np.zeros((n, d))
    o, l = orc.attention_fwd_head(q, k, v, 0.5, True, window=w, sinks=s)
    for i in range(n):
        lo = max(0, i - w + 1)
        rows = list(range(lo, i + 1)) + list(range(0, min(s, lo)))
        assert len(rows) == min(i + 1, w) + max(0, min(s, i - w + 1))
        np.testing.assert_allclose(o[i], v[rows].mean(axis=0), atol=1e-14)
        np.testing.assert_allclose(l[i], np.log(len(rows)), atol=1e-14)


@pytest.mark.parametrize("Br,Bc", [(16, 16), (7, 13), (13, 7), (64, 5)])
@pytest.mark.parametrize("w,s", [(1, 0), (9, 0), (9, 3), (50, 4)])
def test_tiled_recurrence_with_window(Br, Bc, w, s):
    """The tiled recurrence with the window mask (whole block rows masked
    before and after the window) equals the direct computation."""
    q, k, v = _qkv(70, 8, 504)
    o1, l1 = orc.attention_fwd_head(q, k, v, 0.4, True, window=w, sinks=s)
    o2, l2 = orc.tiled_fwd_partials(q, k, v, 0.4, True, Br, Bc, window=w, sinks=s)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(l2, l1, atol=1e-12)


@pytest.mark.parametrize("w,s", [(1, 0), (3, 0), (3, 2), (6, 1)])
def test_window_gradients_finite_differences(w, s):
    n, d, tau = 9, 4, 0.6
    q, k, v = _qkv(n, d, 505)
    do = np.random.default_rng(506).standard_normal((n, d))
    g = orc.attention_bwd_head(q, k, v, do, tau, True, window=w, sinks=s)
    f = lambda qq, kk, vv: float((orc.attention_fwd_head(qq, kk, vv, tau, True, window=w,
                                                         sinks=s)[0] * do).sum())
    h = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [xp if x is a else a for a in (q, k, v)]
            args_m = [xm if x is a else a for a in (q, k, v)]
            num[idx] = (f(*args_p) - f(*args_m)) / (2 * h)
        np.testing.assert_allclose(g[name], num, rtol=1e-6, atol=1e-8)
    # the identities hold under any mask that keeps every row non-empty
    np.testing.assert_allclose(g["D"], g["D_from_o"], atol=1e-12)
    np.testing.assert_allclose(g["dk"].sum(axis=0), 0, atol=1e-12)
    np.testing.assert_allclose(g["dv"].sum(axis=0), do.sum(axis=0), atol=1e-12)


def test_window_needs_causal():
    q, k, v = _qkv(4, 2, 507)
    with pytest.raises(ValueError):
        orc.attention_fwd_head(q, k, v, 1.0, False, window=2)
    with pytest.raises(ValueError):
        orc.attention_fwd_head(q, k, v, 1.0, True, window=0)


# --- dropout: Philox4x32-10 and the dropped attention -------------------------

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_philox_known_answers():
    """Philox4x32-10 reproduces the generator's published known-answer vectors."""
    kat = json.load(open(os.path.join(GOLDEN_DIR, "philox4x32_10_kat.json")))
    for v in kat["vectors"]:
        ctr = np.array([int(x, 16) for x in v["ctr"]], dtype=np.uint64)
        key = [int(x, 16) for x in v["key"]]
        out = orc.philox4x32_10(ctr[None, :], key)[0]
        assert [int(x) for x in out] == [int(x, 16) for x in v["out"]]


# Keep patterns of one 4 x 4 block of (query, key) pairs, written out by hand
# from the published Philox4x32-10 known-answer vectors (the golden file
# above) under the layout the design notes fix: counter (j/4, i/4, b*H + h,
# offset), key (seed low word, seed high word), pair (i, j) kept iff byte j%4
# (byte 0 = least significant) of output word i%4 is >= round(256 p).
#   ctr 0, key 0 -> 6627e8d5 e169c58d bc57ac4c 9b00dbd8, bytes by row:
#     d5 e8 27 66 | 8d c5 69 e1 | 4c ac 57 bc | d8 db 00 9b
#   ctr ffffffff x4, key ffffffff x2 -> 408f276d 41c83b0e a20bc7c6 6d5451fd:
#     6d 27 8f 40 | 0e 3b c8 41 | c6 c7 0b a2 | fd 51 54 6d
#   ctr 243f6a88 85a308d3 13198a2e 03707344, key a4093822 299f31d0
#     -> d16cfe09 94fdcceb 5001e420 24126ea1:
#     09 fe 6c d1 | eb cc fd 94 | 20 e4 01 50 | a1 6e 12 24
HAND_BLOCKS = [
    # (i/4, j/4, head, offset, seed, p, rows of the keep pattern)
    (0, 0, 0, 0, 0, 0.5, ["1100", "1101", "0101", "1101"]),
    (0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFFFFFFFFFF, 0.5,
     ["0010", "0010", "1101", "1000"]),
    (0x85A308D3, 0x243F6A88, 0x13198A2E, 0x03707344, 0x299F31D0A4093822, 0.5,
     ["0101", "1111", "0100", "1000"]),
    (0x85A308D3, 0x243F6A88, 0x13198A2E, 0x03707344, 0x299F31D0A4093822, 0.25,
     ["0111", "1111", "0101", "1100"]),
]


@pytest.mark.parametrize("blk", HAND_BLOCKS)
def test_dropout_mask_layout_from_published_vectors(blk):
    """Pins which counter word carries the key index and which the query index,
    the seed's word order, the head and offset words, the word/byte choice
    within a block and the threshold comparison: each hand-written pattern
    comes from a published output vector, not from the oracle's code (swapping
    the query and key roles, or words and bytes, gives other patterns)."""
    i4, j4, bh, offset, seed, p, want = blk
    keep = orc.dropout_keep(4 * i4 + np.arange(4), 4 * j4 + np.arange(4), bh, seed, offset, p)
    got = ["".join("1" if x else "0" for x in row) for row in keep]
    assert got == want


def test_dropout_threshold_and_rate():
    assert orc.dropout_threshold(0.0) == 0 and orc.dropout_threshold(0.5) == 128
    assert orc.dropout_threshold(0.1) == 26
    with pytest.raises(ValueError):
        orc.dropout_threshold(0.999)
    keep = orc.dropout_keep(np.arange(256), np.arange(512), 3, 1234567, 0, 0.1)
    rate = 1 - keep.mean()
    pe = 26 / 256
    sigma = np.sqrt(pe * (1 - pe) / keep.size)
    assert abs(rate - pe) < 5 * sigma
    # p = 0 keeps everything; other heads, seeds and offsets give other masks
    assert orc.dropout_keep(np.arange(64), np.arange(64), 0, 9, 0, 0.0).all()
    base = orc.dropout_keep(np.arange(64), np.arange(64), 0, 9, 0, 0.5)
    for other in ((1, 9, 0), (0, 10, 0), (0, 9, 1), (0, 9 + (1 << 32), 0)):
        m = orc.dropout_keep(np.arange(64), np.arange(64), other[0], other[1], other[2], 0.5)
        assert (m != base).mean() > 0.3


def test_dropout_zero_probability_is_plain_attention():
    q, k, v = _qkv(30, 8, 701)
    for causal in (False, True):
        o1, l1 = orc.attention_fwd_head(q, k, v, 0.4, causal)
        o2, l2 = orc.attention_fwd_head(q, k, v, 0.4, causal, drop=orc.head_dropout((5, 0, 0.0), 0))
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)


def test_dropout_uniform_weights_closed_form():
    """Q = 0: P_ij = 1/n_i over the visible keys, so O_i = sum over kept
    visible keys of V_j / (n_i (1 - p)); the LSE ignores dropout (ln n_i)."""
    n, d, p = 24, 6, 0.25
    _, k, v = _qkv(n, d, 702)
    q = np.zeros((n, d))
    keep, pe = orc.head_dropout((77, 3, p), 5)
    o, l = orc.attention_fwd_head(q, k, v, 0.5, True, drop=(keep, pe))
    km = keep(np.arange(n), np.arange(n))
    for i in range(n):
        kept = [j for j in range(i + 1) if km[i, j]]
        want = v[kept].sum(axis=0) / ((i + 1) * (1 - pe)) if kept else np.zeros(d)
        np.testing.assert_allclose(o[i], want, atol=1e-14)
        np.testing.assert_allclose(l[i], np.log(i + 1), atol=1e-14)


def test_dropout_expectation():
    """Averaged over seeds the dropped output tends to the undropped one
    (E[keep / (1 - p)] = 1)."""
    q, k, v = _qkv(12, 4, 703)
    o_ref, _ = orc.attention_fwd_head(q, k, v, 0.5, True)
    acc = np.zeros_like(o_ref)
    S = 400
    for seed in range(S):
        acc += orc.attention_fwd_head(q, k, v, 0.5, True, drop=orc.head_dropout((seed, 0, 0.3), 0))[0]
    assert np.abs(acc / S - o_ref).max() < 0.25


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_gradients_finite_differences(causal):
    """With the mask fixed (it depends on indices and the seed only) the
    dropped attention is a smooth function of Q, K, V: central differences
    match dQ, dK, dV; D = dO . O and sum_j dK_j = 0 still hold."""
    n, d, tau = 10, 4, 0.7
    q, k, v = _qkv(n, d, 704)
    do = np.random.default_rng(705).standard_normal((n, d))
    drop = orc.head_dropout((31337, 1, 0.4), 2)
    g = orc.attention_bwd_head(q, k, v, do, tau, causal, drop=drop)
    f = lambda qq, kk, vv: float((orc.attention_fwd_head(qq, kk, vv, tau, causal, drop=drop)[0]
                                  * do).sum())
    h = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            num[idx] = (f(*[xp if x is a else a for a in (q, k, v)])
                        - f(*[xm if x is a else a for a in (q, k, v)])) / (2 * h)
        np.testing.assert_allclose(g[name], num, rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(g["D"], g["D_from_o"], atol=1e-12)
    np.testing.assert_allclose(g["dk"].sum(axis=0), 0, atol=1e-12)
    o_fwd, _ = orc.attention_fwd_head(q, k, v, tau, causal, drop=drop)
    np.testing.assert_allclose(g["o"], o_fwd, atol=1e-14)


# --- block-sparse attention -------------------------------------------------

def test_block_mask_all_ones_is_dense():
    q, k, v = _qkv(50, 8, 801)
    for causal in (False, True):
        o1, l1 = orc.attention_fwd_head(q, k, v, 0.3, causal)
        ones = np.ones((4, 7), dtype=np.uint8)
        o2, l2 = orc.attention_fwd_head(q, k, v, 0.3, causal, block=(ones, 16, 8))
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)


def test_block_lower_triangle_with_causal_is_causal():
    """A lower-triangular block mask (square blocks) under the causal mask
    drops only blocks the causal mask drops anyway."""
    q, k, v = _qkv(64, 8, 802)
    tri = np.tril(np.ones((4, 4), dtype=np.uint8))
    o1, l1 = orc.attention_fwd_head(q, k, v, 0.3, True)
    o2, l2 = orc.attention_fwd_head(q, k, v, 0.3, True, block=(tri, 16, 16))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_block_diagonal_is_independent_segments():
    """A block-diagonal mask makes each block of rows attend to its own block
    of keys only: standard attention on each segment separately."""
    n, bs = 48, 16
    q, k, v = _qkv(n, 6, 803)
    diag = np.eye(n // bs, dtype=np.uint8)
    for causal in (False, True):
        o, l = orc.attention_fwd_head(q, k, v, 0.5, causal, block=(diag, bs, bs))
        for a in range(0, n, bs):
            oo, ll = orc.attention_fwd_head(q[a:a + bs], k[a:a + bs], v[a:a + bs], 0.5, causal)
            np.testing.assert_allclose(o[a:a + bs], oo, atol=1e-14)
            np.testing.assert_allclose(l[a:a + bs], ll, atol=1e-14)


def test_block_uniform_weights_and_empty_rows():
    """Q = 0: O_i is the mean of V over the visible keys and LSE_i = ln(count);
    a row whose blocks are all clear has O = 0 and LSE = -inf."""
    n, d = 40, 4
    _, k, v = _qkv(n, d, 804)
    q = np.zeros((n, d))
    mask = np.array([[1, 0, 1], [0, 0, 0], [1, 1, 0], [0, 1, 1], [1, 0, 0]], dtype=np.uint8)
    o, l = orc.attention_fwd_head(q, k, v, 0.5, False, block=(mask, 8, 16))
    for i in range(n):
        keys = [j for j in range(n) if mask[i // 8, j // 16]]
        if keys:
            np.testing.assert_allclose(o[i], v[keys].mean(axis=0), atol=1e-14)
            np.testing.assert_allclose(l[i], np.log(len(keys)), atol=1e-14)
        else:
            assert np.all(o[i] == 0) and np.isneginf(l[i])


@pytest.mark.parametrize("Br,Bc", [(16, 16), (7, 13), (64, 5)])
def test_tiled_recurrence_with_block_mask(Br, Bc):
    q, k, v = _qkv(64, 8, 805)
    mask = (np.random.default_rng(806).random((8, 4)) < 0.5).astype(np.uint8)
    mask[0, 0] = 1
    for causal in (False, True):
        o1, l1 = orc.attention_fwd_head(q, k, v, 0.4, causal, block=(mask, 8, 16))
        o2, l2 = orc.tiled_fwd_partials(q, k, v, 0.4, causal, Br, Bc, block=(mask, 8, 16))
        live = np.isfinite(l1)
        np.testing.assert_allclose(o2, o1, atol=1e-12)
        np.testing.assert_allclose(l2[live], l1[live], atol=1e-12)
        assert np.array_equal(np.isneginf(l2), ~live)


def test_block_gradients_finite_differences():
    n, d, tau = 12, 4, 0.7
    q, k, v = _qkv(n, d, 807)
    do = np.random.default_rng(808).standard_normal((n, d))
    mask = np.array([[1, 0, 1], [0, 1, 1], [0, 0, 0]], dtype=np.uint8)
    blk = (mask, 4, 4)
    for causal in (False, True):
        g = orc.attention_bwd_head(q, k, v, do, tau, causal, block=blk)
        f = lambda qq, kk, vv: float((orc.attention_fwd_head(qq, kk, vv, tau, causal, block=blk)[0]
                                      * do).sum())
        h = 1e-6
        for name, x in (("dq", q), ("dk", k), ("dv", v)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                num[idx] = (f(*[xp if x is a else a for a in (q, k, v)])
                            - f(*[xm if x is a else a for a in (q, k, v)])) / (2 * h)
            np.testing.assert_allclose(g[name], num, rtol=1e-6, atol=1e-8)
        # rows 8..11 see nothing: no gradient flows through them
        assert np.all(g["dq"][8:] == 0) and np.all(g["D"][8:] == 0)
