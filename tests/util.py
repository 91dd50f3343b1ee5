"""Helpers for the parity tests: upload seeded host tensors and compare to the oracle."""
import numpy as np

# Tolerances on |GPU - oracle| (absolute), per output and input dtype.
TOL = {
    "bf16": {"max": 2e-2, "mean": 2e-3, "lse": 1e-3},
    "f32": {"max": 1e-5, "mean": 1e-5, "lse": 1e-5},
}


def to_device(ht, device="cuda"):
    """HostTensor -> torch tensor on the GPU holding exactly the same bits."""
    import torch
    if ht.dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(ht.raw).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(ht.raw))
    return t.to(device)


def to_f64(t):
    """GPU tensor -> float64 numpy array (exact widening)."""
    import torch
    return t.detach().to("cpu", torch.float64).numpy()


def err_stats(got, ref):
    d = np.abs(np.asarray(got, dtype=np.float64) - np.asarray(ref, dtype=np.float64))
    return float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0


def bf16_ulp(x):
    """One bf16 unit in the last place at |x| (2^(e-7) for |x| in [2^e, 2^(e+1)))."""
    ax = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), np.finfo(np.float32).tiny)
    return np.exp2(np.floor(np.log2(ax)) - 7)


# Max and mean |GPU - oracle| of the outputs compared at each workload's full
# size, collected over the test session; conftest writes them out when
# FA_PARITY_LOG names a file.
RECORDS = []


def record(config, output, got, ref):
    """Keeps the error of one compared output for the session's error table."""
    d = np.abs(np.asarray(got, dtype=np.float64) - np.asarray(ref, dtype=np.float64))
    if d.size:
        RECORDS.append({"config": config, "output": output, "max_abs": float(d.max()),
                        "sum_abs": float(d.sum()), "n": int(d.size)})


def assert_close(got, ref, dtype, what, kind="out", ulp_allow=False, extra=None, tag=None):
    """|got - ref| within TOL.  ulp_allow (bf16 outputs only) adds one bf16 unit
    of the reference value to the max bound per element: an output stored in
    bf16 can be off by that much through its own rounding, which exceeds the
    absolute bound once |ref| > 5.12 (outputs of that size arise when a small
    attention window concentrates the probabilities).  extra: a further
    per-element allowance (array like ref) derived from the arithmetic."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "%s: non-finite values" % what
    if tag is not None:
        record(tag[0], tag[1], got, ref)
    mx, mean = err_stats(got, ref)
    tol = TOL[dtype]
    if kind == "lse":
        assert mx <= tol["lse"], "%s: max |err| %.3g > %.3g" % (what, mx, tol["lse"])
    else:
        if (ulp_allow and dtype == "bf16") or extra is not None:
            allow = tol["max"] + (bf16_ulp(ref) if ulp_allow else 0.0)
            excess = np.abs(got - ref) - (allow + (0.0 if extra is None else extra))
            assert excess.max() <= 0, "%s: max |err| %.3g beyond its bound by %.3g (mean %.3g)" % (
                what, mx, excess.max(), mean)
        else:
            assert mx <= tol["max"], "%s: max |err| %.3g > %.3g (mean %.3g)" % (what, mx, tol["max"], mean)
        assert mean <= tol["mean"], "%s: mean |err| %.3g > %.3g" % (what, mean, tol["mean"])
    return mx, mean


def rounding_allowance(g, q, k, do, tau):
    """Per-element error allowance of one head's gradients for the bf16
    operands the kernels feed to their MFMA products: P (dropped, if dropout)
    and dS are rounded to bfloat16 (relative error <= 2^-9 each, round to
    nearest) before dV = (P o Z)^T dO, dK = tau dS^T Q and dQ = tau dS K, so an
    output can be off by 2^-9 times the sum of the magnitudes of its terms.
    The stated absolute bound assumes those sums are of order one; with a few
    visible keys per row (small windows, short causal rows under dropout) they
    are not.  g: the oracle's attention_bwd_head result."""
    u = 2.0 ** -9
    return {"dv": u * (np.abs(g["pz"]).T @ np.abs(do)),
            "dk": u * tau * (np.abs(g["ds"]).T @ np.abs(q)),
            "dq": u * tau * (np.abs(g["ds"]) @ np.abs(k))}


def saved_o_allowance(g, o_gpu, q, k, do, tau):
    """Per-element allowance on dQ and dK for the D the kernels form.

    The backward takes D_i = dO_i . O_i from the O its forward stored (bf16),
    not from the exact O, so D_gpu - D = dO_i . (O_gpu_i - O_i) plus the
    float32 rounding of that length-d sum of exact bf16 products:
        |dD_i| <= sum_c |dO_ic| |O_gpu_ic - O_ic| + 2^-17 sum_c |dO_ic| |O_gpu_ic|.
    dS_ij = P_ij (dP_ij - D_i) (dropout: P_ij (Z_ij dP_ij - D_i)) then moves by
    -P_ij dD_i, so
        |d dQ_ic| <= tau |dD_i| sum_j P_ij |K_jc|,
        |d dK_jc| <= tau sum_i P_ij |dD_i| |Q_ic|,
    and dV does not depend on D.  P is the undropped softmax of the exact
    scores.  g: the oracle's attention_bwd_head result; o_gpu: the forward's
    output for the same head (float64 view of what the kernel stored)."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    do = np.abs(np.asarray(do, dtype=np.float64))
    dD = (do * np.abs(o_gpu - g["o"])).sum(axis=1) + 2.0 ** -17 * (do * np.abs(o_gpu)).sum(axis=1)
    p = g["p"]
    return {"dq": tau * dD[:, None] * (p @ np.abs(k)),
            "dk": tau * (p.T @ (dD[:, None] * np.abs(q))),
            "dv": np.zeros_like(o_gpu)}


def bwd_allowance(g, o_gpu, q, k, do, tau):
    """rounding_allowance + saved_o_allowance, per output."""
    a = rounding_allowance(g, q, k, do, tau)
    b = saved_o_allowance(g, o_gpu, q, k, do, tau)
    return {n: a[n] + b[n] for n in a}
