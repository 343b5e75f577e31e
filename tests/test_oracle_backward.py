"""Pins of the two backward oracles -- oracle/backward.py (numpy, dense products per head) and
rattn_ref_cpu_backward (oracle/rattn_oracle_bwd.c, plain loops one query row at a time) --
against things they do not compute themselves.  Each pin runs on both.

* Central finite differences of the forward oracle (the C implementation, itself pinned in
  test_oracle.py) of L = sum(dO * O), in float64, for entries of q, k, v and r: full causal
  with R shorter than the sequence (clamped distances share one r entry), a window, and
  more queries per KV head than one.
* Window 1: every query sees only its own key, so P = 1, dS = 0: dq = dk = dr = 0 and
  dv[j] = sum over the heads of the group of dO at the same token.
* Sums fixed by the softmax: every row of dS sums to zero, so sum_d dr[h, d] = 0; every row
  of P sums to one, so sum_j dv[j] = sum_i sum_(h in group) dO[i, h].
* The magnitude sums (error-bound ingredients): never below the magnitude of the gradient
  they go with (triangle inequality), equal to the gradient itself when every term is
  non-negative in the dv sum (dO >= 0), and the same from both implementations.
"""
import numpy as np
import pytest

import oracle
from oracle.backward import prefill_backward


def _case(seed, B, Lq, Lk, Hq, Hkv, R, D=128):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Lq, Hq, D))
    k = rng.standard_normal((B, Lk, Hkv, D))
    v = rng.standard_normal((B, Lk, Hkv, D))
    r = rng.standard_normal((Hq, R)) * 0.7
    do = rng.standard_normal((B, Lq, Hq, D))
    return q, k, v, r, do


def _numpy_bwd(q, k, v, r, do, window):
    dq, dk, dv, dr, absums = prefill_backward(q, k, v, r, do, window)
    return (dq, dk, dv, dr), absums


def _c_bwd(q, k, v, r, do, window):
    return oracle.ref_backward(q, k, v, r, do, window)


IMPLS = {"numpy": _numpy_bwd, "c": _c_bwd}


def _loss(q, k, v, r, do, window):
    out, _, _ = oracle.ref_prefill(q, k, v, r, window)
    return float((out * do).sum())


FD_CASES = [
    # seed, B, Lq, Lk, Hq, Hkv, R, window
    (1, 1, 6, 9, 2, 1, 4, 0),     # full causal, distances 4..8 share r[h, 3]
    (2, 2, 5, 5, 4, 2, 16, 3),    # window 3, two query heads per KV head
    (3, 1, 7, 7, 3, 3, 2, 0),     # one query head per KV head, R = 2
]


@pytest.mark.parametrize("impl", sorted(IMPLS))
@pytest.mark.parametrize("seed,B,Lq,Lk,Hq,Hkv,R,window", FD_CASES)
def test_backward_matches_finite_differences(impl, seed, B, Lq, Lk, Hq, Hkv, R, window):
    q, k, v, r, do = _case(seed, B, Lq, Lk, Hq, Hkv, R)
    (dq, dk, dv, dr), _ = IMPLS[impl](q, k, v, r, do, window)
    rng = np.random.default_rng(100 + seed)
    eps = 1e-5
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv), ("r", r, dr)):
        flat = x.reshape(-1)
        gflat = g.reshape(-1)
        picks = rng.choice(flat.size, size=min(12, flat.size), replace=False)
        if name == "r":
            picks = np.arange(flat.size)  # every entry, the clamped one included
        for idx in picks:
            keep = flat[idx]
            flat[idx] = keep + eps
            lp = _loss(q, k, v, r, do, window)
            flat[idx] = keep - eps
            lm = _loss(q, k, v, r, do, window)
            flat[idx] = keep
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - gflat[idx]) <= 1e-6 * (1 + abs(fd)), (name, idx, fd, gflat[idx])


@pytest.mark.parametrize("impl", sorted(IMPLS))
def test_backward_window_one_closed_form(impl):
    q, k, v, r, do = _case(7, 2, 8, 8, 4, 2, 5)
    (dq, dk, dv, dr), _ = IMPLS[impl](q, k, v, r, do, 1)
    assert np.abs(dq).max() == 0 and np.abs(dk).max() == 0 and np.abs(dr).max() == 0
    expect = do.reshape(2, 8, 2, 2, 128).sum(axis=3)  # heads 2 hk, 2 hk + 1 -> KV head hk
    assert np.allclose(dv, expect, rtol=0, atol=1e-12)


@pytest.mark.parametrize("impl", sorted(IMPLS))
@pytest.mark.parametrize("window", [0, 5])
def test_backward_softmax_sums(impl, window):
    q, k, v, r, do = _case(8, 2, 12, 20, 6, 2, 7)
    (dq, dk, dv, dr), absums = IMPLS[impl](q, k, v, r, do, window)
    assert np.all(np.abs(dr.sum(axis=1)) <= 1e-10 * (1 + absums[3].sum(axis=1)))
    expect = do.reshape(2, 12, 2, 3, 128).sum(axis=(1, 3))
    assert np.allclose(dv.sum(axis=1), expect, rtol=1e-12, atol=1e-10)
    # a bf16 input gives the same result as its exact float64 value
    from oracle.sconv import bf16_to_f64, f64_to_bf16
    qb, kb, vb, gb = (f64_to_bf16(x) for x in (q, k, v, do))
    a = IMPLS[impl](qb, kb, vb, r, gb, window)[0]
    b = IMPLS[impl](*(bf16_to_f64(x) for x in (qb, kb, vb)), r, bf16_to_f64(gb), window)[0]
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("window", [0, 4])
def test_dq_rows_equal_full_call(window):
    q, k, v, r, do = _case(9, 2, 10, 15, 4, 2, 6)
    from oracle.backward import prefill_backward_dq_rows
    dq = prefill_backward(q, k, v, r, do, window)[0]
    rows = [(0, 0, 0), (1, 9, 3), (0, 5, 2), (1, 3, 1)]
    got = prefill_backward_dq_rows(q, k, v, r, do, window, rows)
    for n, (b, t, h) in enumerate(rows):
        assert np.allclose(got[n], dq[b, t, h], rtol=1e-12, atol=1e-12)


ABS_CASES = [
    # seed, B, Lq, Lk, Hq, Hkv, R, window
    (11, 1, 20, 20, 4, 2, 8, 0),
    (12, 2, 13, 30, 6, 2, 40, 7),
    (13, 1, 9, 9, 3, 1, 3, 1),
]


@pytest.mark.parametrize("seed,B,Lq,Lk,Hq,Hkv,R,window", ABS_CASES)
def test_backward_implementations_agree(seed, B, Lq, Lk, Hq, Hkv, R, window):
    """The dense numpy form and the row-by-row C form compute the same gradients and
    magnitude sums (summation orders differ: agreement to rounding)."""
    q, k, v, r, do = _case(seed, B, Lq, Lk, Hq, Hkv, R)
    ga, aa = _numpy_bwd(q, k, v, r, do, window)
    gb, ab = _c_bwd(q, k, v, r, do, window)
    for name, x, y, scale in zip(("dq", "dk", "dv", "dr"), ga, gb, aa):
        assert np.all(np.abs(x - y) <= 1e-12 * (1 + scale)), name
    for name, x, y in zip(("dq_abs", "dk_abs", "dv_abs", "dr_abs"), aa, ab):
        assert np.allclose(x, y, rtol=1e-12, atol=1e-14), name


@pytest.mark.parametrize("impl", sorted(IMPLS))
@pytest.mark.parametrize("seed,B,Lq,Lk,Hq,Hkv,R,window", ABS_CASES)
def test_backward_magnitude_sums(impl, seed, B, Lq, Lk, Hq, Hkv, R, window):
    q, k, v, r, do = _case(seed, B, Lq, Lk, Hq, Hkv, R)
    grads, absums = IMPLS[impl](q, k, v, r, do, window)
    # triangle inequality: a sum is never larger than the sum of its terms' magnitudes
    for name, g, a in zip(("dq", "dk", "dv", "dr"), grads, absums):
        assert np.all(a >= np.abs(g) * (1 - 1e-12)), name
    # with dO >= 0 every term of dv = P^T dO is non-negative: its magnitude sum is itself
    grads, absums = IMPLS[impl](q, k, v, r, np.abs(do), window)
    assert np.allclose(absums[2], grads[2], rtol=1e-12, atol=0)
    # keys that no query sees get nothing
    if Lk > Lq and window > 0:
        first_seen = (Lk - Lq) - window + 1
        if first_seen > 0:
            for a in absums[1:3]:
                assert np.all(a[:, :first_seen] == 0)


@pytest.mark.parametrize("seed,B,Lq,Lk,Hq,Hkv,R,window", ABS_CASES)
def test_backward_given_output(seed, B, Lq, Lk, Hq, Hkv, R, window):
    """D from a given forward output: with the exact output (the forward oracle's, float64)
    both implementations reproduce the exact gradients; with that output rounded to bf16 they
    agree with each other (gradients and magnitude sums, any weight)."""
    from oracle.sconv import f64_to_bf16
    q, k, v, r, do = _case(seed, B, Lq, Lk, Hq, Hkv, R)
    out, _, _ = oracle.ref_prefill(q, k, v, r, window)
    exact, _ = _c_bwd(q, k, v, r, do, window)
    for impl in ("numpy", "c"):
        if impl == "numpy":
            got = prefill_backward(q, k, v, r, do, window, out=out)[:4]
        else:
            got = oracle.ref_backward(q, k, v, r, do, window, out=out)[0]
        for name, x, y in zip(("dq", "dk", "dv", "dr"), got, exact):
            assert np.allclose(x, y, rtol=1e-10, atol=1e-12), (impl, name)
    qb, kb, vb, gb, ob = (f64_to_bf16(x) for x in (q, k, v, do, out))
    w = 2.0 ** -6
    res_np = prefill_backward(qb, kb, vb, r, gb, window, out=ob, abs_weight=w)
    g_np, a_np = res_np[:4], res_np[4]
    g_c, a_c = oracle.ref_backward(qb, kb, vb, r, gb, window, out=ob, abs_weight=w)
    for name, x, y, scale in zip(("dq", "dk", "dv", "dr"), g_np, g_c, a_np):
        assert np.all(np.abs(x - y) <= 1e-12 * (1 + scale)), name
    for name, x, y in zip(("dq_abs", "dk_abs", "dv_abs", "dr_abs"), a_np, a_c):
        assert np.allclose(x, y, rtol=1e-12, atol=1e-14), name
    # the D term of the magnitude sums scales with the weight
    a_1 = oracle.ref_backward(qb, kb, vb, r, gb, window, out=ob, abs_weight=1.0)[1]
    a_0 = oracle.ref_backward(qb, kb, vb, r, gb, window, out=ob, abs_weight=0.0)[1]
    for x0, xw, x1 in zip(a_0, a_c, a_1):
        assert np.allclose(xw, x0 + w * (x1 - x0), rtol=1e-12, atol=1e-12)
