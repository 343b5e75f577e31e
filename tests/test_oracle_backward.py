"""Pins of the backward oracle (oracle/backward.py) against things it does not compute itself.

* Central finite differences of the forward oracle (the C implementation, itself pinned in
  test_oracle.py) of L = sum(dO * O), in float64, for entries of q, k, v and r: full causal
  with R shorter than the sequence (clamped distances share one r entry), a window, and
  more queries per KV head than one.
* Window 1: every query sees only its own key, so P = 1, dS = 0: dq = dk = dr = 0 and
  dv[j] = sum over the heads of the group of dO at the same token.
* Sums fixed by the softmax: every row of dS sums to zero, so sum_d dr[h, d] = 0; every row
  of P sums to one, so sum_j dv[j] = sum_i sum_(h in group) dO[i, h].
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


def _loss(q, k, v, r, do, window):
    out, _, _ = oracle.ref_prefill(q, k, v, r, window)
    return float((out * do).sum())


FD_CASES = [
    # seed, B, Lq, Lk, Hq, Hkv, R, window
    (1, 1, 6, 9, 2, 1, 4, 0),     # full causal, distances 4..8 share r[h, 3]
    (2, 2, 5, 5, 4, 2, 16, 3),    # window 3, two query heads per KV head
    (3, 1, 7, 7, 3, 3, 2, 0),     # one query head per KV head, R = 2
]


@pytest.mark.parametrize("seed,B,Lq,Lk,Hq,Hkv,R,window", FD_CASES)
def test_backward_matches_finite_differences(seed, B, Lq, Lk, Hq, Hkv, R, window):
    q, k, v, r, do = _case(seed, B, Lq, Lk, Hq, Hkv, R)
    dq, dk, dv, dr, _ = prefill_backward(q, k, v, r, do, window)
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


def test_backward_window_one_closed_form():
    q, k, v, r, do = _case(7, 2, 8, 8, 4, 2, 5)
    dq, dk, dv, dr, _ = prefill_backward(q, k, v, r, do, window=1)
    assert np.abs(dq).max() == 0 and np.abs(dk).max() == 0 and np.abs(dr).max() == 0
    expect = do.reshape(2, 8, 2, 2, 128).sum(axis=3)  # heads 2 hk, 2 hk + 1 -> KV head hk
    assert np.allclose(dv, expect, rtol=0, atol=1e-12)


@pytest.mark.parametrize("window", [0, 5])
def test_backward_softmax_sums(window):
    q, k, v, r, do = _case(8, 2, 12, 20, 6, 2, 7)
    dq, dk, dv, dr, dabs = prefill_backward(q, k, v, r, do, window)
    assert np.all(np.abs(dr.sum(axis=1)) <= 1e-10 * (1 + dabs.sum(axis=1)))
    expect = do.reshape(2, 12, 2, 3, 128).sum(axis=(1, 3))
    assert np.allclose(dv.sum(axis=1), expect, rtol=1e-12, atol=1e-10)
    # a bf16 input gives the same result as its exact float64 value
    from oracle.sconv import f64_to_bf16
    qb = f64_to_bf16(q)
    a = prefill_backward(qb, k, v, r, do, window)[0]
    b = prefill_backward(oracle.sconv.bf16_to_f64(qb), k, v, r, do, window)[0]
    assert np.array_equal(a, b)


@pytest.mark.parametrize("window", [0, 4])
def test_dq_rows_equal_full_call(window):
    q, k, v, r, do = _case(9, 2, 10, 15, 4, 2, 6)
    from oracle.backward import prefill_backward_dq_rows
    dq = prefill_backward(q, k, v, r, do, window)[0]
    rows = [(0, 0, 0), (1, 9, 3), (0, 5, 2), (1, 3, 1)]
    got = prefill_backward_dq_rows(q, k, v, r, do, window, rows)
    for n, (b, t, h) in enumerate(rows):
        assert np.allclose(got[n], dq[b, t, h], rtol=1e-12, atol=1e-12)
