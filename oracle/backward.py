"""fp64 CPU oracle for the backward pass of relative-bias grouped-query attention.

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the test suite and the benchmark use it.  It
shares nothing with the HIP library.

The forward pass is the one of the vLLM recipes page "thinkingmachines/Inkling", Overview >
Architectural highlights > Attention (GQA, head size 128, no RoPE: a trained bias that
depends on the query-key distance enters the logits before the softmax), with the term read as r[h, min(i - j, R - 1)]:

    s[i, j] = q_i . k_j / sqrt(D) + r[h, min(p_i - j, R - 1)]   over the visible keys j,
    P = softmax_j(s),  O = P V,

where query i of a prefill with Lk keys sits at p_i = Lk - Lq + i and key j is visible iff
0 <= p_i - j (and p_i - j <= W - 1 for a window W > 0).  The page lists training and LoRA
among what the model is used for; the backward pass is the plain chain rule of that
definition for a loss whose gradient with respect to O is dO:

    dP = dO V^T,  dS = P * (dP - rowsum(P * dP)),
    dQ = dS K / sqrt(D),  dK = dS^T Q / sqrt(D),  dV = P^T dO,
    dr[h, d] = sum of dS[i, j] over the visible (i, j) with min(p_i - j, R - 1) = d,

with dK and dV summed over the query heads that share a KV head.  Every step is a dense
matrix product or an elementwise operation in float64, one (sequence, head) at a time.
"""
from __future__ import annotations

import numpy as np

from .sconv import bf16_to_f64


def _f64(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a)
    return bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def prefill_backward(q, k, v, bias, dout, window: int = 0, out=None, abs_weight: float = 1.0):
    """Gradients of a prefill (every sequence has Lk keys; query t at Lk - Lq + t).

    q [B, Lq, Hq, D], k and v [B, Lk, Hkv, D], dout [B, Lq, Hq, D]: uint16 (bf16 bits),
    float32 or float64; bias [Hq, R].  Returns float64 arrays
    (dq [B, Lq, Hq, D], dk [B, Lk, Hkv, D], dv [B, Lk, Hkv, D], dbias [Hq, R], absums) with
    absums = (dq_abs, dk_abs, dv_abs, dbias_abs): the same sums with every term taken by
    absolute value and dS replaced by dS_abs = P * (|dP - D| + w (A + D_abs)), where
    A = |dO| |V|^T holds the sizes of dP's terms, D_abs = rowsum(P * A) the size of D's
    terms and w = abs_weight.  They bound an implementation's rounding errors element by
    element (the gradients are sums whose terms cancel).
    out: None, or a forward output like q: then D = rowsum(dO * out) (the row sum a
    backward implementation takes from the forward's rounded output), D_abs =
    rowsum(|dO * out|)."""
    Q, K, V, dO = _f64(q), _f64(k), _f64(v), _f64(dout)
    O = None if out is None else _f64(out)
    r = np.asarray(bias, dtype=np.float64)
    B, Lq, Hq, D = Q.shape
    Lk, Hkv = K.shape[1], K.shape[2]
    G = Hq // Hkv
    R = r.shape[1]
    scale = 1.0 / np.sqrt(D)
    p = (Lk - Lq) + np.arange(Lq)[:, None]
    dist = p - np.arange(Lk)[None, :]
    vis = dist >= 0
    if window > 0:
        vis &= dist <= window - 1
    didx = np.minimum(np.maximum(dist, 0), R - 1)
    dq = np.zeros_like(Q)
    dk = np.zeros_like(K)
    dv = np.zeros_like(V)
    dbias = np.zeros((Hq, R))
    dq_abs = np.zeros_like(Q)
    dk_abs = np.zeros_like(K)
    dv_abs = np.zeros_like(V)
    dbias_abs = np.zeros((Hq, R))
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            s = Q[b, :, h] @ K[b, :, hk].T * scale + r[h][didx]
            s = np.where(vis, s, -np.inf)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            P = e / e.sum(axis=1, keepdims=True)
            dP = dO[b, :, h] @ V[b, :, hk].T
            A = np.abs(dO[b, :, h]) @ np.abs(V[b, :, hk]).T
            if O is None:
                Drow = (P * dP).sum(axis=1, keepdims=True)
                Dabs = (P * A).sum(axis=1, keepdims=True)
            else:
                Drow = (dO[b, :, h] * O[b, :, h]).sum(axis=1, keepdims=True)
                Dabs = np.abs(dO[b, :, h] * O[b, :, h]).sum(axis=1, keepdims=True)
            dS = P * (dP - Drow)
            dq[b, :, h] = dS @ K[b, :, hk] * scale
            dk[b, :, hk] += dS.T @ Q[b, :, h] * scale
            dv[b, :, hk] += P.T @ dO[b, :, h]
            dbias[h] += np.bincount(didx[vis], weights=dS[vis], minlength=R)
            # magnitude sums
            dSa = P * (np.abs(dP - Drow) + abs_weight * (A + Dabs))
            dq_abs[b, :, h] = dSa @ np.abs(K[b, :, hk]) * scale
            dk_abs[b, :, hk] += dSa.T @ np.abs(Q[b, :, h]) * scale
            dv_abs[b, :, hk] += P.T @ np.abs(dO[b, :, h])
            dbias_abs[h] += np.bincount(didx[vis], weights=dSa[vis], minlength=R)
    return dq, dk, dv, dbias, (dq_abs, dk_abs, dv_abs, dbias_abs)


def prefill_backward_dq_rows(q, k, v, bias, dout, window: int, rows):
    """dq for selected query rows [(b, t, h), ...] of a prefill, each from its own row of the
    definition: the row's visible logits, P, dP = dO_t V^T, D = sum(P * dP), dS, dq = dS K /
    sqrt(D).  Returns float64 [n, D].  Same inputs and reading as prefill_backward."""
    Lq = np.asarray(q).shape[1]
    Lk, Hkv = np.asarray(k).shape[1], np.asarray(k).shape[2]
    Hq, R = np.asarray(q).shape[2], np.asarray(bias).shape[1]
    G = Hq // Hkv
    D = np.asarray(q).shape[3]
    r = np.asarray(bias, dtype=np.float64)
    out = []
    for (b, t, h) in rows:
        p = (Lk - Lq) + t
        lo = max(0, p - window + 1) if window > 0 else 0
        js = np.arange(lo, p + 1)
        Kb = _f64(np.asarray(k)[b, lo:p + 1, h // G])
        Vb = _f64(np.asarray(v)[b, lo:p + 1, h // G])
        qi = _f64(np.asarray(q)[b, t, h])
        gi = _f64(np.asarray(dout)[b, t, h])
        s = Kb @ qi / np.sqrt(D) + r[h][np.minimum(p - js, R - 1)]
        e = np.exp(s - s.max())
        P = e / e.sum()
        dP = Vb @ gi
        dS = P * (dP - (P * dP).sum())
        out.append(dS @ Kb / np.sqrt(D))
    return np.stack(out) if out else np.zeros((0, D))
