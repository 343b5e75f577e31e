"""Checks that pin the CPU oracle to facts it does not itself define.

Each pin takes an oracle build (``lib``; None = the normal one) and raises
AssertionError when the oracle disagrees with:
  * a library special case (torch scaled-dot-product attention in float64 with an
    explicit bottom-right mask, for zero bias; ALiBi, a published linear
    relative bias, through the same routine with a float mask),
  * hand-derived worked examples (tests/golden/hand_examples.json),
  * closed forms (window 1, position 0, R = 1, K = 0, constant V),
  * invariants (per-head bias shift, window >= L, chunk == full, paged ==
    contiguous, decode == last prefill rows, probabilities sum to 1),
  * brute force over tiny inputs with pure-Python loops,
and the token-dependent variant (one table per query row) to the static one
(equal rows), SDPA with a per-row float mask, closed forms, a per-row shift,
row independence and brute force.
The definition being pinned is the one on the vLLM recipes page
"thinkingmachines/Inkling", Overview > Architectural highlights > Attention:
GQA with head size 128 whose logits carry a trained, distance-dependent bias
in place of RoPE, with the term fixed as r[h, min(i-j, R-1)].

tests/test_oracle.py runs every pin on the real oracle; tests/test_oracle_mutants.py
runs them on deliberately broken copies and requires each copy to fail one.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_examples.json")


def _ref(lib, q, k, v, bias, ctx, windows=None, block_table=None, block_size=128, probs=False, Lk_max=None):
    return oracle.ref_attention(q, k, v, bias, ctx, windows, block_table, block_size, want_probs=probs,
                                lib=lib, Lk_max=Lk_max)


def _prefill(lib, q, k, v, bias, window=0, probs=False):
    B = q.shape[0]
    return _ref(lib, q, k, v, bias, [k.shape[1]] * B, [window] * B, probs=probs)


def _rand(seed, B, Lq, Lk, Hq, Hkv, D, R, scale_bias=0.5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Lq, Hq, D))
    k = rng.standard_normal((B, Lk, Hkv, D))
    v = rng.standard_normal((B, Lk, Hkv, D))
    r = scale_bias * rng.standard_normal((Hq, R))
    return q, k, v, r


# ----------------------------------------------------------------------------
# library special cases
# ----------------------------------------------------------------------------
def _sdpa(q, k, v, float_mask, scale):
    """torch SDPA, float64 CPU.  q [B,Lq,Hq,D], k/v [B,Lk,Hkv,D] already expanded
    to Hq heads by the caller; float_mask [B or 1, Hq or 1, Lq, Lk] additive."""
    import torch
    import torch.nn.functional as F
    tq = torch.from_numpy(np.ascontiguousarray(q.transpose(0, 2, 1, 3)))
    tk = torch.from_numpy(np.ascontiguousarray(k.transpose(0, 2, 1, 3)))
    tv = torch.from_numpy(np.ascontiguousarray(v.transpose(0, 2, 1, 3)))
    tm = torch.from_numpy(np.ascontiguousarray(float_mask))
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=tm, scale=scale)
    return o.numpy().transpose(0, 2, 1, 3)


def _expand_kv(x, G):
    # contiguous groups, the torch repeat_interleave convention
    return np.repeat(x, G, axis=2)


def _visibility(Lq, Lk, window):
    """Bottom-right aligned causal (and window) visibility as a boolean [Lq, Lk]."""
    i = np.arange(Lq)[:, None] + (Lk - Lq)
    j = np.arange(Lk)[None, :]
    vis = j <= i
    if window > 0:
        vis &= (i - j) < window
    return vis


def pin_zero_bias_is_sdpa(lib):
    """r = 0 reduces to ordinary (bottom-right causal / windowed) GQA attention."""
    for (B, Lq, Lk, Hq, Hkv, window) in [(2, 9, 9, 4, 2, 0), (1, 5, 13, 6, 3, 0), (1, 13, 13, 4, 1, 5),
                                         (2, 7, 20, 8, 2, 6), (1, 1, 17, 2, 2, 0)]:
        D = 16
        q, k, v, _ = _rand(11 + Lq + Lk, B, Lq, Lk, Hq, Hkv, D, 4)
        r = np.zeros((Hq, 4))
        out, _, _ = _prefill(lib, q, k, v, r, window)
        vis = _visibility(Lq, Lk, window)
        mask = np.where(vis, 0.0, -np.inf)[None, None]
        G = Hq // Hkv
        ref = _sdpa(q, _expand_kv(k, G), _expand_kv(v, G), mask, 1.0 / math.sqrt(D))
        np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def pin_alibi_is_sdpa(lib):
    """A linear table r[h, d] = -m_h * d (R larger than every distance) is ALiBi
    (Press et al., 'Train Short, Test Long'): a penalty proportional to the
    query-key distance, with head-specific slopes m_h = 2^(-8h/H)."""
    B, L, Hq, Hkv, D = 1, 12, 4, 2, 8
    q, k, v, _ = _rand(5, B, L, L, Hq, Hkv, D, 1)
    slopes = np.array([2.0 ** (-8.0 * (h + 1) / Hq) for h in range(Hq)])
    R = L + 3
    r = -slopes[:, None] * np.arange(R)[None, :]
    out, lse, _ = _prefill(lib, q, k, v, r, 0)
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    penalty = -slopes[:, None, None] * (i - j)[None]          # ALiBi: -m * distance
    mask = np.where((j <= i)[None], penalty, -np.inf)[None]
    G = Hq // Hkv
    ref = _sdpa(q, _expand_kv(k, G), _expand_kv(v, G), mask, 1.0 / math.sqrt(D))
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# hand-derived examples
# ----------------------------------------------------------------------------
def _val(s: str) -> float:
    s = s.strip()
    if s.startswith("ln(") and s.endswith(")"):
        return math.log(float(Fraction(s[3:-1])))
    return float(Fraction(s))


def _arr(x):
    if isinstance(x, list):
        return np.array([_arr(e) for e in x], dtype=np.float64)
    return _val(x)


def pin_golden_examples(lib):
    with open(GOLDEN) as f:
        g = json.load(f)
    for c in g["cases"]:
        q, k, v, r = _arr(c["q"]), _arr(c["k"]), _arr(c["v"]), _arr(c["bias"])
        out, lse, _ = _prefill(lib, q, k, v, r, c["window"])
        np.testing.assert_allclose(out, _arr(c["out"]), rtol=0, atol=1e-12, err_msg=c["name"])
        np.testing.assert_allclose(lse, _arr(c["lse"]), rtol=0, atol=1e-12, err_msg=c["name"])
    for c in g["paged_cases"]:
        q, kc, vc, r = _arr(c["q"]), _arr(c["k_cache"]), _arr(c["v_cache"]), _arr(c["bias"])
        bt = np.array(c["block_table"], dtype=np.int32)
        out, lse, _ = _ref(lib, q, kc, vc, r, [c["ctx"]], [c["window"]], bt, c["block_size"])
        np.testing.assert_allclose(out, _arr(c["out"]), rtol=0, atol=1e-12, err_msg=c["name"])
        np.testing.assert_allclose(lse, _arr(c["lse"]), rtol=0, atol=1e-12, err_msg=c["name"])


# ----------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------
def pin_window_one(lib):
    """W = 1: each query sees only itself: out_i = v_i, lse_i = q_i.k_i/sqrt(D) + r[h, 0]."""
    B, L, Hq, Hkv, D, R = 2, 10, 4, 2, 8, 5
    q, k, v, r = _rand(2, B, L, L, Hq, Hkv, D, R)
    out, lse, _ = _prefill(lib, q, k, v, r, 1)
    G = Hq // Hkv
    for h in range(Hq):
        kv = h // G
        np.testing.assert_allclose(out[:, :, h], v[:, :, kv], rtol=0, atol=1e-12)
        dots = np.einsum("bld,bld->bl", q[:, :, h], k[:, :, kv])
        np.testing.assert_allclose(lse[:, :, h], dots / math.sqrt(D) + r[h, 0], rtol=0, atol=1e-12)


def pin_position_zero(lib):
    """The first query of a fresh prefill (position 0) sees only key 0."""
    B, L, Hq, Hkv, D, R = 1, 6, 2, 1, 8, 4
    q, k, v, r = _rand(3, B, L, L, Hq, Hkv, D, R)
    out, lse, _ = _prefill(lib, q, k, v, r, 0)
    for h in range(Hq):
        np.testing.assert_allclose(out[0, 0, h], v[0, 0, 0], rtol=0, atol=1e-12)
        assert abs(lse[0, 0, h] - (q[0, 0, h] @ k[0, 0, 0] / math.sqrt(D) + r[h, 0])) < 1e-12


def pin_R_one(lib):
    """R = 1: every distance clamps to r[h, 0], a per-head constant: standard
    attention with lse shifted by r[h, 0]."""
    B, L, Hq, Hkv, D = 1, 11, 4, 2, 8
    q, k, v, _ = _rand(4, B, L, L, Hq, Hkv, D, 1)
    r = np.array([[0.3], [-1.1], [2.0], [0.0]])
    out, lse, _ = _prefill(lib, q, k, v, r, 0)
    out0, lse0, _ = _prefill(lib, q, k, v, np.zeros((Hq, 1)), 0)
    np.testing.assert_allclose(out, out0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse0 + r[:, 0][None, None, :], rtol=0, atol=1e-12)
    vis = _visibility(L, L, 0)
    G = Hq // Hkv
    ref = _sdpa(q, _expand_kv(k, G), _expand_kv(v, G), np.where(vis, 0.0, -np.inf)[None, None], 1 / math.sqrt(D))
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def pin_zero_keys(lib):
    """K = 0: the weights are the softmax of the bias entries alone, whatever Q is."""
    B, L, Hq, Hkv, D, R = 1, 9, 2, 1, 8, 6
    q, _, v, r = _rand(6, B, L, L, Hq, Hkv, D, R)
    k = np.zeros((B, L, Hkv, D))
    _, lse, probs = _prefill(lib, q, k, v, r, 0, probs=True)
    _, _, probs2 = _prefill(lib, 7.0 * q[:, ::-1].copy(), k, v, r, 0, probs=True)
    np.testing.assert_allclose(probs, probs2, rtol=0, atol=1e-14)
    for i in range(L):
        for h in range(Hq):
            b = np.array([r[h, min(i - j, R - 1)] for j in range(i + 1)])
            w = np.exp(b - b.max())
            np.testing.assert_allclose(probs[0, i, h, :i + 1], w / w.sum(), rtol=0, atol=1e-13)
            assert abs(lse[0, i, h] - (b.max() + math.log(w.sum()))) < 1e-12


def pin_constant_values(lib):
    """Convexity: if every V row is the same vector c, out = c."""
    B, L, Hq, Hkv, D, R = 1, 8, 4, 2, 8, 3
    q, k, _, r = _rand(7, B, L, L, Hq, Hkv, D, R)
    c = np.linspace(-2, 3, D)
    v = np.broadcast_to(c, (B, L, Hkv, D)).copy()
    for window in (0, 3):
        out, _, _ = _prefill(lib, q, k, v, r, window)
        np.testing.assert_allclose(out, np.broadcast_to(c, out.shape), rtol=0, atol=1e-13)


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------
def pin_bias_shift(lib):
    """Adding c_h to every entry of r[h, :] leaves out unchanged and adds c_h to lse."""
    B, Lq, Lk, Hq, Hkv, D, R = 1, 6, 10, 4, 2, 8, 7
    q, k, v, r = _rand(8, B, Lq, Lk, Hq, Hkv, D, R)
    c = np.array([1.5, -2.25, 0.0, 4.0])
    for window in (0, 4):
        out, lse, _ = _prefill(lib, q, k, v, r, window)
        out2, lse2, _ = _prefill(lib, q, k, v, r + c[:, None], window)
        np.testing.assert_allclose(out2, out, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse2, lse + c[None, None, :], rtol=0, atol=1e-12)


def pin_wide_window_is_full(lib):
    """A window at least as long as the sequence equals full attention, exactly."""
    B, L, Hq, Hkv, D, R = 1, 9, 2, 2, 8, 5
    q, k, v, r = _rand(9, B, L, L, Hq, Hkv, D, R)
    out0, lse0, _ = _prefill(lib, q, k, v, r, 0)
    for W in (L, L + 1, 1000):
        out, lse, _ = _prefill(lib, q, k, v, r, W)
        assert np.array_equal(out, out0) and np.array_equal(lse, lse0)
    out, _, _ = _prefill(lib, q, k, v, r, L - 1)
    assert not np.allclose(out, out0)


def pin_probs_sum_to_one(lib):
    B, Lq, Lk, Hq, Hkv, D, R = 2, 5, 12, 4, 1, 8, 6
    q, k, v, r = _rand(10, B, Lq, Lk, Hq, Hkv, D, R)
    for window in (0, 3):
        out, _, probs = _prefill(lib, q, k, v, r, window, probs=True)
        np.testing.assert_allclose(probs.sum(-1), 1.0, rtol=0, atol=1e-12)
        # out is the probability-weighted sum of V rows, and only visible keys get weight
        G = Hq // Hkv
        ref = np.einsum("bthj,bjhd->bthd", probs, _expand_kv(v, G))
        np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
        vis = _visibility(Lq, Lk, window)
        for t in range(Lq):
            assert np.all(probs[:, t, :, ~vis[t]] == 0)


def pin_chunk_equals_full(lib):
    """Rows of a chunk (Lq < Lk) equal the same rows of the full-length prefill."""
    B, L, Hq, Hkv, D, R = 1, 14, 4, 2, 8, 6
    q, k, v, r = _rand(12, B, L, L, Hq, Hkv, D, R)
    for window in (0, 5):
        out, lse, _ = _prefill(lib, q, k, v, r, window)
        for Lq in (1, 4, 9):
            o2, l2, _ = _prefill(lib, q[:, L - Lq:], k, v, r, window)
            np.testing.assert_allclose(o2, out[:, L - Lq:], rtol=0, atol=1e-13)
            np.testing.assert_allclose(l2, lse[:, L - Lq:], rtol=0, atol=1e-13)


def pin_paged_equals_contiguous(lib):
    """A paged cache behind a permuted block table gives the contiguous result, and a
    decode of n_q queries equals the last n_q rows of the prefill."""
    rng = np.random.default_rng(13)
    Hq, Hkv, D, R, bs = 4, 2, 8, 9, 4
    ctx = np.array([13, 6, 16], dtype=np.int32)
    windows = np.array([0, 0, 5], dtype=np.int32)
    n_q = 3
    B = len(ctx)
    Lk = int(ctx.max())
    q = rng.standard_normal((B, n_q, Hq, D))
    k = rng.standard_normal((B, Lk, Hkv, D))
    v = rng.standard_normal((B, Lk, Hkv, D))
    r = 0.5 * rng.standard_normal((Hq, R))
    mb = (Lk + bs - 1) // bs
    perm = rng.permutation(B * mb)
    bt = perm.reshape(B, mb).astype(np.int32)
    kc = np.full((B * mb, bs, Hkv, D), np.nan)
    vc = np.full((B * mb, bs, Hkv, D), np.nan)
    for b in range(B):
        for j in range(int(ctx[b])):
            kc[bt[b, j // bs], j % bs] = k[b, j]
            vc[bt[b, j // bs], j % bs] = v[b, j]
    out, lse, _ = _ref(lib, q, kc, vc, r, ctx, windows, bt, bs)
    for b in range(B):
        c = int(ctx[b])
        qq = np.zeros((1, c, Hq, D))
        qq[0, c - n_q:] = q[b]
        o2, l2, _ = _prefill(lib, qq, k[b:b + 1, :c], v[b:b + 1, :c], r, int(windows[b]))
        np.testing.assert_allclose(out[b], o2[0, c - n_q:], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[b], l2[0, c - n_q:], rtol=0, atol=1e-13)


def pin_input_widening(lib):
    """bf16 bit patterns and fp32 inputs widen exactly: the same values given as
    float64 give bitwise the same result."""
    from relative_bias_gqa_amd import synth
    c = synth.make_prefill(21, 1, 6, 9, 4, 2, 5, 0, "bf16")
    out, lse, _ = _prefill(lib, c.q, c.k, c.v, c.bias, 0)
    f = lambda a: synth.to_float(a).astype(np.float64)
    out2, lse2, _ = _prefill(lib, f(c.q), f(c.k), f(c.v), c.bias, 0)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    c32 = synth.make_prefill(22, 1, 6, 9, 4, 2, 5, 3, "fp32")
    out, lse, _ = _prefill(lib, c32.q, c32.k, c32.v, c32.bias, 3)
    out2, lse2, _ = _prefill(lib, c32.q.astype(np.float64), c32.k.astype(np.float64),
                             c32.v.astype(np.float64), c32.bias, 3)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


# ----------------------------------------------------------------------------
# brute force
# ----------------------------------------------------------------------------
def _brute(q, k, v, r, ctx, window):
    """Pure-Python: explicit exp of each logit (no max subtraction), math.fsum."""
    B, n_q, Hq, D = q.shape
    Hkv = k.shape[2]
    R = r.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, n_q, Hq, D))
    lse = np.zeros((B, n_q, Hq))
    for b in range(B):
        for t in range(n_q):
            i = int(ctx[b]) - n_q + t
            for h in range(Hq):
                weights, keys = [], []
                for j in range(int(ctx[b])):
                    dist = i - j
                    if dist < 0 or (window > 0 and dist >= window):
                        continue
                    logit = math.fsum(float(q[b, t, h, e]) * float(k[b, j, h // G, e]) for e in range(D))
                    logit = logit / math.sqrt(D) + float(r[h, min(dist, R - 1)])
                    weights.append(math.exp(logit))
                    keys.append(j)
                Z = math.fsum(weights)
                for e in range(D):
                    out[b, t, h, e] = math.fsum(w * float(v[b, j, h // G, e]) for w, j in zip(weights, keys)) / Z
                lse[b, t, h] = math.log(Z)
    return out, lse


def pin_brute_force(lib):
    for (seed, B, Lq, Lk, Hq, Hkv, D, R, window) in [(30, 1, 7, 7, 2, 1, 4, 3, 0), (31, 2, 3, 8, 4, 2, 4, 10, 0),
                                                      (32, 1, 8, 8, 3, 3, 3, 2, 3), (33, 1, 5, 11, 4, 1, 5, 6, 4)]:
        q, k, v, r = _rand(seed, B, Lq, Lk, Hq, Hkv, D, R, scale_bias=1.0)
        out, lse, _ = _prefill(lib, q, k, v, r, window)
        bo, bl = _brute(q, k, v, r, [Lk] * B, window)
        np.testing.assert_allclose(out, bo, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, bl, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# token-dependent bias: every query row has its own table r_t[h, :]
# (the "qkvr" linears of the recipes page's Variants section read as producing a
# per-token table: logit = q.k/sqrt(D) + r_t[h, min(p - j, R - 1)])
# ----------------------------------------------------------------------------
def _prefill_tok(lib, q, k, v, rt, window=0, probs=False):
    B = q.shape[0]
    return oracle.ref_attention(q, k, v, rt, [k.shape[1]] * B, [window] * B, None, want_probs=probs, lib=lib,
                                token_bias=True)


def _rand_tok(seed, B, Lq, Hq, R, scale=0.5):
    return scale * np.random.default_rng(seed).standard_normal((B, Lq, Hq, R))


def pin_tokbias_equal_rows_is_static(lib):
    """Every row given the static table r[h, :]: the same result as the static-table
    oracle, bit for bit."""
    for (B, Lq, Lk, Hq, Hkv, D, R, window) in [(2, 6, 11, 4, 2, 8, 5, 0), (1, 9, 9, 3, 1, 8, 20, 4)]:
        q, k, v, r = _rand(40 + Lq, B, Lq, Lk, Hq, Hkv, D, R)
        rt = np.broadcast_to(r[None, None], (B, Lq, Hq, R)).copy()
        o1, l1, _ = _prefill(lib, q, k, v, r, window)
        o2, l2, _ = _prefill_tok(lib, q, k, v, rt, window)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def pin_tokbias_row_shift(lib):
    """Adding c[b, t, h] to every entry of row (b, t, h)'s table leaves out unchanged and
    adds c[b, t, h] to that row's lse."""
    B, Lq, Lk, Hq, Hkv, D, R = 2, 5, 9, 4, 2, 8, 6
    q, k, v, _ = _rand(41, B, Lq, Lk, Hq, Hkv, D, R)
    rt = _rand_tok(42, B, Lq, Hq, R)
    c = np.random.default_rng(43).uniform(-3, 3, (B, Lq, Hq))
    for window in (0, 3):
        o1, l1, _ = _prefill_tok(lib, q, k, v, rt, window)
        o2, l2, _ = _prefill_tok(lib, q, k, v, rt + c[..., None], window)
        np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l2, l1 + c, rtol=0, atol=1e-12)


def pin_tokbias_window_one(lib):
    """W = 1: out_t = v_t and lse_t = q_t.k_t/sqrt(D) + r_t[h, 0]."""
    B, L, Hq, Hkv, D, R = 2, 7, 4, 2, 8, 5
    q, k, v, _ = _rand(44, B, L, L, Hq, Hkv, D, R)
    rt = _rand_tok(45, B, L, Hq, R)
    out, lse, _ = _prefill_tok(lib, q, k, v, rt, 1)
    G = Hq // Hkv
    for h in range(Hq):
        np.testing.assert_allclose(out[:, :, h], v[:, :, h // G], rtol=0, atol=1e-12)
        dots = np.einsum("bld,bld->bl", q[:, :, h], k[:, :, h // G])
        np.testing.assert_allclose(lse[:, :, h], dots / math.sqrt(D) + rt[:, :, h, 0], rtol=0, atol=1e-12)


def pin_tokbias_zero_keys(lib):
    """K = 0: the weights of row (b, t, h) are the softmax of its own table's entries at the
    clamped distances, whatever Q is."""
    B, Lq, Lk, Hq, Hkv, D, R = 1, 6, 10, 2, 1, 8, 4
    q, _, v, _ = _rand(46, B, Lq, Lk, Hq, Hkv, D, R)
    k = np.zeros((B, Lk, Hkv, D))
    rt = _rand_tok(47, B, Lq, Hq, R, 1.0)
    _, lse, probs = _prefill_tok(lib, q, k, v, rt, 0, probs=True)
    for t in range(Lq):
        p = Lk - Lq + t
        for h in range(Hq):
            b = np.array([rt[0, t, h, min(p - j, R - 1)] for j in range(p + 1)])
            w = np.exp(b - b.max())
            np.testing.assert_allclose(probs[0, t, h, :p + 1], w / w.sum(), rtol=0, atol=1e-13)
            assert abs(lse[0, t, h] - (b.max() + math.log(w.sum()))) < 1e-12


def pin_tokbias_is_sdpa(lib):
    """torch SDPA (float64) with the float mask m[b, h, t, j] = r_t[h, min(p - j, R - 1)] on
    the visible pairs and -inf elsewhere, for a chunk after a prefix and a window."""
    for (B, Lq, Lk, Hq, Hkv, D, R, window) in [(2, 5, 12, 4, 2, 8, 7, 0), (1, 8, 8, 6, 3, 8, 3, 4)]:
        q, k, v, _ = _rand(48 + Lk, B, Lq, Lk, Hq, Hkv, D, R)
        rt = _rand_tok(49 + Lk, B, Lq, Hq, R)
        out, _, _ = _prefill_tok(lib, q, k, v, rt, window)
        vis = _visibility(Lq, Lk, window)
        dist = (Lk - Lq + np.arange(Lq))[:, None] - np.arange(Lk)[None, :]
        idx = np.clip(dist, 0, R - 1)
        mask = np.full((B, Hq, Lq, Lk), -np.inf)
        for b in range(B):
            for h in range(Hq):
                for t in range(Lq):
                    mask[b, h, t, vis[t]] = rt[b, t, h, idx[t, vis[t]]]
        G = Hq // Hkv
        ref = _sdpa(q, _expand_kv(k, G), _expand_kv(v, G), mask, 1.0 / math.sqrt(D))
        np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def pin_tokbias_brute_force(lib):
    """Pure-Python loops, explicit exp, math.fsum, each row with its own table."""
    B, Lq, Lk, Hq, Hkv, D, R, window = 1, 4, 7, 2, 1, 4, 3, 5
    q, k, v, _ = _rand(50, B, Lq, Lk, Hq, Hkv, D, R, scale_bias=1.0)
    rt = _rand_tok(51, B, Lq, Hq, R, 1.0)
    out, lse, _ = _prefill_tok(lib, q, k, v, rt, window)
    for t in range(Lq):
        i = Lk - Lq + t
        for h in range(Hq):
            ws, js = [], []
            for j in range(Lk):
                d = i - j
                if d < 0 or d >= window:
                    continue
                logit = math.fsum(float(q[0, t, h, e]) * float(k[0, j, 0, e]) for e in range(D)) / math.sqrt(D)
                ws.append(math.exp(logit + float(rt[0, t, h, min(d, R - 1)])))
                js.append(j)
            Z = math.fsum(ws)
            for e in range(D):
                ref = math.fsum(w * float(v[0, j, 0, e]) for w, j in zip(ws, js)) / Z
                assert abs(out[0, t, h, e] - ref) <= 1e-12
            assert abs(lse[0, t, h] - math.log(Z)) <= 1e-12


def pin_tokbias_rows_independent(lib):
    """Changing the table of one row (b, t, h) changes that row's output only."""
    B, Lq, Lk, Hq, Hkv, D, R = 2, 6, 9, 4, 2, 8, 5
    q, k, v, _ = _rand(52, B, Lq, Lk, Hq, Hkv, D, R)
    rt = _rand_tok(53, B, Lq, Hq, R)
    o1, l1, _ = _prefill_tok(lib, q, k, v, rt, 0)
    rt2 = rt.copy()
    rt2[1, 3, 2, :] += np.linspace(-1, 2, R)
    o2, l2, _ = _prefill_tok(lib, q, k, v, rt2, 0)
    changed = np.abs(o2 - o1).max(axis=-1) > 0
    expect = np.zeros((B, Lq, Hq), dtype=bool)
    expect[1, 3, 2] = True
    assert np.array_equal(changed, expect) and np.array_equal(l2 != l1, expect)


ALL_PINS = [
    pin_zero_bias_is_sdpa, pin_alibi_is_sdpa, pin_golden_examples, pin_window_one, pin_position_zero,
    pin_R_one, pin_zero_keys, pin_constant_values, pin_bias_shift, pin_wide_window_is_full,
    pin_probs_sum_to_one, pin_chunk_equals_full, pin_paged_equals_contiguous, pin_input_widening,
    pin_brute_force,
    pin_tokbias_equal_rows_is_static, pin_tokbias_row_shift, pin_tokbias_window_one, pin_tokbias_zero_keys,
    pin_tokbias_is_sdpa, pin_tokbias_brute_force, pin_tokbias_rows_independent,
]
