"""Backward pass of the bf16 prefill (rattn_prefill_backward) against the fp64 oracle.

The forward runs on the GPU (rattn_prefill) to give out and lse, as in training; the oracle
recomputes everything from q, k, v, r and dO.  Tolerances (bf16 inputs, fp32 accumulation;
the rounding of P and dS to bf16 for the MFMAs and of out to bf16 in D = rowsum(dO * out)
each move a term by at most 2^-9 of its size):
  dq, dk, dv: |gpu - ref|_2 <= 1e-2 |ref|_2 and max |gpu - ref| <= 3e-2 max |ref|;
  dbias[h, d]: |gpu - ref| <= 1e-2 * (sum of |dS| behind the entry) + 1e-6 * max of those sums
  + 1e-6 per pair behind the entry;
  a reference that is exactly zero: max |gpu| <= 1e-4 (fp32 rounding of dP - D).
Cases: ragged lengths (tails of 12 and 20 rows), a chunk after a prefix (Lq < Lk), a window
with one KV head, one query head per KV head with window 1 (closed form: dq = dk = dbias = 0),
three query heads per KV head (the kernels pair heads; the odd one out runs alone).
"""
import numpy as np
import pytest
import torch

from gpu_util import dev, host

import relative_bias_gqa_amd as rb
from relative_bias_gqa_amd import synth
from oracle.backward import prefill_backward

pytestmark = pytest.mark.gpu

CASES = [
    # name, seed, B, Lq, Lk, Hq, Hkv, R, window
    ("full_ragged", 81, 2, 300, 300, 8, 2, 100, 0),
    ("chunk_after_prefix", 82, 1, 200, 660, 16, 2, 1000, 0),
    ("window_one_kv_head", 83, 2, 500, 500, 8, 1, 64, 129),
    ("window_one", 84, 1, 100, 130, 4, 4, 9, 1),
    ("three_heads_per_kv_head", 85, 1, 77, 333, 6, 2, 50, 100),
    ("sixteen_heads_per_kv_head", 86, 1, 150, 150, 32, 2, 40, 0),
]


def run_backward(case):
    f = case.fwd
    q, k, v, r = dev(f.q), dev(f.k), dev(f.v), dev(f.bias)
    out, lse = rb.prefill(q, k, v, r, f.window)
    dq, dk, dv, dbias = rb.prefill_backward(q, k, v, r, out, lse, dev(case.dout), f.window)
    torch.cuda.synchronize()
    return host(dq), host(dk), host(dv), host(dbias)


def check(name, got, ref):
    assert np.isfinite(got).all(), f"{name}: non-finite"
    err = got - ref
    nrm = np.linalg.norm(ref)
    rel = np.linalg.norm(err) / max(nrm, 1e-30)
    mx = np.abs(err).max() if err.size else 0.0
    print(f"  {name}: normwise {rel:.2e}, max {mx:.2e} (max |ref| {np.abs(ref).max():.2e})", flush=True)
    if nrm == 0:
        # an exact zero that the kernel reaches as dS = P (dP - D) with P = 1 and dP, D two
        # fp32 dot products of 128 terms of size ~1 taken in different orders
        assert mx <= 1e-4, name
        return
    assert rel <= 1e-2, name
    assert mx <= 3e-2 * np.abs(ref).max(), name


@pytest.mark.parametrize("name,seed,B,Lq,Lk,Hq,Hkv,R,window", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(name, seed, B, Lq, Lk, Hq, Hkv, R, window):
    print(f"case backward {name}", flush=True)
    case = synth.make_backward(seed, B, Lq, Lk, Hq, Hkv, R, window, name)
    dq, dk, dv, dr = run_backward(case)
    f = case.fwd
    rq, rk, rv, rr, rabs = prefill_backward(f.q, f.k, f.v, f.bias, case.dout, window)
    check("dq", dq, rq)
    check("dk", dk, rk)
    check("dv", dv, rv)
    derr = np.abs(dr - rr)
    # pairs behind each entry: every dS carries the fp32 rounding of dP - D (up to ~1e-6)
    pos = (Lk - Lq) + np.arange(Lq)[:, None]
    dist = pos - np.arange(Lk)[None, :]
    vis = (dist >= 0) & ((window <= 0) | (dist <= window - 1))
    npairs = B * np.bincount(np.minimum(dist[vis], R - 1), minlength=R)
    bound = 1e-2 * rabs + 1e-6 * max(rabs.max(), 1e-30) + 1e-6 * npairs[None, :]
    print(f"  dbias: max err {derr.max():.2e}, worst err/bound {(derr / bound).max():.2f}", flush=True)
    assert (derr <= bound).all()


def test_backward_full_size_sampled():
    """The backward of the 8K-token window-4096 prefill (16/2 heads, R 4096) at full size, in the
    launch configuration the benchmark times: 27 dq rows against the oracle row by row (same
    bar as above), and two sums that hold at any size, bounded from the inputs alone:
      sum_j dv[j] = sum_i sum_(h in group) dO[i, h] (every row of P sums to one): the sum of
        8192 dv entries, each within ~2e-3 of its size (the cases above), is bounded by
        2e-2 of the root-sum-square of the dO terms (a head left out would miss by ~90);
      sum_d dr[h, d] = 0 (every row of dS sums to zero), a coarse check: D comes from the bf16
        output (|out| <= max |V|), so |error| <= 2^-8 max|V| sum |dO| over the head."""
    print("case backward full size swa_prefill_8k_bwd", flush=True)
    from oracle.backward import prefill_backward_dq_rows
    from oracle.sconv import bf16_to_f64
    case = synth.swa_prefill_8k_bwd()
    dq, dk, dv, dr = run_backward(case)
    f = case.fwd
    assert np.isfinite(dk).all() and np.isfinite(dv).all() and np.isfinite(dr).all()
    rng = np.random.default_rng(5)
    rows = [(0, int(t), int(h)) for t, h in zip(rng.integers(0, f.Lq, 24), rng.integers(0, f.Hq, 24))]
    rows += [(0, 0, 0), (0, f.Lq - 1, f.Hq - 1), (0, f.window - 1, 7)]
    ref = prefill_backward_dq_rows(f.q, f.k, f.v, f.bias, case.dout, f.window, rows)
    check("dq rows", np.stack([dq[b, t, h] for (b, t, h) in rows]), ref)
    do = bf16_to_f64(case.dout)  # [1, L, Hq, 128]
    G = f.Hq // f.Hkv
    grp = do.reshape(1, f.Lq, f.Hkv, G, 128)
    expect = grp.sum(axis=(1, 3))
    bound = 2e-2 * np.sqrt((grp ** 2).sum(axis=(1, 3))) + 1e-3
    err = np.abs(dv.sum(axis=1) - expect)
    print(f"  sum dv: max err {err.max():.3e}, worst err/bound {(err / bound).max():.3f}", flush=True)
    assert (err <= bound).all()
    vmax = np.abs(bf16_to_f64(f.v)).max()
    rbound = 2.0 ** -8 * vmax * np.abs(do).sum(axis=(0, 1, 3)) + 1e-3
    rerr = np.abs(dr.sum(axis=1))
    print(f"  sum dr: max {rerr.max():.3e}, worst err/bound {(rerr / rbound).max():.3f}", flush=True)
    assert (rerr <= rbound).all()


def test_backward_empty_chunk_zeroes_gradients():
    """No queries (Lq = 0) over 300 keys: dk, dv and dbias are written as zeros (they start
    as NaN here), dq has no elements."""
    print("case backward empty chunk", flush=True)
    Lk, Hq, Hkv, R = 300, 8, 2, 32
    k = torch.randn(1, Lk, Hkv, 128, device="cuda").to(torch.bfloat16)
    v = torch.randn(1, Lk, Hkv, 128, device="cuda").to(torch.bfloat16)
    q = torch.empty(1, 0, Hq, 128, device="cuda", dtype=torch.bfloat16)
    r = torch.randn(Hq, R, device="cuda")
    lse = torch.empty(1, 0, Hq, device="cuda")
    dq = torch.empty(1, 0, Hq, 128, device="cuda")
    dk = torch.full((1, Lk, Hkv, 128), float("nan"), device="cuda")
    dv = torch.full_like(dk, float("nan"))
    dr = torch.full((Hq, R), float("nan"), device="cuda")
    ws = torch.empty(rb.rattn_prefill_backward_workspace_bytes(1, 0, Hq), dtype=torch.uint8, device="cuda")
    # zero-size tensors may have no storage: pass a live one-element pointer for q, out, dout, lse, dq
    dummy = torch.zeros(1, device="cuda")
    rc = rb.load().rattn_prefill_backward(q.data_ptr() or dummy.data_ptr(), k.data_ptr(), v.data_ptr(),
                                          r.data_ptr(), dummy.data_ptr(), dummy.data_ptr(), dummy.data_ptr(),
                                          dummy.data_ptr(), dk.data_ptr(), dv.data_ptr(), dr.data_ptr(), 1, 0,
                                          Lk, Hq, Hkv, 128, R, 0, ws.data_ptr(), ws.numel(), None)
    torch.cuda.synchronize()
    assert rc == rb.RATTN_OK, rb.rattn_last_error()
    assert int((dk != 0).sum()) == 0 and int((dv != 0).sum()) == 0 and int((dr != 0).sum()) == 0
