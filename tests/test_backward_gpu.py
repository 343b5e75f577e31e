"""Backward pass of the bf16 prefill (rattn_prefill_backward) against the fp64 oracle, element
by element.

The forward runs on the GPU (rattn_prefill) to give out and lse, as in training; the C oracle
(rattn_ref_cpu_backward) recomputes everything from q, k, v, r and dO in double and also
returns, for every gradient entry, the sum of its terms' magnitudes (absum: dS replaced by
dS_abs = P_j (|dP_j - D| + a_j + D_abs), a_j = sum_e |dO_e v_j,e| the size of dP_j's terms,
D_abs = sum_j P_j a_j the size of D's).

Bound, per entry:  |gpu - oracle| <= 2^-6 * absum + 1e-7.
Derivation (u = 2^-8, the unit roundoff of bf16):
  - P and dS are rounded to bf16 as MFMA operands: relative error u per term;
  - D comes from the bf16 output of the GPU forward, which is within u (P rounded to bf16 in
    P.V) plus u (output rounding) of the exact O: |error of D| <= 2u D_abs, and every dS_j
    carries P_j times that;
  - P is recomputed from the fp32 logits and the forward's lse (error ~1e-5 relative, far
    below u), the fp32 sums of <= 8192 terms add at most 8192 * 2^-24 = 2^-11 of absum;
so each entry is within (2u + 2^-11) absum ~ 2^-7 absum; the bound takes twice that.  The
1e-7 covers entries whose exact value and absum are both zero (keys no query sees: the GPU
must write exact zeros there) and fp32 rounding at that scale.
The D term dominates these sums (a_j + D_abs is ~10x |dP - D|) and it is summed over
every pair, so for dbias, whose entries are sums over up to 8192 pairs, the bound is loose.
The second family of tests feeds the backward the forward oracle's output rounded to bf16
and its lse rounded to fp32 (oracle outputs, not GPU results) and the oracle takes D from
that same output (D = rowsum(dO * out), the kernels' definition).  What remains is the
backward's own arithmetic:
  - P from fp32 logits (128-term fp32 sums, ~2^-17 of sum |q k|) and the fp32 lse: relative
    error below 2^-13;
  - dP and D as fp32 sums of 128 products: within 2^-17 of a_j and D_abs;
  - dq, dk, dv: dS and P rounded to bf16 (u) and fp32 accumulation over <= 8192 terms
    (2^-11): within (2^-8 + 2^-11 + 2^-13) sum|dS||x| + 2^-17 sum P (a + D_abs)|x|;
  - dbias: dS summed in fp32 without rounding to bf16: within (2^-11 + 2^-13) sum|dS| +
    2^-17 sum P (a + D_abs);
so with the oracle's magnitude sums at weight w = 2^-6 on the D term, the bound is
2^-6 * absum for dq, dk, dv and 2^-9 * absum for dbias (each 3-4x the derived worst case),
per entry, plus 1e-7.
Cases: ragged lengths (tails of 12 and 20 rows), a chunk after a prefix (Lq < Lk), a window
with one KV head, one query head per KV head with window 1 (closed form: dq = dk = dbias = 0),
three query heads per KV head (the kernels pair heads; the odd one out runs alone), sixteen
query heads per KV head, and the full 8K-token window-4096 workload the benchmark times.
"""
import numpy as np
import pytest
import torch

from gpu_util import dev, host

import oracle
import relative_bias_gqa_amd as rb
from relative_bias_gqa_amd import synth

pytestmark = pytest.mark.gpu

BOUND_REL = 2.0 ** -6
BOUND_ABS = 1e-7

CASES = [
    # name, seed, B, Lq, Lk, Hq, Hkv, R, window
    ("full_ragged", 81, 2, 300, 300, 8, 2, 100, 0),
    ("chunk_after_prefix", 82, 1, 200, 660, 16, 2, 1000, 0),
    ("window_one_kv_head", 83, 2, 500, 500, 8, 1, 64, 129),
    ("window_one", 84, 1, 100, 130, 4, 4, 9, 1),
    ("three_heads_per_kv_head", 85, 1, 77, 333, 6, 2, 50, 100),
    ("sixteen_heads_per_kv_head", 86, 1, 150, 150, 32, 2, 40, 0),
    ("window_chunk_unseen_keys", 87, 1, 64, 400, 8, 2, 30, 50),
]


def run_backward(case):
    f = case.fwd
    q, k, v, r = dev(f.q), dev(f.k), dev(f.v), dev(f.bias)
    out, lse = rb.prefill(q, k, v, r, f.window)
    dq, dk, dv, dbias = rb.prefill_backward(q, k, v, r, out, lse, dev(case.dout), f.window)
    torch.cuda.synchronize()
    return host(dq), host(dk), host(dv), host(dbias)


def check(name, got, ref, absum, rel=BOUND_REL):
    """Every entry within rel * absum + BOUND_ABS of the oracle."""
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite"
    err = np.abs(got - ref)
    bound = rel * absum + BOUND_ABS
    ratio = err / bound
    worst = np.unravel_index(np.argmax(ratio), ratio.shape) if ratio.size else ()
    nrm = np.linalg.norm(ref)
    normwise = np.linalg.norm(got - ref) / nrm if nrm > 0 else 0.0
    print(f"  {name}: max err {err.max() if err.size else 0:.2e}, worst err/bound "
          f"{ratio.max() if ratio.size else 0:.3f} at {worst}, normwise {normwise:.2e}", flush=True)
    assert (err <= bound).all(), f"{name}: {int((err > bound).sum())} entries beyond the bound"


_ORACLE = {}


def oracle_backward(case):
    """The oracle's gradients and magnitude sums for a case, computed once per case name."""
    if case.name not in _ORACLE:
        f = case.fwd
        _ORACLE[case.name] = oracle.ref_backward(f.q, f.k, f.v, f.bias, case.dout, f.window)
    return _ORACLE[case.name]


def compare_all(grads, case):
    refs, absums = oracle_backward(case)
    for name, g, ref, a in zip(("dq", "dk", "dv", "dbias"), grads, refs, absums):
        check(name, g, ref, a)


@pytest.mark.parametrize("name,seed,B,Lq,Lk,Hq,Hkv,R,window", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(name, seed, B, Lq, Lk, Hq, Hkv, R, window):
    print(f"case backward {name}", flush=True)
    case = synth.make_backward(seed, B, Lq, Lk, Hq, Hkv, R, window, name)
    compare_all(run_backward(case), case)


TIGHT_WEIGHT = 2.0 ** -6
TIGHT_REL = {"dq": 2.0 ** -6, "dk": 2.0 ** -6, "dv": 2.0 ** -6, "dbias": 2.0 ** -9}


def run_backward_given_forward(case):
    """The backward on the GPU with out and lse from the forward oracle (out rounded to bf16
    to nearest even, lse to fp32); returns the gradients and the oracle's output (bf16 bits)."""
    from oracle.sconv import f64_to_bf16
    f = case.fwd
    ref_o, ref_l, _ = oracle.ref_prefill(f.q, f.k, f.v, f.bias, f.window)
    out_b = f64_to_bf16(ref_o)
    q, k, v, r = dev(f.q), dev(f.k), dev(f.v), dev(f.bias)
    lse = dev(ref_l.astype(np.float32))
    dq, dk, dv, dbias = rb.prefill_backward(q, k, v, r, dev(out_b), lse, dev(case.dout), f.window)
    torch.cuda.synchronize()
    return (host(dq), host(dk), host(dv), host(dbias)), out_b


def compare_given_forward(case):
    f = case.fwd
    grads, out_b = run_backward_given_forward(case)
    refs, absums = oracle.ref_backward(f.q, f.k, f.v, f.bias, case.dout, f.window, out=out_b,
                                       abs_weight=TIGHT_WEIGHT)
    for name, g, ref, a in zip(("dq", "dk", "dv", "dbias"), grads, refs, absums):
        check(name, g, ref, a, TIGHT_REL[name])


@pytest.mark.parametrize("name,seed,B,Lq,Lk,Hq,Hkv,R,window", CASES, ids=[c[0] for c in CASES])
def test_backward_given_oracle_forward(name, seed, B, Lq, Lk, Hq, Hkv, R, window):
    print(f"case backward (oracle forward) {name}", flush=True)
    compare_given_forward(synth.make_backward(seed, B, Lq, Lk, Hq, Hkv, R, window, name))


def test_backward_full_size_given_oracle_forward():
    """The full-size workload with the tight bounds (out and lse from the forward oracle)."""
    print("case backward (oracle forward) full size swa_prefill_8k_bwd", flush=True)
    compare_given_forward(synth.swa_prefill_8k_bwd())


def test_backward_full_size():
    """The backward of the 8K-token window-4096 prefill (16/2 heads, R 4096) at full size, in
    the launch configuration the benchmark times: every entry of dq, dk, dv and dbias against
    the oracle (about 30 s of host time on 16 threads)."""
    print("case backward full size swa_prefill_8k_bwd", flush=True)
    case = synth.swa_prefill_8k_bwd()
    grads = run_backward(case)
    compare_all(grads, case)


def test_backward_nan_gradient_row_stays_in_bounds():
    """A non-finite output gradient must not make the kernels write outside their outputs.
    One dO row is NaN; dbias sits inside a larger buffer whose guard entries on both sides
    must come back unchanged.  Gradients that do not depend on that row stay finite: dq of
    every other row, dbias of every other head, dk and dv of the other KV head."""
    print("case backward NaN dout row, guarded dbias", flush=True)
    B, Lq, Lk, Hq, Hkv, R, window = 1, 96, 96, 8, 2, 40, 0
    case = synth.make_backward(88, B, Lq, Lk, Hq, Hkv, R, window, "nan_row")
    f = case.fwd
    q, k, v, r = dev(f.q), dev(f.k), dev(f.v), dev(f.bias)
    out, lse = rb.prefill(q, k, v, r, window)
    dout = dev(case.dout)
    t_nan, h_nan = 37, 3
    dout[0, t_nan, h_nan, :] = float("nan")
    guard = 4096
    sentinel = 12345.0
    buf = torch.full((guard + Hq * R + guard,), sentinel, dtype=torch.float32, device="cuda")
    dbias = buf[guard:guard + Hq * R].view(Hq, R)
    dq = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    dk = torch.empty(k.shape, dtype=torch.float32, device="cuda")
    dv = torch.empty(v.shape, dtype=torch.float32, device="cuda")
    ws = torch.empty(rb.rattn_prefill_backward_workspace_bytes(B, Lq, Lk, Hq, Hkv), dtype=torch.uint8, device="cuda")
    rb.rattn_prefill_backward(q, k, v, r, out, dout, lse, dq, dk, dv, dbias, window, ws)
    torch.cuda.synchronize()
    g = host(buf)
    assert (g[:guard] == sentinel).all() and (g[guard + Hq * R:] == sentinel).all(), "write outside dbias"
    dq_h, dbias_h, dk_h, dv_h = host(dq), host(dbias), host(dk), host(dv)
    rows = np.ones((B, Lq, Hq), dtype=bool)
    rows[0, t_nan, h_nan] = False
    assert np.isfinite(dq_h[rows]).all()
    assert np.isfinite(np.delete(dbias_h, h_nan, axis=0)).all()
    other_kv = 1 - h_nan // (Hq // Hkv)
    assert np.isfinite(dk_h[:, :, other_kv]).all() and np.isfinite(dv_h[:, :, other_kv]).all()


def test_backward_empty_chunk_zeroes_gradients():
    """No queries (Lq = 0) over 300 keys: dk, dv and dbias are written as zeros (they start
    as NaN here), dq has no elements."""
    print("case backward empty chunk", flush=True)
    Lk, Hq, Hkv, R = 300, 8, 2, 32
    k = torch.randn(1, Lk, Hkv, 128, device="cuda").to(torch.bfloat16)
    v = torch.randn(1, Lk, Hkv, 128, device="cuda").to(torch.bfloat16)
    q = torch.empty(1, 0, Hq, 128, device="cuda", dtype=torch.bfloat16)
    r = torch.randn(Hq, R, device="cuda")
    dk = torch.full((1, Lk, Hkv, 128), float("nan"), device="cuda")
    dv = torch.full_like(dk, float("nan"))
    dr = torch.full((Hq, R), float("nan"), device="cuda")
    ws = torch.empty(rb.rattn_prefill_backward_workspace_bytes(1, 0, Lk, Hq, Hkv), dtype=torch.uint8, device="cuda")
    # zero-size tensors may have no storage: pass a live one-element pointer for q, out, dout, lse, dq
    dummy = torch.zeros(1, device="cuda")
    rc = rb.load().rattn_prefill_backward(q.data_ptr() or dummy.data_ptr(), k.data_ptr(), v.data_ptr(),
                                          r.data_ptr(), dummy.data_ptr(), dummy.data_ptr(), dummy.data_ptr(),
                                          dummy.data_ptr(), dk.data_ptr(), dv.data_ptr(), dr.data_ptr(), 1, 0,
                                          Lk, Hq, Hkv, 128, R, 0, ws.data_ptr(), ws.numel(), None)
    torch.cuda.synchronize()
    assert rc == rb.RATTN_OK, rb.rattn_last_error()
    assert int((dk != 0).sum()) == 0 and int((dv != 0).sum()) == 0 and int((dr != 0).sum()) == 0


DETERMINISM_SHAPES = [
    # name, seed, B, Lq, Lk, Hq, Hkv, R, window
    ("swa_prefill_8k_bwd", None, 1, 8192, 8192, 16, 2, 4096, 4096),
    ("causal_2k", 89, 1, 2048, 2048, 16, 2, 2048, 0),
]


@pytest.mark.parametrize("name,seed,B,Lq,Lk,Hq,Hkv,R,window", DETERMINISM_SHAPES,
                         ids=[c[0] for c in DETERMINISM_SHAPES])
def test_backward_deterministic_with_reused_workspace(name, seed, B, Lq, Lk, Hq, Hkv, R, window):
    """dq, dk and dv are sums in a fixed order, whichever workgroup of a token tile or key block
    cut in two finishes last.  The 8K-token window-4096 workload (512 units per pass: one
    chunk each) and a causal 2048-token prefill (few units: its tiles and key blocks are cut
    in two) each run
    once on a fresh zeroed workspace and three times on one workspace whose bytes start as
    0xFF (split counters -1, partial slots NaN: every call must reset what it counts on); every
    call gives the first one's dq, dk and dv bit for bit; the first call is within the bound
    of the oracle, and so is every call's dr (fp32 atomic adds in any order: its last bits may
    differ from call to call)."""
    print(f"case backward determinism, reused poisoned workspace, {name}", flush=True)
    case = synth.swa_prefill_8k_bwd() if seed is None else synth.make_backward(seed, B, Lq, Lk, Hq, Hkv, R, window,
                                                                               name)
    f = case.fwd
    q, k, v, r = dev(f.q), dev(f.k), dev(f.v), dev(f.bias)
    out, lse = rb.prefill(q, k, v, r, f.window)
    dout = dev(case.dout)
    n = rb.rattn_prefill_backward_workspace_bytes(B, Lq, Lk, Hq, Hkv)

    def call(ws):
        dq = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
        dk = torch.full(k.shape, float("nan"), dtype=torch.float32, device="cuda")
        dv = torch.full(v.shape, float("nan"), dtype=torch.float32, device="cuda")
        dbias = torch.full(r.shape, float("nan"), dtype=torch.float32, device="cuda")
        rb.rattn_prefill_backward(q, k, v, r, out, dout, lse, dq, dk, dv, dbias, f.window, ws)
        torch.cuda.synchronize()
        return host(dq), host(dk), host(dv), host(dbias)

    refs, absums = oracle_backward(case)
    first = call(torch.zeros(n, dtype=torch.uint8, device="cuda"))
    compare_all(first, case)
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")
    for i in range(3):
        got = call(ws)
        for gname, a, b in zip(("dq", "dk", "dv"), first, got):
            assert np.array_equal(a, b), f"call {i + 1}: {gname} differs from the first call"
        check(f"call {i + 1} dbias", got[3], refs[3], absums[3])


def test_backward_graph_capture():
    """Captured in a graph, the backward's launches replay with the eager call's results.  A
    causal 1024-token prefill (16/2 heads, R 300; its tiles and key blocks are cut in two) is
    captured once and replayed three times, each replay after an eager call into other
    buffers and a synchronisation; every eager call is within the bound of the oracle and
    every replay gives the eager dq, dk and dv bit for bit and a dr within the same bound (fp32
    atomic adds in any order: with R = 300 every distance from 299 on lands in one entry, a
    sum of 263K terms per head that cancel, so its last bits differ from run to run)."""
    print("case backward graph capture, causal 1024", flush=True)
    B, Lq, Lk, Hq, Hkv, R, window = 1, 1024, 1024, 16, 2, 300, 0
    case = synth.make_backward(90, B, Lq, Lk, Hq, Hkv, R, window, "graph_causal_1k")
    f = case.fwd
    q, k, v, r = dev(f.q), dev(f.k), dev(f.v), dev(f.bias)
    out, lse = rb.prefill(q, k, v, r, window)
    dout = dev(case.dout)
    refs, absums = oracle_backward(case)

    def buffers():
        return (torch.empty(q.shape, dtype=torch.float32, device="cuda"),
                torch.empty(k.shape, dtype=torch.float32, device="cuda"),
                torch.empty(v.shape, dtype=torch.float32, device="cuda"),
                torch.empty(r.shape, dtype=torch.float32, device="cuda"))

    n = rb.rattn_prefill_backward_workspace_bytes(B, Lq, Lk, Hq, Hkv)
    ws_g = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")
    ws_e = torch.empty(n, dtype=torch.uint8, device="cuda")
    g_out, e_out = buffers(), buffers()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        rb.rattn_prefill_backward(q, k, v, r, out, dout, lse, *g_out, window, ws_g)
    torch.cuda.synchronize()
    for i in range(3):
        for t in e_out + g_out:
            t.fill_(float("nan"))
        rb.rattn_prefill_backward(q, k, v, r, out, dout, lse, *e_out, window, ws_e)
        torch.cuda.synchronize()
        eager = [host(t) for t in e_out]
        for gname, g, ref, a in zip(("dq", "dk", "dv", "dbias"), eager, refs, absums):
            check(f"eager {i} {gname}", g, ref, a)
        graph.replay()
        torch.cuda.synchronize()
        got = [host(t) for t in g_out]
        for gname, a, b in zip(("dq", "dk", "dv"), eager, got):
            assert np.array_equal(a, b), f"replay {i}: {gname} differs from the eager call"
        check(f"replay {i} dbias", got[3], refs[3], absums[3])
