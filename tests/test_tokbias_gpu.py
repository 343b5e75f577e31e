"""The token-dependent relative-bias prefill (rattn_prefill_tokbias) against the fp64 oracle
(rattn_ref_cpu_tokbias), element by element, through the C ABI.

Every query row t has its own bf16 table r_t[h, :] (the recipes page keeps the "qkvr" linears
in BF16; read as the projection producing one table per token).  Cases span several tiles
with ragged tails; the table length R is short (every tile's distances clamp: SAT tiles),
medium (tiles that cross R - 1 and the diagonal: MIXED) and longer than every distance
(INNER tiles), with windows, a chunk after a prefix, one and sixteen query heads per KV head,
the key-range split, and table entries the definition never uses poisoned with NaN.  The
8K-token window-4096 workload with R = 512 is compared in full.
Bar: O max abs <= 2e-2, O mean abs <= 2e-3, LSE max abs <= 1e-3 (the attention parity bar).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import compare, dev, host

import relative_bias_gqa_amd as rb
from relative_bias_gqa_amd import synth

pytestmark = pytest.mark.gpu

CASES = [
    # name, seed, B, Lq, Lk, Hq, Hkv, R, window
    ("ragged_short_table", 91, 2, 300, 300, 8, 2, 4, 0),
    ("mixed_tiles", 92, 1, 333, 333, 16, 2, 100, 0),
    ("inner_tiles", 93, 1, 200, 200, 8, 1, 512, 0),
    ("window_chunk", 94, 2, 150, 700, 8, 2, 77, 120),
    ("g1_odd_table", 95, 1, 129, 400, 4, 4, 33, 0),
    ("g16", 96, 1, 96, 96, 32, 2, 64, 0),
    ("window_one", 97, 1, 70, 70, 8, 2, 5, 1),
    ("single_token", 98, 1, 1, 50, 8, 1, 8, 0),
]


def run(case, kv_splits=0, workspace=None):
    f = case.fwd
    q, k, v, rt = dev(f.q), dev(f.k), dev(f.v), dev(case.bias_tok)
    out, lse = rb.prefill_tokbias(q, k, v, rt, f.window, kv_splits=kv_splits, workspace=workspace)
    torch.cuda.synchronize()
    return host(out), host(lse)


def reference(case):
    f = case.fwd
    o, l, _ = oracle.ref_prefill_tokbias(f.q, f.k, f.v, case.bias_tok, f.window)
    return o, l


@pytest.mark.parametrize("name,seed,B,Lq,Lk,Hq,Hkv,R,window", CASES, ids=[c[0] for c in CASES])
def test_tokbias_matches_oracle(name, seed, B, Lq, Lk, Hq, Hkv, R, window):
    print(f"case tokbias {name}", flush=True)
    case = synth.make_prefill_tokbias(seed, B, Lq, Lk, Hq, Hkv, R, window, name)
    out, lse = run(case)
    ref_o, ref_l = reference(case)
    compare(out, lse, ref_o, ref_l, name)


@pytest.mark.parametrize("parts", [2, 3])
def test_tokbias_key_split(parts):
    print(f"case tokbias key split {parts}", flush=True)
    case = synth.make_prefill_tokbias(99, 1, 500, 1500, 16, 2, 300, 0, "split")
    n = rb.rattn_prefill_workspace_bytes(1, 500, 1500, 16, 2, 0, rb.RATTN_BF16, parts)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    out, lse = run(case, parts, ws)
    ref_o, ref_l = reference(case)
    compare(out, lse, ref_o, ref_l, f"split {parts}")
    assert int(ws[:256].count_nonzero()) == 0


def test_tokbias_unused_entries_may_hold_nan():
    """Entries at distances no visible key of the row has (d > p, and d >= window) are never
    used: filled with NaN they change nothing, bit for bit."""
    print("case tokbias NaN in unused entries", flush=True)
    B, Lq, Lk, Hq, Hkv, R, window = 1, 200, 260, 8, 2, 300, 90
    case = synth.make_prefill_tokbias(100, B, Lq, Lk, Hq, Hkv, R, window, "poison")
    out0, lse0 = run(case)
    tab = case.bias_tok.copy()
    pos = (Lk - Lq) + np.arange(Lq)
    d = np.arange(R)
    # entry d < R - 1 is used iff a visible key sits at distance d; the clamp entry R - 1 iff a
    # visible key sits at a distance >= R - 1
    used = (d[None, :] <= pos[:, None]) & (d[None, :] < window)      # [Lq, R]
    used[:, R - 1] = (pos >= R - 1) & (window - 1 >= R - 1)
    tab[0][np.broadcast_to((~used)[:, None, :], tab.shape[1:])] = 0x7FC0  # bf16 NaN
    case.bias_tok = tab
    out1, lse1 = run(case)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)
    ref_o, ref_l = reference(synth.make_prefill_tokbias(100, B, Lq, Lk, Hq, Hkv, R, window, "poison"))
    compare(out1, lse1, ref_o, ref_l, "poisoned table")


def test_tokbias_equal_rows_match_static_table():
    """Every row given the same table r[h, :] (bf16 values): the result of rattn_prefill with
    that table, within the parity bar of each other (the two paths add the bias at different
    points of the fp32 arithmetic, so not bit for bit)."""
    print("case tokbias equal rows", flush=True)
    c = synth.make_prefill(101, 1, 256, 256, 8, 2, 64, 0, "bf16")
    r_bits = synth.bf16_round(c.bias)
    tab = np.broadcast_to(r_bits[None, None], (1, 256, 8, 64)).copy()
    q, k, v = dev(c.q), dev(c.k), dev(c.v)
    o1, l1 = rb.prefill_tokbias(q, k, v, dev(tab), 0)
    o2, l2 = rb.prefill(q, k, v, dev(synth.to_float(r_bits)), 0)
    torch.cuda.synchronize()
    compare(host(o1), host(l1), host(o2).astype(np.float64), host(l2).astype(np.float64), "token vs static table")


def test_tokbias_workload_full():
    print("case swa_prefill_8k_tokbias (full output)", flush=True)
    case = synth.swa_prefill_8k_tokbias()
    out, lse = run(case)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    ref_o, ref_l = reference(case)
    compare(out, lse, ref_o, ref_l, "swa_prefill_8k_tokbias (all rows)")
