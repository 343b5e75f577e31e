"""HIP path against the fp64 oracle, element by element, through the C ABI.

Small cases span several tiles and end in ragged tails; the five named workloads run at
full size and are compared in full: every output element and every lse entry (the 32K-key
chunked prefill costs the oracle about 45 s of host time on 16 threads).
Bar: O max abs <= 2e-2, O mean abs <= 2e-3 (over all elements), LSE max abs <= 1e-3."""
import numpy as np
import pytest

import oracle
from gpu_util import compare, decode_to_device, dev, host
from relative_bias_gqa_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import relative_bias_gqa_amd as rb  # noqa: E402


def run_prefill(case):
    q, k, v, r = dev(case.q), dev(case.k), dev(case.v), dev(case.bias)
    out, lse = rb.prefill(q, k, v, r, case.window)
    torch.cuda.synchronize()
    return host(out), host(lse)


PREFILL_CASES = [
    # name, seed, B, Lq, Lk, Hq, Hkv, R, window, dtype
    ("single_token", 1, 1, 1, 1, 8, 1, 1, 0, "bf16"),
    ("ragged_clamp", 2, 2, 300, 300, 8, 2, 100, 0, "bf16"),
    ("chunk_ragged", 3, 1, 200, 333, 16, 2, 50, 0, "bf16"),
    ("window_64", 4, 1, 500, 500, 8, 1, 600, 64, "bf16"),
    ("g1_window_chunk", 5, 1, 129, 1000, 4, 4, 7, 100, "bf16"),
    ("g2_fp32", 6, 1, 77, 77, 6, 3, 13, 0, "fp32"),
    ("window_1", 7, 1, 96, 96, 8, 2, 16, 1, "bf16"),
    ("window_ge_L", 8, 1, 150, 150, 8, 2, 16, 150, "bf16"),
    ("g16", 9, 1, 64, 64, 32, 2, 20, 0, "bf16"),
    ("mtp_chunk", 10, 2, 9, 1000, 16, 2, 300, 0, "bf16"),
    ("batch_window_chunk", 11, 3, 100, 180, 8, 2, 40, 30, "bf16"),
    ("fp32_window_chunk", 12, 2, 65, 190, 4, 1, 70, 33, "fp32"),
]


@pytest.mark.parametrize("name,seed,B,Lq,Lk,Hq,Hkv,R,window,dtype", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_small(name, seed, B, Lq, Lk, Hq, Hkv, R, window, dtype):
    print(f"case {name}", flush=True)
    case = synth.make_prefill(seed, B, Lq, Lk, Hq, Hkv, R, window, dtype)
    out, lse = run_prefill(case)
    ref_o, ref_l, _ = oracle.ref_prefill(case.q, case.k, case.v, case.bias, window)
    compare(out, lse, ref_o, ref_l, name)


SPLIT_CASES = [
    # name, seed, B, Lq, Lk, Hq, Hkv, R, window, kv_splits
    ("split2_causal", 21, 1, 600, 1400, 16, 2, 700, 0, 2),
    ("split3_window", 22, 2, 500, 900, 8, 2, 300, 300, 3),
    ("split4_g4_ragged", 23, 1, 333, 2000, 8, 2, 2100, 0, 4),
    ("split8_g1", 24, 1, 130, 1500, 4, 4, 64, 0, 8),
]


@pytest.mark.parametrize("name,seed,B,Lq,Lk,Hq,Hkv,R,window,kv_splits", SPLIT_CASES,
                         ids=[c[0] for c in SPLIT_CASES])
def test_prefill_key_split(name, seed, B, Lq, Lk, Hq, Hkv, R, window, kv_splits):
    """Query tiles whose keys are split into pieces merged by log-sum-exp, against the oracle."""
    print(f"case {name}", flush=True)
    case = synth.make_prefill(seed, B, Lq, Lk, Hq, Hkv, R, window, "bf16")
    n = rb.rattn_prefill_workspace_bytes(B, Lq, Lk, Hq, Hkv, window, rb.RATTN_BF16, kv_splits)
    assert n > 0
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    q, k, v, r = dev(case.q), dev(case.k), dev(case.v), dev(case.bias)
    out, lse = rb.prefill(q, k, v, r, window, kv_splits=kv_splits, workspace=ws)
    torch.cuda.synchronize()
    ref_o, ref_l, _ = oracle.ref_prefill(case.q, case.k, case.v, case.bias, window)
    compare(host(out), host(lse), ref_o, ref_l, name)
    # the per-tile counters at the head of the workspace are back at zero
    assert int(ws[:256].count_nonzero()) == 0


def test_tiny_prefill_fp32_workload():
    case = synth.tiny_prefill_fp32()
    out, lse = run_prefill(case)
    ref_o, ref_l, _ = oracle.ref_prefill(case.q, case.k, case.v, case.bias, case.window)
    compare(out, lse, ref_o, ref_l, case.name)


@pytest.mark.parametrize("workload", ["swa_prefill_8k", "chunked_prefill_32k"])
def test_prefill_workload_full(workload):
    """The full-size workload in the launch configuration the benchmark times (the library's
    key-range split plan and job queue), every element against the oracle."""
    print(f"case {workload} (full output)", flush=True)
    case = synth.WORKLOAD_FNS[workload]()
    out, lse = run_prefill(case)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    ref_o, ref_l, _ = oracle.ref_prefill(case.q, case.k, case.v, case.bias, case.window)
    compare(out, lse, ref_o, ref_l, f"{workload} (all {case.Lq} rows x {case.Hq} heads)")


# ---------------------------------------------------------------------------------------
# paged decode
# ---------------------------------------------------------------------------------------
def run_decode(case, num_splits=0):
    d = decode_to_device(case)
    out, lse = rb.decode_paged(d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["ctx_lens"], d["windows"],
                               d["bias"], case.max_ctx_len, num_splits)
    torch.cuda.synchronize()
    return host(out), host(lse)


DECODE_CASES = [
    # name, seed, ctx_lens, windows, n_q, Hq, Hkv, R
    ("n1_edges", 21, [1, 127, 128, 129, 300, 1000], [0] * 6, 1, 16, 2, 64),
    ("n9_mixed", 22, [9, 130, 257, 2000], [0, 0, 100, 50], 9, 16, 2, 300),
    ("n3_g1", 23, [5, 600], [0, 7], 3, 8, 8, 40),
    ("n9_g8_unsat", 24, [5000, 777], [0, 0], 9, 64, 8, 8192),
    ("n9_g16_subgroups", 25, [400, 1300], [0, 129], 9, 32, 2, 200),
    ("n1_window1", 26, [250, 129], [1, 1], 1, 16, 2, 9),
    # 16 queries x 8 heads = 128 rows: four 32-row blocks, every wave of the 8-wave split computes
    ("n16_g8_rows128", 27, [200, 3000, 16], [0, 500, 0], 16, 16, 2, 300),
]


@pytest.mark.parametrize("name,seed,ctx,windows,n_q,Hq,Hkv,R", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_small(name, seed, ctx, windows, n_q, Hq, Hkv, R):
    print(f"case {name}", flush=True)
    case = synth.make_decode(seed, ctx, windows, n_q, Hq, Hkv, R)
    ref_o, ref_l, _ = oracle.ref_decode(case)
    # the KV stream is split among 256 (default), 1, 3, 7 or 5000 workgroups; 5000 exceeds
    # the number of 64-token units, so some workgroups get none
    for ns in (0, 1, 3, 7, 5000):
        out, lse = run_decode(case, ns)
        compare(out, lse, ref_o, ref_l, f"{name} splits={ns}")


def test_paged_decode_b64_workload():
    case = synth.paged_decode_b64()
    out, lse = run_decode(case)
    ref_o, ref_l, _ = oracle.ref_decode(case)
    compare(out, lse, ref_o, ref_l, case.name)


def test_mtp_verify_1m_workload():
    case = synth.mtp_verify_1m()
    out, lse = run_decode(case)
    ref_o, ref_l, _ = oracle.ref_decode(case)
    compare(out, lse, ref_o, ref_l, case.name)


def test_decode_batch_over_one_launch():
    """2100 sequences: the library runs launches of at most 2048 sequences, one after the
    other through the same workspace; every sequence still matches the oracle."""
    print("case decode 2100 sequences", flush=True)
    rng = np.random.default_rng(29)
    B = 2100
    ctx = rng.integers(1, 129, size=B).tolist()
    windows = [int(w) for w in np.where(np.arange(B) % 3 == 0, 40, 0)]
    case = synth.make_decode(29, ctx, windows, 1, 16, 2, 64)
    ref_o, ref_l, _ = oracle.ref_decode(case)
    for ns in (0, 7):
        out, lse = run_decode(case, ns)
        compare(out, lse, ref_o, ref_l, f"decode B=2100 splits={ns}")

