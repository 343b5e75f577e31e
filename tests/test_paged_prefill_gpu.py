"""Chunked prefill over a paged KV cache (rattn_prefill_paged) on the GPU.

* Parity with the fp64 oracle, which reads the same paged cache through the block table and
  places query t of sequence b at ctx_lens[b] - Lq + t (the decode formula with n_q = Lq):
  ragged chunks and contexts, windows (W = 1 included), one and sixteen query heads per KV
  head, a 1024-token chunk; invisible slots and blocks hold NaN.
* Through a permuted block table it equals the contiguous prefill of the same keys, bitwise.
* NaN in the slots before the first query's window changes nothing, bitwise.
* The job queue (with a workspace, sequences taken longest context first) gives the same
  bits as one workgroup per job, and is left at zero.
* Packed queries of different lengths per sequence (cu_seqlens_q; none, one, ragged and the
  longest chunk) match the oracle's rows for the same positions.
"""
import numpy as np
import pytest
import torch

from gpu_util import compare, decode_to_device, dev, host

import oracle
import relative_bias_gqa_amd as rb
from relative_bias_gqa_amd import synth

pytestmark = pytest.mark.gpu


def _bitwise_equal(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def run_paged(case, window, k_cache=None, v_cache=None):
    d = decode_to_device(case)
    out, lse = rb.prefill_paged(d["q"], d["k_cache"] if k_cache is None else k_cache,
                                d["v_cache"] if v_cache is None else v_cache, d["block_table"], d["ctx_lens"],
                                d["bias"], case.max_ctx_len, window)
    torch.cuda.synchronize()
    return out, lse


CASES = [
    # name, seed, ctx_lens, Lq, window, Hq, Hkv, R
    ("ragged_full", 61, [300, 1000, 777], 200, 0, 16, 2, 256),
    ("window", 62, [2000, 650, 4100], 300, 300, 16, 2, 1000),
    ("no_prefix_g1", 63, [257, 64], 64, 0, 8, 8, 40),
    ("g16_subgroups", 64, [1500, 900], 129, 0, 32, 2, 200),
    ("window_one", 65, [300, 130], 100, 1, 16, 2, 9),
    ("chunk_1024", 66, [4096, 3000, 5000], 1024, 2048, 16, 2, 2048),
]


@pytest.mark.parametrize("name,seed,ctx,Lq,window,Hq,Hkv,R", CASES, ids=[c[0] for c in CASES])
def test_paged_prefill_matches_oracle(name, seed, ctx, Lq, window, Hq, Hkv, R):
    print(f"case paged prefill {name}", flush=True)
    case = synth.make_decode(seed, ctx, [window] * len(ctx), Lq, Hq, Hkv, R, name=name)
    out, lse = run_paged(case, window)
    ref_o, ref_l, _ = oracle.ref_decode(case)
    compare(host(out), host(lse), ref_o, ref_l, name)


@pytest.mark.parametrize("window", [0, 300])
def test_paged_prefill_equals_contiguous_prefill(window):
    """The same keys as a contiguous [B, Lk, Hkv, 128] tensor and as 128-token blocks placed by a
    random permutation: the paged call reproduces the contiguous call (no workspace: one
    workgroup per tile, the same tiles in the same order) bit for bit."""
    print(f"case paged vs contiguous window={window}", flush=True)
    B, Lq, Lk, Hq, Hkv, R = 2, 300, 1000, 16, 2, 600
    pre = synth.make_prefill(71, B, Lq, Lk, Hq, Hkv, R, window, "bf16")
    q, k, v, r = dev(pre.q), dev(pre.k), dev(pre.v), dev(pre.bias)
    out_c = torch.empty_like(q)
    lse_c = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    rb.rattn_prefill(q, k, v, r, out_c, lse_c, window, 0, None)
    nbps = (Lk + 127) // 128
    perm = np.random.default_rng(72).permutation(B * nbps)
    kc = np.zeros((B * nbps, 128, Hkv, 128), dtype=np.uint16)  # slots past Lk stay zero
    vc = np.zeros_like(kc)
    bt = np.empty((B, nbps), dtype=np.int32)
    for b in range(B):
        for blk in range(nbps):
            phys = perm[b * nbps + blk]
            bt[b, blk] = phys
            n = min(128, Lk - 128 * blk)
            kc[phys, :n] = pre.k[b, 128 * blk:128 * blk + n]
            vc[phys, :n] = pre.v[b, 128 * blk:128 * blk + n]
    ctx = torch.full((B,), Lk, dtype=torch.int32, device=q.device)
    out_p, lse_p = rb.prefill_paged(q, dev(kc), dev(vc), dev(bt), ctx, r, Lk, window)
    torch.cuda.synchronize()
    assert _bitwise_equal(out_c, out_p) and _bitwise_equal(lse_c, lse_p)


def test_paged_prefill_poison_before_window_is_invisible():
    print("case paged prefill poison before window", flush=True)
    Lq, window = 300, 300
    case = synth.make_decode(62, [2000, 650, 4100], [window] * 3, Lq, 16, 2, 1000, name="window")
    out_a, lse_a = run_paged(case, window)
    # NaN in every resident slot before the first visible key of each sequence
    kc, vc = case.k_cache.copy(), case.v_cache.copy()
    nan16 = np.uint16(0x7FC0)
    for b, c in enumerate(case.ctx_lens):
        vis_lo = max(0, int(c) - Lq - window + 1)
        for j in range((vis_lo // 128) * 128, vis_lo):
            kc[case.block_table[b, j // 128], j % 128] = nan16
            vc[case.block_table[b, j // 128], j % 128] = nan16
    out_b, lse_b = run_paged(case, window, k_cache=dev(kc), v_cache=dev(vc))
    assert torch.isfinite(out_b.float()).all()
    assert _bitwise_equal(out_a, out_b) and _bitwise_equal(lse_a, lse_b)


def test_paged_prefill_job_queue_matches_one_workgroup_per_job():
    print("case paged prefill job queue", flush=True)
    Lq = 256
    case = synth.make_decode(67, [700, 5000, 256, 3000, 1200], [0] * 5, Lq, 16, 2, 4096, name="queue")
    d = decode_to_device(case)
    args = (d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["ctx_lens"], d["bias"], case.max_ctx_len, 0)
    out_n, lse_n = rb.prefill_paged(*args, workspace=None)
    ws = torch.zeros(rb.PREFILL_PAGED_WORKSPACE_BYTES, dtype=torch.uint8, device=d["q"].device)
    for _ in range(3):
        out_q, lse_q = rb.prefill_paged(*args, workspace=ws)
        torch.cuda.synchronize()
        assert _bitwise_equal(out_n, out_q) and _bitwise_equal(lse_n, lse_q)
        assert int(ws.sum().item()) == 0
    ref_o, ref_l, _ = oracle.ref_decode(case)
    compare(host(out_q), host(lse_q), ref_o, ref_l, "queue")


@pytest.mark.parametrize("window", [0, 200])
def test_paged_prefill_packed_varlen_queries(window):
    """Sequence b's chunk is its last n_b queries: the last n_b rows of a fixed-length case at the
    same context (same positions ctx - n_b + t), so the oracle of that case gives the expected rows."""
    print(f"case paged prefill packed varlen window={window}", flush=True)
    max_q = 300
    ctx = [1000, 300, 2500, 700, 1500]
    qlens = [300, 0, 1, 129, 77]
    case = synth.make_decode(68, ctx, [window] * len(ctx), max_q, 16, 2, 1500, name="varlen")
    ref_o, ref_l, _ = oracle.ref_decode(case)
    d = decode_to_device(case)
    qp = np.ascontiguousarray(np.concatenate([case.q[b, max_q - n:] for b, n in enumerate(qlens)], axis=0))
    cu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    out, lse = rb.prefill_paged(dev(qp), d["k_cache"], d["v_cache"], d["block_table"], d["ctx_lens"], d["bias"],
                                case.max_ctx_len, window, cu_seqlens_q=dev(cu), max_q_len=max_q)
    torch.cuda.synchronize()
    exp_o = np.concatenate([ref_o[b, max_q - n:] for b, n in enumerate(qlens)], axis=0)
    exp_l = np.concatenate([ref_l[b, max_q - n:] for b, n in enumerate(qlens)], axis=0)
    compare(host(out), host(lse), exp_o, exp_l, f"varlen window={window}")


def test_paged_prefill_many_sequences():
    """More sequences than the workgroups rank by context length (1024): jobs go in sequence
    order; with and without the job queue the result is the same bit for bit and matches the
    oracle."""
    print("case paged prefill 1100 sequences", flush=True)
    rng = np.random.default_rng(69)
    B, Lq = 1100, 8
    ctx = rng.integers(Lq, 200, size=B).tolist()
    case = synth.make_decode(69, ctx, [0] * B, Lq, 16, 2, 64, name="many")
    d = decode_to_device(case)
    args = (d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["ctx_lens"], d["bias"], case.max_ctx_len, 0)
    out_q, lse_q = rb.prefill_paged(*args)
    out_n, lse_n = rb.prefill_paged(*args, workspace=None)
    torch.cuda.synchronize()
    assert _bitwise_equal(out_q, out_n) and _bitwise_equal(lse_q, lse_n)
    ref_o, ref_l, _ = oracle.ref_decode(case)
    compare(host(out_q), host(lse_q), ref_o, ref_l, "many sequences")

