"""The allocation-free paged decode (rattn_decode_paged_noalloc) through the C ABI.

Two calls in a row on one stream, the second with a smaller input (fewer sequences, one
query instead of nine, shorter contexts), so the second call runs on scratch that still
holds the first call's partials.  Each is compared with the allocating entry point
rattn_decode_paged on the same inputs (same kernels and split plan: bit-identical output
and lse) and with the fp64 oracle at the parity bar (O max abs <= 2e-2, mean <= 2e-3,
lse max abs <= 1e-3).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import compare, decode_to_device, host

import relative_bias_gqa_amd as rb
from relative_bias_gqa_amd import synth

pytestmark = pytest.mark.gpu


def _both(case):
    d = decode_to_device(case)
    B, n_q, Hq, _ = case.q.shape
    outs = []
    for noalloc in (True, False):
        out = torch.empty_like(d["q"])
        lse = torch.empty((B, n_q, Hq), dtype=torch.float32, device="cuda")
        if noalloc:
            rb.rattn_decode_paged_noalloc(d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["ctx_lens"],
                                          d["windows"], d["bias"], out, lse, case.max_ctx_len)
        else:
            ws = rb.decode_workspace(B, n_q, Hq, case.k_cache.shape[2], case.max_ctx_len, 0, "cuda")
            rb.rattn_decode_paged(d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["ctx_lens"], d["windows"],
                                  d["bias"], out, lse, case.max_ctx_len, 0, ws)
        torch.cuda.synchronize()
        outs.append((out, lse))
    return outs


def test_noalloc_decode_two_calls():
    first = synth.make_decode(61, [9000, 130, 4100], [0, 0, 4096], 9, 16, 2, 8192, "noalloc_first")
    second = synth.make_decode(62, [700, 64], [0, 50], 1, 16, 2, 300, "noalloc_second")
    for case in (first, second):
        print(f"case {case.name}: B={case.q.shape[0]} n_q={case.q.shape[1]} ctx={list(case.ctx_lens)}", flush=True)
        (o_s, l_s), (o_w, l_w) = _both(case)
        assert torch.equal(o_s.view(torch.int16), o_w.view(torch.int16)), f"{case.name}: output differs"
        assert torch.equal(l_s, l_w), f"{case.name}: lse differs"
        ref_o, ref_l, _ = oracle.ref_decode(case)
        compare(host(o_s), host(l_s), ref_o, ref_l, f"{case.name} (no-alloc)")


def test_noalloc_decode_workload_then_smaller():
    """The batch-64 decode workload, then a single short sequence."""
    big = synth.paged_decode_b64()
    small = synth.make_decode(63, [333], [0], 1, 16, 2, 8192, "noalloc_small")
    for case in (big, small):
        print(f"case {case.name}", flush=True)
        (o_s, l_s), (o_w, l_w) = _both(case)
        assert torch.equal(o_s.view(torch.int16), o_w.view(torch.int16)), f"{case.name}: output differs"
        assert torch.equal(l_s, l_w), f"{case.name}: lse differs"
        ref_o, ref_l, _ = oracle.ref_decode(case)
        compare(host(o_s), host(l_s), ref_o, ref_l, f"{case.name} (no-alloc)")
