"""Properties of the HIP path that hold at any size, checked through the C ABI.

* Poisoned cache slots (NaN wherever no query can see) change nothing, bitwise.
* A different physical block layout of the same logical cache changes nothing, bitwise.
* The number of split workgroups only changes the summation order (tight tolerance).
* Decode of n_q queries equals the last n_q rows of a prefill over the same keys.
* A chunk of a prefill equals the same rows of the full-length prefill.
* With one-hot V rows the output is the attention weights: they match the oracle's
  probabilities and every row of weights sums to one.
* Repeated calls are bitwise identical.
* The prefill job queue changes nothing, bitwise, and is left at zero.
* Empty calls are no-ops that touch nothing.
"""
import numpy as np
import pytest

import oracle
from gpu_util import O_MAX_ABS, O_MEAN_ABS, compare, decode_to_device, dev, host
from relative_bias_gqa_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import relative_bias_gqa_amd as rb  # noqa: E402


def _decode(d, case, num_splits=0, k_cache=None, v_cache=None, block_table=None):
    out, lse = rb.decode_paged(d["q"], d["k_cache"] if k_cache is None else k_cache,
                               d["v_cache"] if v_cache is None else v_cache,
                               d["block_table"] if block_table is None else block_table, d["ctx_lens"],
                               d["windows"], d["bias"], case.max_ctx_len, num_splits)
    torch.cuda.synchronize()
    return out, lse


def _bitwise_equal(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def test_decode_poison_is_invisible():
    print("case decode poison", flush=True)
    case = synth.make_decode(41, [300, 1000, 129, 4000], [0, 100, 0, 700], 9, 16, 2, 256, poison=True)
    d = decode_to_device(case)
    out_p, lse_p = _decode(d, case)
    # the same cache with every poisoned slot replaced by zeros
    kc = case.k_cache.copy()
    vc = case.v_cache.copy()
    kc[np.isnan(synth.to_float(kc))] = 0
    vc[np.isnan(synth.to_float(vc))] = 0
    out_z, lse_z = _decode(d, case, k_cache=dev(kc), v_cache=dev(vc))
    assert torch.isfinite(out_p.float()).all()
    assert _bitwise_equal(out_p, out_z) and _bitwise_equal(lse_p, lse_z)


def test_decode_block_layout_is_invisible():
    print("case decode block layout", flush=True)
    case = synth.make_decode(42, [777, 2048, 3000], [0, 0, 1000], 1, 16, 2, 512, poison=False)
    d = decode_to_device(case)
    out_a, lse_a = _decode(d, case)
    # move every physical block to a new slot: new_id = perm[old_id]
    rng = np.random.default_rng(5)
    perm = rng.permutation(case.num_blocks)
    kc = np.empty_like(case.k_cache)
    vc = np.empty_like(case.v_cache)
    kc[perm] = case.k_cache
    vc[perm] = case.v_cache
    bt = perm[case.block_table].astype(np.int32)
    out_b, lse_b = _decode(d, case, k_cache=dev(kc), v_cache=dev(vc), block_table=dev(bt))
    assert _bitwise_equal(out_a, out_b) and _bitwise_equal(lse_a, lse_b)


def test_decode_split_count_only_reorders_sums():
    print("case decode split count", flush=True)
    case = synth.make_decode(43, [5000, 300, 12000], [0, 0, 4096], 9, 16, 2, 8192)
    d = decode_to_device(case)
    ref_o, ref_l = _decode(d, case, 1)
    for ns in (2, 5, 64, 256, 1000):
        o, l = _decode(d, case, ns)
        assert (o.float() - ref_o.float()).abs().max().item() <= 8e-3  # one bf16 ulp near 1
        assert (l - ref_l).abs().max().item() <= 1e-5


@pytest.mark.parametrize("n_q,window", [(1, 0), (9, 0), (9, 300), (1, 64)])
def test_decode_equals_last_prefill_rows(n_q, window):
    print(f"case decode vs prefill n_q={n_q} window={window}", flush=True)
    L, Hq, Hkv, R = 1500, 16, 2, 700
    pre = synth.make_prefill(44, 1, L, L, Hq, Hkv, R, window, "bf16")
    out_p, lse_p = rb.prefill(dev(pre.q), dev(pre.k), dev(pre.v), dev(pre.bias), window)
    # the same keys as a paged cache (identity block table), the last n_q tokens as queries
    nb = (L + 127) // 128
    kc = np.zeros((nb, 128, Hkv, 128), dtype=np.uint16)
    vc = np.zeros((nb, 128, Hkv, 128), dtype=np.uint16)
    kc.reshape(nb * 128, Hkv, 128)[:L] = pre.k[0]
    vc.reshape(nb * 128, Hkv, 128)[:L] = pre.v[0]
    bt = np.arange(nb, dtype=np.int32)[None]
    q = np.ascontiguousarray(pre.q[:, L - n_q:])
    out_d, lse_d = rb.decode_paged(dev(q), dev(kc), dev(vc), dev(bt), dev(np.array([L], np.int32)),
                                   dev(np.array([window], np.int32)), dev(pre.bias), L)
    torch.cuda.synchronize()
    diff = (out_d.float() - out_p[:, L - n_q:].float()).abs()
    assert diff.max().item() <= O_MAX_ABS and diff.mean().item() <= O_MEAN_ABS
    assert (lse_d - lse_p[:, L - n_q:]).abs().max().item() <= 1e-4


@pytest.mark.parametrize("window", [0, 200])
def test_chunk_equals_full_prefill(window):
    print(f"case chunk vs full window={window}", flush=True)
    L, Lq = 1100, 333
    case = synth.make_prefill(45, 2, L, L, 16, 2, 400, window, "bf16")
    q, k, v, r = dev(case.q), dev(case.k), dev(case.v), dev(case.bias)
    out_f, lse_f = rb.prefill(q, k, v, r, window)
    out_c, lse_c = rb.prefill(q[:, L - Lq:].contiguous(), k, v, r, window)
    torch.cuda.synchronize()
    diff = (out_c.float() - out_f[:, L - Lq:].float()).abs()
    assert diff.max().item() <= O_MAX_ABS and diff.mean().item() <= O_MEAN_ABS
    assert (lse_c - lse_f[:, L - Lq:]).abs().max().item() <= 1e-4


def test_key_split_only_reorders_sums():
    """Any key-range split of the query tiles gives the unsplit result up to summation order,
    and a split call repeated is bitwise identical (the merge runs in piece order whichever
    piece finishes last)."""
    print("case key split", flush=True)
    L, Hq, Hkv, R, W = 2000, 16, 2, 900, 700
    case = synth.make_prefill(50, 1, L, L, Hq, Hkv, R, W, "bf16")
    q, k, v, r = dev(case.q), dev(case.k), dev(case.v), dev(case.bias)
    ref_o, ref_l = rb.prefill(q, k, v, r, W, kv_splits=1)
    for ns in (0, 2, 3, 5, 8):
        n = rb.rattn_prefill_workspace_bytes(1, L, L, Hq, Hkv, W, rb.RATTN_BF16, ns)
        ws = torch.zeros(max(n, 1), dtype=torch.uint8, device="cuda")
        o1, l1 = rb.prefill(q, k, v, r, W, kv_splits=ns, workspace=ws)
        o2, l2 = rb.prefill(q, k, v, r, W, kv_splits=ns, workspace=ws)
        torch.cuda.synchronize()
        assert _bitwise_equal(o1, o2) and _bitwise_equal(l1, l2)
        assert (o1.float() - ref_o.float()).abs().max().item() <= 8e-3  # one bf16 ulp near 1
        assert (l1 - ref_l).abs().max().item() <= 1e-5
        # the job queue (first 256 bytes) and the per-tile counters after it are left at zero
        assert int(ws[:256 + 256 * 1024].count_nonzero()) == 0


@pytest.mark.parametrize("B,L,window", [(2, 4096, 0), (1, 6000, 1500)])
def test_job_queue_matches_one_workgroup_per_tile(B, L, window):
    """With a workspace the launch has one workgroup per compute unit taking query tiles
    from a queue (here more tiles than compute units); without one, one workgroup per tile.
    Unsplit, the two are the same bit for bit, and the queue is left at zero."""
    print(f"case job queue B={B} L={L} window={window}", flush=True)
    case = synth.make_prefill(51, B, L, L, 16, 2, 1000, window, "bf16")
    q, k, v, r = dev(case.q), dev(case.k), dev(case.v), dev(case.bias)
    lib = rb.load()
    outs = []
    for use_ws in (False, True):
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
        n = rb.rattn_prefill_workspace_bytes(B, L, L, 16, 2, window, rb.RATTN_BF16, 1)
        assert n == 256
        ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
        for _ in range(2):
            st = lib.rattn_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), r.data_ptr(), out.data_ptr(),
                                   lse.data_ptr(), B, L, L, 16, 2, 128, 1000, window, rb.RATTN_BF16, 1,
                                   ws.data_ptr() if use_ws else None, n if use_ws else 0, None)
            assert st == rb.RATTN_OK
        torch.cuda.synchronize()
        assert int(ws.count_nonzero()) == 0
        outs.append((out, lse))
    assert _bitwise_equal(outs[0][0], outs[1][0]) and _bitwise_equal(outs[0][1], outs[1][1])
    ref_o, ref_l = rb.prefill(q, k, v, r, window)  # the library's plan (maybe split), queued
    torch.cuda.synchronize()
    assert (ref_o.float() - outs[0][0].float()).abs().max().item() <= 8e-3
    assert (ref_l - outs[0][1]).abs().max().item() <= 1e-5


def test_workspace_shared_by_different_plans():
    """One workspace, zero-filled once, serves calls whose plans lay it out differently:
    each call's result equals its own-workspace result, bit for bit."""
    print("case shared workspace", flush=True)
    shapes = [(1, 2000, 2000, 700, 2), (1, 600, 1400, 0, 3), (2, 900, 900, 300, 0), (1, 3000, 3000, 1000, 4)]
    cases = [synth.make_prefill(60 + i, B, Lq, Lk, 16, 2, 800, W, "bf16") for i, (B, Lq, Lk, W, _) in enumerate(shapes)]
    big = max(rb.rattn_prefill_workspace_bytes(B, Lq, Lk, 16, 2, W, rb.RATTN_BF16, ns) for (B, Lq, Lk, W, ns) in shapes)
    shared = torch.zeros(big, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        for c, (B, Lq, Lk, W, ns) in zip(cases, shapes):
            q, k, v, r = dev(c.q), dev(c.k), dev(c.v), dev(c.bias)
            n = rb.rattn_prefill_workspace_bytes(B, Lq, Lk, 16, 2, W, rb.RATTN_BF16, ns)
            own = torch.zeros(n, dtype=torch.uint8, device="cuda")
            o1, l1 = rb.prefill(q, k, v, r, W, kv_splits=ns, workspace=own)
            o2, l2 = rb.prefill(q, k, v, r, W, kv_splits=ns, workspace=shared)
            torch.cuda.synchronize()
            assert _bitwise_equal(o1, o2) and _bitwise_equal(l1, l2)
    assert int(shared[:256 + 256 * 1024].count_nonzero()) == 0


def test_one_hot_values_expose_the_weights():
    print("case one-hot V", flush=True)
    # 256 keys, one KV head: two runs with V_j = e_j (j < 128) and V_j = e_(j-128) (j >= 128)
    L, Hq, R, window = 256, 4, 100, 0
    case = synth.make_prefill(46, 1, L, L, Hq, 1, R, window, "bf16")
    eye = np.zeros((1, L, 1, 128), dtype=np.float32)
    eye2 = np.zeros((1, L, 1, 128), dtype=np.float32)
    for j in range(L):
        (eye if j < 128 else eye2)[0, j, 0, j % 128] = 1.0
    w = np.zeros((1, L, Hq, L))
    for half, vv in enumerate((eye, eye2)):
        out, _ = rb.prefill(dev(case.q), dev(case.k), dev(synth.bf16_round(vv)), dev(case.bias), window)
        torch.cuda.synchronize()
        w[..., 128 * half:128 * (half + 1)] = host(out)
    _, _, probs = oracle.ref_prefill(case.q, case.k, case.v, case.bias, window, want_probs=True)
    err = np.abs(w - probs)
    print(f"weights: max err {err.max():.3e}, mean {err.mean():.3e}", flush=True)
    assert err.max() <= O_MAX_ABS and err.mean() <= O_MEAN_ABS
    # every row of weights sums to one (bf16 outputs: 256 terms, each within 2^-9 relative)
    np.testing.assert_allclose(w.sum(-1), 1.0, atol=1e-2)
    # and no weight falls on an invisible (future) key
    for t in range(L):
        assert np.all(w[0, t, :, t + 1:] == 0)


def test_repeated_calls_are_bitwise_identical():
    print("case determinism", flush=True)
    pre = synth.make_prefill(47, 1, 700, 900, 16, 2, 500, 256, "bf16")
    q, k, v, r = dev(pre.q), dev(pre.k), dev(pre.v), dev(pre.bias)
    first = rb.prefill(q, k, v, r, 256)
    for _ in range(3):
        again = rb.prefill(q, k, v, r, 256)
        torch.cuda.synchronize()
        assert _bitwise_equal(first[0], again[0]) and _bitwise_equal(first[1], again[1])
    case = synth.make_decode(48, [3000, 700], [0, 512], 9, 16, 2, 1000)
    d = decode_to_device(case)
    first = _decode(d, case)
    for _ in range(3):
        again = _decode(d, case)
        assert _bitwise_equal(first[0], again[0]) and _bitwise_equal(first[1], again[1])


def test_empty_calls_are_noops():
    print("case empty", flush=True)
    lib = rb.load()
    sentinel = torch.full((4,), 7.0, device="cuda")
    # B = 0 and Lq = 0 prefill, B = 0 decode: status OK, nothing written
    assert lib.rattn_prefill(None, None, None, None, None, sentinel.data_ptr(), 0, 5, 5, 4, 1, 128, 8, 0, 0, 0,
                             None, 0, None) == rb.RATTN_OK
    assert lib.rattn_prefill(None, None, None, None, None, sentinel.data_ptr(), 1, 0, 5, 4, 1, 128, 8, 0, 0, 0,
                             None, 0, None) == rb.RATTN_OK
    assert lib.rattn_decode_paged(None, None, None, None, None, None, None, None, sentinel.data_ptr(), 0, 1, 16,
                                  2, 128, 128, 8, 4, 2, 200, 0, None, 0, None) == rb.RATTN_OK
    torch.cuda.synchronize()
    assert torch.all(sentinel == 7.0)


def test_window_one_and_single_bias_entry():
    """Degenerate shapes: a window of one key (out = v_i) and a one-entry bias table."""
    print("case degenerate", flush=True)
    case = synth.make_prefill(49, 1, 300, 300, 8, 2, 1, 1, "bf16")
    out, lse = rb.prefill(dev(case.q), dev(case.k), dev(case.v), dev(case.bias), 1)
    torch.cuda.synchronize()
    v = synth.to_float(case.v).astype(np.float64)
    np.testing.assert_array_equal(host(out), np.repeat(v, 4, axis=2))  # bf16 round trip is exact
    ref_o, ref_l, _ = oracle.ref_prefill(case.q, case.k, case.v, case.bias, 1)
    compare(host(out), host(lse), ref_o, ref_l, "window 1, R 1")
