"""Pins of the short-convolution oracle (oracle/sconv.py) on the CPU, against what the
definition and library routines fix independently of it: single-tap weights reduce to a copy
and a one-token shift, a fresh sequence equals numpy.convolve per channel, splitting a
sequence into chunks (the state carried through the state cache) equals one call, the
rounding equals torch's float32 -> bfloat16 conversion, and the block table is honoured."""
import numpy as np
import pytest
import torch

from oracle import sconv

BLOCK = 128


def _bf16(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    return (torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def _setup(rng, ctx, n_new, Hkv=2, perm=True):
    """Caches with random raw state for the prefix and random garbage elsewhere, a block table
    (a random permutation of the blocks), packed new tokens."""
    B = len(ctx)
    nbps = max((c + BLOCK - 1) // BLOCK for c in ctx)
    nb = B * nbps
    ids = rng.permutation(nb) if perm else np.arange(nb)
    bt = ids.reshape(B, nbps).astype(np.int32)
    shape = (nb, BLOCK, Hkv, 128)
    kc, vc, ks, vs = (_bf16(rng, shape) for _ in range(4))
    T = sum(n_new)
    k_new, v_new = _bf16(rng, (T, Hkv, 128)), _bf16(rng, (T, Hkv, 128))
    cu = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
    return kc, vc, ks, vs, bt, np.asarray(ctx, dtype=np.int32), cu, k_new, v_new


def _weights(rng, Hkv=2):
    return rng.standard_normal((4, Hkv, 128)), rng.standard_normal((4, Hkv, 128))


def test_rounding_matches_torch_bf16():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(sconv.f64_to_bf16(x.astype(np.float64)), ref)
    # exact halfway cases round to even
    halves = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8)], dtype=np.float64)
    assert list(sconv.bf16_to_f64(sconv.f64_to_bf16(halves))) == [1.0, 1.0 + 2 ** -6, -1.0]


@pytest.mark.parametrize("tap", [0, 1, 3])
def test_single_tap_is_a_shift(tap):
    """w[s] = 1 for s = tap, else 0: y[p] = x[p - tap], from the chunk or the state cache, or
    zero before position 0; bf16 values pass through exactly."""
    rng = np.random.default_rng(1 + tap)
    ctx, n_new = [300, 5, 200], [50, 5, 1]
    kc, vc, ks, vs, bt, ctx, cu, k_new, v_new = _setup(rng, ctx, n_new)
    w = np.zeros((4, 2, 128))
    w[tap] = 1.0
    ok, ov, oks, ovs, yk, yv = sconv.sconv_write(k_new, v_new, w, w, kc, vc, ks, vs, bt, ctx, cu)
    for b in range(len(ctx)):
        start = ctx[b] - n_new[b]
        for t in range(n_new[b]):
            p, src = start + t, start + t - tap
            if src < 0:
                want = np.zeros((2, 128), dtype=np.uint16)
            elif src >= start:
                want = k_new[cu[b] + src - start]
            else:
                want = ks[bt[b, src // BLOCK], src % BLOCK]
            got = ok[bt[b, p // BLOCK], p % BLOCK]
            assert np.array_equal(sconv.bf16_to_f64(got), sconv.bf16_to_f64(want)), (b, t)
            assert np.array_equal(oks[bt[b, p // BLOCK], p % BLOCK], k_new[cu[b] + t])


def test_fresh_sequence_equals_numpy_convolve():
    rng = np.random.default_rng(7)
    n = 260
    kc, vc, ks, vs, bt, ctx, cu, k_new, v_new = _setup(rng, [n], [n])
    wk, wv = _weights(rng)
    _, _, _, _, yk, yv = sconv.sconv_write(k_new, v_new, wk, wv, kc, vc, ks, vs, bt, ctx, cu)
    xk, xv = sconv.bf16_to_f64(k_new), sconv.bf16_to_f64(v_new)
    for h in range(2):
        for c in range(0, 128, 7):
            np.testing.assert_allclose(yk[:, h, c], np.convolve(xk[:, h, c], wk[:, h, c])[:n], rtol=0, atol=1e-12)
            np.testing.assert_allclose(yv[:, h, c], np.convolve(xv[:, h, c], wv[:, h, c])[:n], rtol=0, atol=1e-12)


def test_chunks_equal_one_call():
    """A sequence written in three chunks (the raw state carried by the state cache) leaves
    the same caches as one call over all its tokens."""
    rng = np.random.default_rng(11)
    total = 390
    kc, vc, ks, vs, bt, _, _, k_all, v_all = _setup(rng, [total], [total])
    wk, wv = _weights(rng)
    one = sconv.sconv_write(k_all, v_all, wk, wv, kc, vc, ks, vs, bt, np.array([total], np.int32),
                            np.array([0, total], np.int32))
    caches = (kc, vc, ks, vs)
    pos = 0
    for n in (130, 1, 259):
        caches = sconv.sconv_write(k_all[pos:pos + n], v_all[pos:pos + n], wk, wv, *caches, bt,
                                   np.array([pos + n], np.int32), np.array([0, n], np.int32))[:4]
        pos += n
    for a, b in zip(one[:4], caches):
        assert np.array_equal(a, b)


def test_untouched_slots_and_block_table():
    """Only the new positions change, at the physical blocks the table names."""
    rng = np.random.default_rng(13)
    ctx, n_new = [700, 129], [200, 129]
    kc, vc, ks, vs, bt, ctx, cu, k_new, v_new = _setup(rng, ctx, n_new)
    wk, wv = _weights(rng)
    ok, ov, oks, ovs, _, _ = sconv.sconv_write(k_new, v_new, wk, wv, kc, vc, ks, vs, bt, ctx, cu)
    changed = np.zeros(kc.shape[:2], dtype=bool)
    for b in range(2):
        for p in range(ctx[b] - n_new[b], ctx[b]):
            changed[bt[b, p // BLOCK], p % BLOCK] = True
    for before, after in ((kc, ok), (vc, ov), (ks, oks), (vs, ovs)):
        assert np.array_equal(before[~changed], after[~changed])
