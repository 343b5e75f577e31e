"""The key/value short convolution written into the paged caches (rattn_kv_sconv_write) on
the GPU, against the fp64 oracle (oracle/sconv.py): conv outputs within one bf16 unit in the
last place of the exact value plus the fp32 accumulation error of four terms (bounded by
2^-20 times the sum of the terms' magnitudes, which the oracle gives when run on absolute
values: where the terms cancel that is what dominates), the raw state rows bit for bit,
every other slot untouched; fresh sequences, chunks after a prefix (the taps reaching into the
state cache), chunks of 0, 1 and 2 tokens, several blocks per chunk, 1, 2 and 8 KV heads;
and a sequence written in chunks equals one call, bitwise."""
import numpy as np
import pytest
import torch

from gpu_util import dev

from oracle import sconv

pytestmark = pytest.mark.gpu

import relative_bias_gqa_amd as rb  # noqa: E402

BLOCK = 128


def _bf16(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _case(seed, ctx, n_new, Hkv):
    rng = np.random.default_rng(seed)
    B = len(ctx)
    nbps = max((c + BLOCK - 1) // BLOCK for c in ctx)
    nb = B * nbps
    bt = rng.permutation(nb).reshape(B, nbps).astype(np.int32)
    shape = (nb, BLOCK, Hkv, 128)
    caches = [_bf16(rng, shape) for _ in range(4)]
    T = sum(n_new)
    k_new, v_new = _bf16(rng, (max(T, 1), Hkv, 128))[:T], _bf16(rng, (max(T, 1), Hkv, 128))[:T]
    w_k = rng.standard_normal((4, Hkv, 128)).astype(np.float32)
    w_v = rng.standard_normal((4, Hkv, 128)).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
    return dict(k_new=k_new, v_new=v_new, w_k=w_k, w_v=w_v, caches=caches, bt=bt, ctx=np.asarray(ctx, np.int32),
                cu=cu, max_new=max(n_new))


def _run_gpu(c, caches=None, k_new=None, v_new=None, ctx=None, cu=None, max_new=None):
    caches = [dev(x) for x in (caches or c["caches"])]
    kn = dev(c["k_new"] if k_new is None else k_new)
    vn = dev(c["v_new"] if v_new is None else v_new)
    rb.rattn_kv_sconv_write(kn, vn, dev(c["w_k"]), dev(c["w_v"]), *caches, dev(c["bt"]),
                            dev(c["ctx"] if ctx is None else ctx), dev(c["cu"] if cu is None else cu),
                            c["max_new"] if max_new is None else max_new)
    torch.cuda.synchronize()
    return [x.view(torch.int16).cpu().numpy().view(np.uint16) for x in caches]


CASES = [
    # name, seed, ctx (after the write), new tokens, Hkv
    ("mixed", 81, [300, 2, 900, 1, 129, 700], [300, 2, 200, 1, 0, 65], 2),
    ("one_head", 82, [500, 260], [130, 260], 1),
    ("eight_heads", 83, [400, 3], [70, 2], 8),
]


@pytest.mark.parametrize("name,seed,ctx,n_new,Hkv", CASES, ids=[c[0] for c in CASES])
def test_sconv_write_matches_oracle(name, seed, ctx, n_new, Hkv):
    print(f"case sconv {name}", flush=True)
    c = _case(seed, ctx, n_new, Hkv)
    got = _run_gpu(c)
    ok, ov, oks, ovs, yk, yv = sconv.sconv_write(c["k_new"], c["v_new"], c["w_k"], c["w_v"], *c["caches"], c["bt"],
                                                 c["ctx"], c["cu"])
    # state caches and untouched slots: bit for bit
    assert np.array_equal(got[2], oks) and np.array_equal(got[3], ovs)
    written = np.zeros(c["caches"][0].shape[:2], dtype=bool)
    for b in range(len(ctx)):
        for p in range(ctx[b] - n_new[b], ctx[b]):
            written[c["bt"][b, p // BLOCK], p % BLOCK] = True
    for g, before in zip(got[:2], c["caches"][:2]):
        assert np.array_equal(g[~written], before[~written])
    # conv outputs: within one bf16 ulp of the fp64 value plus 2^-20 sum |w x|
    mag = lambda x: x & np.uint16(0x7FFF)
    *_, ak, av = sconv.sconv_write(mag(c["k_new"]), mag(c["v_new"]), np.abs(c["w_k"]), np.abs(c["w_v"]),
                                   *[mag(x) for x in c["caches"]], c["bt"], c["ctx"], c["cu"])
    worst = 0.0
    for g, y, a in ((got[0], yk, ak), (got[1], yv, av)):
        for b in range(len(ctx)):
            for t in range(n_new[b]):
                p = ctx[b] - n_new[b] + t
                gv = sconv.bf16_to_f64(g[c["bt"][b, p // BLOCK], p % BLOCK])
                yy, aa = y[c["cu"][b] + t], a[c["cu"][b] + t]
                ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(yy), 1e-30))) - 7)
                worst = max(worst, float((np.abs(gv - yy) / (ulp + 2.0 ** -20 * aa)).max()))
    print(f"sconv {name}: worst error {worst:.3f} of the bound", flush=True)
    assert worst <= 1.0


def test_sconv_chunks_equal_one_call():
    print("case sconv chunks", flush=True)
    total = 390
    c = _case(84, [total], [total], 2)
    one = _run_gpu(c)
    caches = c["caches"]
    pos = 0
    for n in (130, 1, 259):
        caches = _run_gpu(c, caches=caches, k_new=c["k_new"][pos:pos + n], v_new=c["v_new"][pos:pos + n],
                          ctx=np.array([pos + n], np.int32), cu=np.array([0, n], np.int32), max_new=n)
        pos += n
    for a, b in zip(one, caches):
        assert np.array_equal(a, b)
