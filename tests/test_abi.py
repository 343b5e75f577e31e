"""The C-ABI library on the CPU: it loads, exports what include/rattn.h declares, and
rejects bad arguments with the documented status before touching a device."""
import ctypes
import os
import re

import pytest

import relative_bias_gqa_amd as rb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rattn.h")

FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation or is a no-op


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(rb.LIB_PATH):
        rb_build = __import__("relative_bias_gqa_amd.build", fromlist=["build"])
        rb_build.build()
    return rb.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rattn_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(rb.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version(lib):
    assert lib.rattn_abi_version() == rb.ABI_VERSION == 9


def _prefill(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bias=FAKE, out=FAKE, lse=None, B=1, Lq=4, Lk=4, Hq=4, Hkv=2, D=128, R=8,
             window=0, dtype=0, kv_splits=0, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.rattn_prefill(a["q"], a["k"], a["v"], a["bias"], a["out"], a["lse"], a["B"], a["Lq"], a["Lk"],
                             a["Hq"], a["Hkv"], a["D"], a["R"], a["window"], a["dtype"], a["kv_splits"], a["ws"],
                             a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), rb.RATTN_ERR_INVALID_ARG, "null"),
    (dict(bias=None), rb.RATTN_ERR_INVALID_ARG, "null"),
    (dict(out=None), rb.RATTN_ERR_INVALID_ARG, "null"),
    (dict(Hq=6, Hkv=4), rb.RATTN_ERR_INVALID_ARG, "multiple"),
    (dict(Hkv=0), rb.RATTN_ERR_INVALID_ARG, "multiple"),
    (dict(Lq=5, Lk=4), rb.RATTN_ERR_INVALID_ARG, "Lq"),
    (dict(R=0), rb.RATTN_ERR_INVALID_ARG, "R="),
    (dict(B=-1), rb.RATTN_ERR_INVALID_ARG, "negative"),
    (dict(D=64), rb.RATTN_ERR_UNSUPPORTED, "head_dim"),
    (dict(dtype=7), rb.RATTN_ERR_UNSUPPORTED, "dtype"),
    (dict(kv_splits=9), rb.RATTN_ERR_INVALID_ARG, "kv_splits"),
    (dict(kv_splits=-1), rb.RATTN_ERR_INVALID_ARG, "kv_splits"),
    (dict(wsb=64), rb.RATTN_ERR_INVALID_ARG, "workspace"),
    (dict(Lq=4096, Lk=4096, kv_splits=2, ws=FAKE, wsb=64), rb.RATTN_ERR_WORKSPACE, "workspace"),
])
def test_prefill_validation(lib, kw, status, needle):
    assert _prefill(lib, **kw) == status
    assert needle in rb.rattn_last_error()


def test_prefill_empty_is_noop(lib):
    assert _prefill(lib, B=0, q=None, k=None, v=None, bias=None, out=None) == rb.RATTN_OK
    assert _prefill(lib, Lq=0, q=None, out=None) == rb.RATTN_OK
    assert rb.rattn_last_error() == ""


def _decode(lib, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, ctx=FAKE, win=None, bias=FAKE, out=FAKE, lse=None, B=2, n_q=1,
             Hq=16, Hkv=2, D=128, bs=128, R=8, nb=4, mb=2, max_ctx=200, ns=0, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.rattn_decode_paged(a["q"], a["kc"], a["vc"], a["bt"], a["ctx"], a["win"], a["bias"], a["out"],
                                  a["lse"], a["B"], a["n_q"], a["Hq"], a["Hkv"], a["D"], a["bs"], a["R"], a["nb"],
                                  a["mb"], a["max_ctx"], a["ns"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), rb.RATTN_ERR_INVALID_ARG, "null"),
    (dict(bt=None), rb.RATTN_ERR_INVALID_ARG, "null"),
    (dict(ctx=None), rb.RATTN_ERR_INVALID_ARG, "null"),
    (dict(Hq=15), rb.RATTN_ERR_INVALID_ARG, "multiple"),
    (dict(n_q=0), rb.RATTN_ERR_INVALID_ARG, "n_q"),
    (dict(R=0), rb.RATTN_ERR_INVALID_ARG, "R="),
    (dict(nb=0), rb.RATTN_ERR_INVALID_ARG, "num_blocks"),
    (dict(max_ctx=0), rb.RATTN_ERR_INVALID_ARG, "max_ctx_len"),
    (dict(max_ctx=257, mb=2), rb.RATTN_ERR_INVALID_ARG, "block table"),
    (dict(D=96), rb.RATTN_ERR_UNSUPPORTED, "head_dim"),
    (dict(bs=16), rb.RATTN_ERR_UNSUPPORTED, "block_size"),
    (dict(n_q=129, max_ctx=256), rb.RATTN_ERR_UNSUPPORTED, "n_q"),
    (dict(ws=None), rb.RATTN_ERR_WORKSPACE, "workspace"),
    (dict(wsb=16), rb.RATTN_ERR_WORKSPACE, "workspace"),
])
def test_decode_validation(lib, kw, status, needle):
    assert _decode(lib, **kw) == status
    assert needle in rb.rattn_last_error()


def _prefill_tok(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, rt=FAKE, out=FAKE, lse=None, B=1, Lq=100, Lk=100, Hq=16, Hkv=2, D=128, R=64,
             window=0, ks=0, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.rattn_prefill_tokbias(a["q"], a["k"], a["v"], a["rt"], a["out"], a["lse"], a["B"], a["Lq"], a["Lk"],
                                     a["Hq"], a["Hkv"], a["D"], a["R"], a["window"], a["ks"], a["ws"], a["wsb"],
                                     a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(rt=None), rb.RATTN_ERR_INVALID_ARG, "null"),
    (dict(q=None), rb.RATTN_ERR_INVALID_ARG, "null"),
    (dict(R=3), rb.RATTN_ERR_UNSUPPORTED, "R >= 4"),
    (dict(R=0), rb.RATTN_ERR_INVALID_ARG, "R="),
    (dict(rt=ctypes.c_void_p(0x1002)), rb.RATTN_ERR_INVALID_ARG, "aligned"),
    (dict(Lq=101), rb.RATTN_ERR_INVALID_ARG, "Lq="),
    (dict(Hq=15), rb.RATTN_ERR_INVALID_ARG, "multiple"),
    (dict(D=64), rb.RATTN_ERR_UNSUPPORTED, "head_dim"),
    (dict(ks=9), rb.RATTN_ERR_INVALID_ARG, "kv_splits"),
    (dict(ws=FAKE, wsb=16), rb.RATTN_ERR_WORKSPACE, "workspace"),
])
def test_prefill_tokbias_validation(lib, kw, status, needle):
    assert _prefill_tok(lib, **kw) == status
    assert needle in rb.rattn_last_error()


def test_prefill_tokbias_empty_is_noop(lib):
    assert _prefill_tok(lib, Lq=0, q=None, rt=None) == rb.RATTN_OK


def test_decode_empty_is_noop(lib):
    assert _decode(lib, B=0, q=None, kc=None) == rb.RATTN_OK


def _decode_noalloc(lib, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, ctx=FAKE, win=None, bias=FAKE, out=FAKE, lse=None, B=2, n_q=1,
             Hq=16, Hkv=2, D=128, bs=128, R=8, nb=4, mb=2, max_ctx=200, ns=0, stream=None)
    a.update(kw)
    return lib.rattn_decode_paged_noalloc(a["q"], a["kc"], a["vc"], a["bt"], a["ctx"], a["win"], a["bias"],
                                          a["out"], a["lse"], a["B"], a["n_q"], a["Hq"], a["Hkv"], a["D"], a["bs"],
                                          a["R"], a["nb"], a["mb"], a["max_ctx"], a["ns"], a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), rb.RATTN_ERR_INVALID_ARG, "null"),
    (dict(Hq=15), rb.RATTN_ERR_INVALID_ARG, "multiple"),
    (dict(n_q=0), rb.RATTN_ERR_INVALID_ARG, "n_q"),
    (dict(D=96), rb.RATTN_ERR_UNSUPPORTED, "head_dim"),
    (dict(max_ctx=257, mb=2), rb.RATTN_ERR_INVALID_ARG, "block table"),
    # 2048 sequences of 9 queries over 64/8 heads need far more split scratch than the
    # static array holds: rejected on the host, before any device call
    (dict(B=2048, n_q=9, Hq=64, Hkv=8, max_ctx=4096, mb=32, nb=64), rb.RATTN_ERR_WORKSPACE, "static"),
    (dict(ns=100000, B=64, n_q=9), rb.RATTN_ERR_WORKSPACE, "static"),
])
def test_decode_noalloc_validation(lib, kw, status, needle):
    assert _decode_noalloc(lib, **kw) == status
    assert needle in rb.rattn_last_error()


def test_decode_noalloc_limit(lib):
    """The static scratch is 64 MiB, and the limit check uses the same plan as the workspace
    query: the batch-64 decode and the 1M-token verify fit, a plan one byte larger would not."""
    limit = lib.rattn_decode_paged_noalloc_max_scratch_bytes()
    assert limit == 64 << 20
    assert rb.rattn_decode_workspace_bytes(64, 1, 16, 2, 131072, 0) <= limit
    assert rb.rattn_decode_workspace_bytes(1, 9, 16, 2, 1 << 20, 0) <= limit
    assert rb.rattn_decode_workspace_bytes(2048, 9, 64, 8, 4096, 0) > limit
    assert _decode_noalloc(lib, B=0, q=None, kc=None) == rb.RATTN_OK


def _prefill_paged(lib, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, ctx=FAKE, cu=None, bias=FAKE, out=FAKE, lse=None, B=2, Lq=100, Hq=16,
             Hkv=2,
             D=128, bs=128, R=8, window=0, nb=4, mb=2, max_ctx=200, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.rattn_prefill_paged(a["q"], a["kc"], a["vc"], a["bt"], a["ctx"], a["cu"], a["bias"], a["out"], a["lse"],
                                   a["B"], a["Lq"], a["Hq"], a["Hkv"], a["D"], a["bs"], a["R"], a["window"], a["nb"],
                                   a["mb"], a["max_ctx"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), rb.RATTN_ERR_INVALID_ARG, "null"),
    (dict(kc=None), rb.RATTN_ERR_INVALID_ARG, "null"),
    (dict(bt=None), rb.RATTN_ERR_INVALID_ARG, "null"),
    (dict(ctx=None), rb.RATTN_ERR_INVALID_ARG, "null"),
    (dict(out=None), rb.RATTN_ERR_INVALID_ARG, "null"),
    (dict(Hq=15), rb.RATTN_ERR_INVALID_ARG, "multiple"),
    (dict(R=0), rb.RATTN_ERR_INVALID_ARG, "R="),
    (dict(nb=0), rb.RATTN_ERR_INVALID_ARG, "num_blocks"),
    (dict(max_ctx=99), rb.RATTN_ERR_INVALID_ARG, "max_ctx_len"),
    (dict(max_ctx=257, mb=2), rb.RATTN_ERR_INVALID_ARG, "block table"),
    (dict(B=-1), rb.RATTN_ERR_INVALID_ARG, "negative"),
    (dict(D=64), rb.RATTN_ERR_UNSUPPORTED, "head_dim"),
    (dict(bs=64), rb.RATTN_ERR_UNSUPPORTED, "block_size"),
    (dict(wsb=256), rb.RATTN_ERR_INVALID_ARG, "workspace"),
    (dict(ws=FAKE, wsb=255), rb.RATTN_ERR_WORKSPACE, "workspace"),
])
def test_prefill_paged_validation(lib, kw, status, needle):
    assert _prefill_paged(lib, **kw) == status
    assert needle in rb.rattn_last_error()


def test_prefill_paged_empty_is_noop(lib):
    assert _prefill_paged(lib, B=0, q=None, kc=None) == rb.RATTN_OK
    assert _prefill_paged(lib, Lq=0, q=None, bt=None) == rb.RATTN_OK


def test_workspace_and_split_plan(lib):
    # the KV stream of the batch is split among P workgroups (256 by default); the workspace
    # holds a partial output (128 fp32) and a log-sum-exp per (workgroup + segment) slot, key
    # half and row of a segment, a segment being (sequence, KV head, query-head subgroup)
    for (B, n_q, Hq, Hkv, ctx, ns, gs) in [(64, 1, 16, 2, 131072, 0, 8), (1, 9, 16, 2, 1 << 20, 0, 8),
                                           (3, 2, 8, 8, 1000, 5, 1), (2, 9, 32, 2, 4000, 7, 8),
                                           (5, 100, 4, 1, 5000, 0, 1)]:
        P = rb.rattn_decode_num_splits(B, n_q, Hq, Hkv, ctx, ns)
        assert P == (ns if ns else 256)
        G = Hq // Hkv
        KH = Hkv * (G // gs)
        rows = n_q * gs
        slots = (P + B * KH) * 2   # the two key halves of a unit run on separate waves
        wsb = rb.rattn_decode_workspace_bytes(B, n_q, Hq, Hkv, ctx, ns)
        assert slots * rows * 129 * 4 <= wsb <= slots * rows * 129 * 4 + 256
    assert rb.rattn_decode_workspace_bytes(1, 0, 8, 1, 300, 0) == 0
    assert rb.rattn_decode_num_splits(1, 129, 8, 1, 300, 0) == 0
    # large batches run in launches of at most 2048 sequences sharing one workspace
    big = rb.rattn_decode_workspace_bytes(5000, 1, 16, 2, 4096, 0)
    assert big == rb.rattn_decode_workspace_bytes(2048, 1, 16, 2, 4096, 0)


def _tile_keys(Lq, Lk, window, rows, tile):
    off, T0 = Lk - Lq, tile * rows
    T1 = min(Lq, T0 + rows)
    weff = window if window > 0 else 1 << 30
    return (off + T1 - 1) // 64 + 1 - max(0, off + T0 - weff + 1) // 64


QUEUE_BYTES = 256  # the job queue and its done counter, at the start of every bf16 workspace
COUNTER_BYTES = 256 * 1024  # split counters, at the same place for every plan


def _split_bytes(jobs, parts):
    align = lambda n: (n + 255) // 256 * 256  # noqa: E731
    pieces = jobs * parts
    return align(QUEUE_BYTES + COUNTER_BYTES + pieces * 256 * 4) + pieces * 256 * 128 * 4


def test_prefill_split_plan(lib):
    # forced split: every 256-row tile (32 tokens x 8 heads) with >= 2n key tiles -> n pieces,
    # workspace = the job queue + per-tile counters + a log2-sum-exp and a 128-float partial
    # per piece row
    for (B, Lq, Lk, Hq, Hkv, W, n) in [(1, 1000, 1000, 16, 2, 0, 2), (2, 300, 5000, 8, 1, 0, 3),
                                       (1, 4096, 4096, 16, 2, 1024, 4)]:
        G = Hq // Hkv
        hpw = max(d for d in range(1, 9) if G % d == 0 and 8 % d == 0)
        rows = 32 * (8 // hpw)
        n_tiles = -(-Lq // rows)
        n_split = sum(1 for t in range(n_tiles) if _tile_keys(Lq, Lk, W, rows, t) >= 2 * n)
        jobs = n_split * B * Hkv * (G // hpw)
        want = _split_bytes(jobs, n) if n_split else QUEUE_BYTES
        assert rb.rattn_prefill_workspace_bytes(B, Lq, Lk, Hq, Hkv, W, rb.RATTN_BF16, n) == want
    # the library's own plan: a long sliding-window prefill is split, a long chunked prefill
    # (whose tiles differ in length and balance by themselves) is not; fp32 inputs use no
    # workspace; an unsplit bf16 plan needs the job queue only
    assert rb.rattn_prefill_workspace_bytes(1, 8192, 8192, 16, 2, 4096, rb.RATTN_BF16, 0) > QUEUE_BYTES
    assert rb.rattn_prefill_workspace_bytes(1, 8192, 32768, 16, 2, 0, rb.RATTN_BF16, 0) == QUEUE_BYTES
    assert rb.rattn_prefill_workspace_bytes(1, 8192, 8192, 16, 2, 4096, rb.RATTN_FP32, 0) == 0
    assert rb.rattn_prefill_workspace_bytes(1, 8192, 8192, 16, 2, 4096, rb.RATTN_BF16, 1) == QUEUE_BYTES
    assert rb.rattn_prefill_workspace_bytes(1, 0, 8, 16, 2, 0, rb.RATTN_BF16, 0) == 0


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        rb.load(str(tmp_path / "missing.so"))


def _sconv(lib, **kw):
    a = dict(kn=FAKE, vn=FAKE, wk=FAKE, wv=FAKE, kc=FAKE, vc=FAKE, ks=FAKE, vs=FAKE, bt=FAKE, ctx=FAKE, cu=FAKE, B=2,
             Hkv=2, D=128, bs=128, nb=4, mb=2, max_new=10, stream=None)
    a.update(kw)
    return lib.rattn_kv_sconv_write(a["kn"], a["vn"], a["wk"], a["wv"], a["kc"], a["vc"], a["ks"], a["vs"], a["bt"],
                                    a["ctx"], a["cu"], a["B"], a["Hkv"], a["D"], a["bs"], a["nb"], a["mb"],
                                    a["max_new"], a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(kn=None), rb.RATTN_ERR_INVALID_ARG, "null"),
    (dict(ks=None), rb.RATTN_ERR_INVALID_ARG, "null"),
    (dict(cu=None), rb.RATTN_ERR_INVALID_ARG, "null"),
    (dict(Hkv=0), rb.RATTN_ERR_INVALID_ARG, "Hkv"),
    (dict(nb=0), rb.RATTN_ERR_INVALID_ARG, "num_blocks"),
    (dict(B=70000), rb.RATTN_ERR_INVALID_ARG, "B="),
    (dict(max_new=-1), rb.RATTN_ERR_INVALID_ARG, "negative"),
    (dict(D=64), rb.RATTN_ERR_UNSUPPORTED, "head_dim"),
    (dict(bs=16), rb.RATTN_ERR_UNSUPPORTED, "block_size"),
    (dict(Hkv=9), rb.RATTN_ERR_UNSUPPORTED, "Hkv"),
])
def test_sconv_validation(lib, kw, status, needle):
    assert _sconv(lib, **kw) == status
    assert needle in rb.rattn_last_error()


def test_sconv_empty_is_noop(lib):
    assert _sconv(lib, B=0, kn=None) == rb.RATTN_OK
    assert _sconv(lib, max_new=0, kc=None) == rb.RATTN_OK



def _bwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, r=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, dr=FAKE, B=1, Lq=64,
             Lk=64, Hq=4, Hkv=2, D=128, R=16, W=0, ws=FAKE, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.rattn_prefill_backward(a["q"], a["k"], a["v"], a["r"], a["o"], a["do"], a["lse"], a["dq"], a["dk"],
                                      a["dv"], a["dr"], a["B"], a["Lq"], a["Lk"], a["Hq"], a["Hkv"], a["D"], a["R"],
                                      a["W"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), rb.RATTN_ERR_INVALID_ARG, "null"),
    (dict(dr=None), rb.RATTN_ERR_INVALID_ARG, "null"),
    (dict(lse=None), rb.RATTN_ERR_INVALID_ARG, "null"),
    (dict(Hq=3), rb.RATTN_ERR_INVALID_ARG, "multiple"),
    (dict(Lq=65), rb.RATTN_ERR_INVALID_ARG, "Lq="),
    (dict(R=0), rb.RATTN_ERR_INVALID_ARG, "R="),
    (dict(B=-1), rb.RATTN_ERR_INVALID_ARG, "negative"),
    (dict(B=70000), rb.RATTN_ERR_INVALID_ARG, "65535"),
    (dict(D=64), rb.RATTN_ERR_UNSUPPORTED, "head_dim"),
    (dict(ws=None), rb.RATTN_ERR_WORKSPACE, "workspace"),
    (dict(wsb=255), rb.RATTN_ERR_WORKSPACE, "workspace"),
])
def test_backward_validation(lib, kw, status, needle):
    assert _bwd(lib, **kw) == status
    assert needle in rb.rattn_last_error()


def test_backward_workspace_formula():
    # D and lse*log2(e) per row; partial dK and dV for 2 chunks x ceil(G/2) pairs, each plane
    # [B, Lk, Hkv, 128] fp32; two partial dq slots per query row and head (Lq rounded up to
    # 256), 128 fp32 each; the scaled bias table, Hq x Lk fp32; split counters,
    # B x Hq x ceil(Lq / 32) int
    rows = 8192 * 16 * 4
    plane = 8192 * 2 * 128 * 4
    table = 16 * 8192 * 4
    counters = 16 * 256 * 4
    assert (rb.rattn_prefill_backward_workspace_bytes(1, 8192, 8192, 16, 2)
            == 2 * rows + 2 * 2 * 4 * plane + 2 * 128 * rows + table + counters)
    # 3 rows: two 256-byte row parts; one pair: 2 chunks x 5 keys x 128 x 4 B = 5120 for dK and
    # for dV; dq slots 2 x 256 x 128 x 4; table 1 x 5 x 4 = 20 -> 256; one counter -> 256
    assert (rb.rattn_prefill_backward_workspace_bytes(1, 3, 5, 1, 1)
            == 256 + 256 + 5120 + 5120 + 2 * 256 * 512 + 256 + 256)
    assert rb.rattn_prefill_backward_workspace_bytes(0, 0, 0, 1, 1) == 256
    assert rb.rattn_prefill_backward_workspace_bytes(-1, 1, 1, 1, 1) == 0
    assert rb.rattn_prefill_backward_workspace_bytes(1, 1, 1, 3, 2) == 0  # Hq not a multiple of Hkv
