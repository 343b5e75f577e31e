"""Seeded synthetic inputs for relative-bias GQA attention.

This module only draws random numbers and lays them out in memory; it holds
none of the attention arithmetic.  Both the CPU oracle and the HIP path are
fed from here so that they see identical bytes.

Conventions (one fresh ``numpy.random.default_rng(seed)`` per workload, draws in
the order listed by each function):

* bf16 tensors are drawn as float32 ``standard_normal`` and rounded to
  bfloat16 with round-to-nearest-even; they are returned as ``uint16`` bit
  patterns (``to_float`` widens them back exactly).
* The relative-bias table ``r[Hq, R]`` is float32 ``0.5 * standard_normal``
  (standard deviation 0.5).
* Layouts: Q ``[B, L, Hq, 128]``, K/V ``[B, L, Hkv, 128]`` token-major; paged
  caches ``[num_blocks, 128, Hkv, 128]``; block table ``int32 [B, max_blocks]``.

The workload shapes follow the Inkling recipe page (vLLM recipes,
"thinkingmachines/Inkling", Overview > Architectural highlights: grouped-query
attention with head size 128, full and sliding-window layers, 9 tokens per
step with MTP; Client Usage: ``--block-size 128``; TP4 on MI355X, so one GPU
holds 16 of 64 query heads and 2 of 8 KV heads).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np

HEAD_DIM = 128
BLOCK_SIZE = 128


# ----------------------------------------------------------------------------
# bf16 helpers (bit-level, no arithmetic of the method)
# ----------------------------------------------------------------------------
def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even.

    NaN inputs stay NaN (quiet bit forced)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # no finite or infinite input can carry past bit 31 here (largest is 0xFF7FFFFF + 0x8000)
    rounded = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = ((u[nan] >> 16) | 0x0040).astype(np.uint16)
    return rounded


def to_float(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32, exact."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


_CHUNK = 1 << 22


def _normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) float32 draws rounded to bf16.

    One 63-bit key is drawn from ``rng``; chunk c of ``_CHUNK`` values then comes from
    its own PCG64 stream seeded with (key, c), so large tensors fill in parallel and the
    bytes do not depend on the number of threads."""
    n = int(np.prod(shape))
    key = int(rng.integers(0, 1 << 63))
    out = np.empty(n, dtype=np.uint16)

    def fill(c: int) -> None:
        s = c * _CHUNK
        e = min(n, s + _CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([key, c])))
        out[s:e] = bf16_round(g.standard_normal(e - s, dtype=np.float32))

    nchunks = (n + _CHUNK - 1) // _CHUNK
    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        workers = max(1, min(16, len(os.sched_getaffinity(0)), nchunks))
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return _normal_bf16(rng, shape)
    if dtype == "fp32":
        return rng.standard_normal(shape, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype}")


def _bias(rng: np.random.Generator, hq: int, r: int) -> np.ndarray:
    return (0.5 * rng.standard_normal((hq, r), dtype=np.float32)).astype(np.float32)


# ----------------------------------------------------------------------------
# Prefill (contiguous K/V)
# ----------------------------------------------------------------------------
@dataclass
class PrefillCase:
    q: np.ndarray            # [B, Lq, Hq, 128] uint16 (bf16 bits) or float32
    k: np.ndarray            # [B, Lk, Hkv, 128]
    v: np.ndarray            # [B, Lk, Hkv, 128]
    bias: np.ndarray         # [Hq, R] float32
    window: int              # <= 0: full causal
    dtype: str               # "bf16" | "fp32"
    name: str = ""

    @property
    def B(self): return self.q.shape[0]
    @property
    def Lq(self): return self.q.shape[1]
    @property
    def Lk(self): return self.k.shape[1]
    @property
    def Hq(self): return self.q.shape[2]
    @property
    def Hkv(self): return self.k.shape[2]
    @property
    def R(self): return self.bias.shape[1]


def make_prefill(seed: int, B: int, Lq: int, Lk: int, Hq: int, Hkv: int, R: int,
                 window: int, dtype: str = "bf16", name: str = "") -> PrefillCase:
    """Draw order: Q, K, V, r."""
    rng = np.random.default_rng(seed)
    q = _normal(rng, (B, Lq, Hq, HEAD_DIM), dtype)
    k = _normal(rng, (B, Lk, Hkv, HEAD_DIM), dtype)
    v = _normal(rng, (B, Lk, Hkv, HEAD_DIM), dtype)
    bias = _bias(rng, Hq, R)
    return PrefillCase(q, k, v, bias, window, dtype, name)


@dataclass
class BackwardCase:
    fwd: PrefillCase          # q, k, v, r, window of the forward pass (bf16)
    dout: np.ndarray          # [B, Lq, Hq, 128] uint16 (bf16 bits): gradient of the output
    name: str = ""


def make_backward(seed: int, B: int, Lq: int, Lk: int, Hq: int, Hkv: int, R: int, window: int,
                  name: str = "") -> BackwardCase:
    """Draw order: the prefill case of the same seed (Q, K, V, r), then dO N(0,1) from a
    generator seeded with (seed, 1)."""
    fwd = make_prefill(seed, B, Lq, Lk, Hq, Hkv, R, window, "bf16", name)
    rng = np.random.default_rng([seed, 1])
    return BackwardCase(fwd, _normal(rng, (B, Lq, Hq, HEAD_DIM), "bf16"), name)


@dataclass
class TokBiasCase:
    """A prefill whose relative-bias table depends on the query token: row (b, t, h) has
    its own table bias_tok[b, t, h, :] (a "qkvr" projection output, bf16)."""
    fwd: PrefillCase          # q, k, v, window of the prefill (bf16); its static table is unused
    bias_tok: np.ndarray      # [B, Lq, Hq, R] uint16 (bf16 bits)
    name: str = ""

    @property
    def R(self): return self.bias_tok.shape[3]


def make_prefill_tokbias(seed: int, B: int, Lq: int, Lk: int, Hq: int, Hkv: int, R: int, window: int,
                         name: str = "") -> TokBiasCase:
    """Draw order: the bf16 prefill case of the same seed (Q, K, V and a one-entry static
    table), then the per-token tables from a generator seeded with (seed, 2): 0.5 * N(0,1)
    rounded to bf16 (the N(0,1) draws rounded to bf16, then halved, which is exact)."""
    fwd = make_prefill(seed, B, Lq, Lk, Hq, Hkv, 1, window, "bf16", name)
    rng = np.random.default_rng([seed, 2])
    tab = bf16_round(0.5 * to_float(_normal_bf16(rng, (B, Lq, Hq, R))))
    return TokBiasCase(fwd, tab, name)


# ----------------------------------------------------------------------------
# Paged decode
# ----------------------------------------------------------------------------
@dataclass
class DecodeCase:
    q: np.ndarray             # [B, n_q, Hq, 128] uint16 (bf16 bits)
    k_cache: np.ndarray       # [num_blocks, 128, Hkv, 128] uint16
    v_cache: np.ndarray       # [num_blocks, 128, Hkv, 128] uint16
    block_table: np.ndarray   # [B, max_blocks_per_seq] int32
    ctx_lens: np.ndarray      # [B] int32, tokens in cache including the n_q queries
    windows: np.ndarray       # [B] int32, <= 0 full
    bias: np.ndarray          # [Hq, R] float32
    name: str = ""
    poison_block: Optional[int] = None

    @property
    def B(self): return self.q.shape[0]
    @property
    def n_q(self): return self.q.shape[1]
    @property
    def Hq(self): return self.q.shape[2]
    @property
    def Hkv(self): return self.k_cache.shape[2]
    @property
    def R(self): return self.bias.shape[1]
    @property
    def num_blocks(self): return self.k_cache.shape[0]
    @property
    def max_blocks_per_seq(self): return self.block_table.shape[1]
    @property
    def max_ctx_len(self): return int(self.ctx_lens.max()) if self.B else 0


def resident_block_range(ctx: int, n_q: int, window: int, block_size: int = BLOCK_SIZE):
    """Logical blocks a serving engine keeps resident for one sequence.

    Full-attention sequences keep every block; a sliding-window sequence keeps
    the blocks overlapping the last ``window + n_q - 1`` positions (a
    conservative superset of what its queries can see).  Other block-table
    entries point at a poison block."""
    nblk = (ctx + block_size - 1) // block_size
    if window <= 0:
        return 0, nblk
    first_pos = max(0, ctx - n_q - window + 1)
    return first_pos // block_size, nblk


def make_decode(seed: int, ctx_lens, windows, n_q: int, Hq: int, Hkv: int, R: int,
                name: str = "", poison: bool = True, draw_ctx=None) -> DecodeCase:
    """Build a paged-KV decode case.

    Draw order: (optional ``draw_ctx(rng)`` for the context lengths), physical
    block permutation, K cache, V cache, Q, r.  Resident blocks get physical
    ids from one random permutation; if ``poison`` is set one extra block of
    NaNs sits at the end and every non-resident block-table entry, as well as
    every cache slot at or beyond a sequence's context length, holds NaN.
    """
    rng = np.random.default_rng(seed)
    if draw_ctx is not None:
        ctx_lens = draw_ctx(rng)
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32)
    windows = np.asarray(windows, dtype=np.int32)
    B = len(ctx_lens)
    ranges = [resident_block_range(int(c), n_q, int(w)) for c, w in zip(ctx_lens, windows)]
    max_blocks = max((e for _, e in ranges), default=1)
    total = sum(e - s for s, e in ranges)
    perm = rng.permutation(total).astype(np.int32)
    num_blocks = total + (1 if poison else 0)
    poison_id = total if poison else 0
    bt = np.full((B, max(1, max_blocks)), poison_id, dtype=np.int32)
    pos = 0
    for b, (s, e) in enumerate(ranges):
        bt[b, s:e] = perm[pos:pos + e - s]
        pos += e - s
    shape = (num_blocks, BLOCK_SIZE, Hkv, HEAD_DIM)
    kc = _normal_bf16(rng, shape)
    vc = _normal_bf16(rng, shape)
    nan16 = np.uint16(0x7FC0)
    if poison:
        kc[poison_id] = nan16
        vc[poison_id] = nan16
        for b, c in enumerate(ctx_lens):
            c = int(c)
            last = (c - 1) // BLOCK_SIZE
            off = c - last * BLOCK_SIZE
            if off < BLOCK_SIZE:
                kc[bt[b, last], off:] = nan16
                vc[bt[b, last], off:] = nan16
    q = _normal_bf16(rng, (B, n_q, Hq, HEAD_DIM))
    bias = _bias(rng, Hq, R)
    return DecodeCase(q, kc, vc, bt, ctx_lens, windows, bias, name, poison_id if poison else None)


@dataclass
class SconvCase:
    k_new: np.ndarray        # [T, Hkv, 128] uint16 (bf16 bits), packed new tokens
    v_new: np.ndarray
    w_k: np.ndarray          # [4, Hkv, 128] float32
    w_v: np.ndarray
    k_cache: np.ndarray      # [num_blocks, 128, Hkv, 128] uint16
    v_cache: np.ndarray
    k_state: np.ndarray
    v_state: np.ndarray
    block_table: np.ndarray  # [B, max_blocks_per_seq] int32
    ctx_lens: np.ndarray     # [B] int32, keys after the write
    cu_seqlens: np.ndarray   # [B + 1] int32
    name: str = ""

    @property
    def n_new(self): return np.diff(self.cu_seqlens)


def make_sconv(seed: int, ctx_lens, n_new, Hkv: int, name: str = "") -> SconvCase:
    """Draw order: block permutation, the four caches, new K, new V, w_k, w_v (N(0,1))."""
    rng = np.random.default_rng(seed)
    ctx = np.asarray(ctx_lens, dtype=np.int32)
    B = len(ctx)
    nbps = max(1, max((int(c) + BLOCK_SIZE - 1) // BLOCK_SIZE for c in ctx))
    bt = rng.permutation(B * nbps).astype(np.int32).reshape(B, nbps)
    shape = (B * nbps, BLOCK_SIZE, Hkv, HEAD_DIM)
    caches = [_normal_bf16(rng, shape) for _ in range(4)]
    T = int(np.sum(n_new))
    k_new = _normal_bf16(rng, (T, Hkv, HEAD_DIM))
    v_new = _normal_bf16(rng, (T, Hkv, HEAD_DIM))
    w_k = rng.standard_normal((4, Hkv, HEAD_DIM)).astype(np.float32)
    w_v = rng.standard_normal((4, Hkv, HEAD_DIM)).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
    return SconvCase(k_new, v_new, w_k, w_v, *caches, bt, ctx, cu, name)


# ----------------------------------------------------------------------------
# The named workloads
# ----------------------------------------------------------------------------
WORKLOADS = {
    "tiny_prefill_fp32": "batch 1, L=256, 4 q / 1 kv heads, fp32, full causal, R=256",
    "swa_prefill_8k": "batch 1, L=8192, 16 q / 2 kv heads, bf16, window 4096, R=4096",
    "chunked_prefill_32k": "batch 1, 8192 queries at 24576..32767 over 32768 keys, 16/2 heads, bf16, full, R=8192",
    "paged_decode_b64": "batch 64, 1 query, ctx U[4096,131072], odd b window 4096, 16/2 heads, bf16, R=8192",
    "mtp_verify_1m": "batch 1, 9 queries at the tail of 1,048,576 keys, 16/2 heads, bf16, full, R=8192",
    "paged_prefill_b4": "batch 4, 2048-query chunks at the tails of 8192/16384/24576/32768-key paged contexts, "
                        "16/2 heads, bf16, full causal, R=8192",
    "kv_sconv_32k": "batch 4, 8192 new tokens each after prefixes of 0/8192/16384/24576 tokens, 2 KV heads, "
                    "bf16, window-4 short convolution into paged caches",
    "swa_prefill_8k_bwd": "backward of swa_prefill_8k (batch 1, L=8192, 16/2 heads, window 4096, R=4096): dq, dk, dv, "
                          "dr for a N(0,1) output gradient",
    "swa_prefill_8k_tokbias": "batch 1, L=8192, 16/2 heads, bf16, window 4096, a token-dependent bf16 table of "
                              "R=512 entries per query row and head (0.5*N(0,1))",
}


def tiny_prefill_fp32(seed: int = 0) -> PrefillCase:
    return make_prefill(seed, 1, 256, 256, 4, 1, 256, 0, "fp32", "tiny_prefill_fp32")


def swa_prefill_8k(seed: int = 0) -> PrefillCase:
    return make_prefill(seed, 1, 8192, 8192, 16, 2, 4096, 4096, "bf16", "swa_prefill_8k")


def chunked_prefill_32k(seed: int = 0) -> PrefillCase:
    return make_prefill(seed, 1, 8192, 32768, 16, 2, 8192, 0, "bf16", "chunked_prefill_32k")


def paged_decode_b64(seed: int = 0) -> DecodeCase:
    B = 64
    windows = np.where(np.arange(B) % 2 == 1, 4096, 0).astype(np.int32)
    draw = lambda rng: rng.integers(4096, 131072, size=B, endpoint=True).astype(np.int32)
    return make_decode(seed, None, windows, 1, 16, 2, 8192, "paged_decode_b64", True, draw)


def mtp_verify_1m(seed: int = 0) -> DecodeCase:
    return make_decode(seed, [1 << 20], [0], 9, 16, 2, 8192, "mtp_verify_1m", poison=False)


def paged_prefill_b4(seed: int = 0) -> DecodeCase:
    """Chunked prefill over a prefix cache: four sequences whose last 2048 tokens are the
    chunk (their K/V already in the paged cache), contexts 8K..32K."""
    return make_decode(seed, [8192, 16384, 24576, 32768], [0, 0, 0, 0], 2048, 16, 2, 8192, "paged_prefill_b4")


def kv_sconv_32k(seed: int = 0) -> SconvCase:
    return make_sconv(seed, [8192, 16384, 24576, 32768], [8192] * 4, 2, "kv_sconv_32k")


def swa_prefill_8k_bwd(seed: int = 0) -> BackwardCase:
    return make_backward(seed, 1, 8192, 8192, 16, 2, 4096, 4096, "swa_prefill_8k_bwd")


def swa_prefill_8k_tokbias(seed: int = 0) -> TokBiasCase:
    """The 8K-token window-4096 prefill with a token-dependent table of 512 entries per row."""
    return make_prefill_tokbias(seed, 1, 8192, 8192, 16, 2, 512, 4096, "swa_prefill_8k_tokbias")


WORKLOAD_FNS = {
    "tiny_prefill_fp32": tiny_prefill_fp32,
    "swa_prefill_8k": swa_prefill_8k,
    "chunked_prefill_32k": chunked_prefill_32k,
    "paged_decode_b64": paged_decode_b64,
    "mtp_verify_1m": mtp_verify_1m,
    "paged_prefill_b4": paged_prefill_b4,
    "kv_sconv_32k": kv_sconv_32k,
    "swa_prefill_8k_bwd": swa_prefill_8k_bwd,
    "swa_prefill_8k_tokbias": swa_prefill_8k_tokbias,
}
