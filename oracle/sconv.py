"""fp64 CPU oracle for the K/V short convolution written into the paged caches.

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the test suite and the benchmark use it.  It
shares nothing with the HIP library.

What it computes (vLLM recipes page "thinkingmachines/Inkling", Overview > Architectural
highlights > Short convolution: each layer runs four-tap short convolutions over the token
axis of, among others, the attention keys and values; their running state lives in paged
storage that the engine handles like an attention cache).  The pages give no formula; the reading taken is the plain causal depthwise
convolution over tokens with four taps and a weight per tap and channel, no bias, no
activation:

    y[p, c] = sum_{s=0..3} w[s, c] * x[p - s, c],      x[p] = 0 for p < 0,

for key and value channels c = (kv head, dim) separately (one weight set each).  For a chunk
of n_b new tokens of sequence b, at positions ctx_lens[b] - n_b .. ctx_lens[b] - 1, the raw
x of earlier positions comes from the state cache (the raw K/V written by earlier calls), the
conv output y goes to the attention cache and the raw x to the state cache, both at the new
positions, through the sequence's block table (128-token blocks).  Outputs are rounded to
bf16 (round to nearest even).
"""
from __future__ import annotations

import numpy as np

BLOCK = 128
TAPS = 4


def bf16_to_f64(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16(a: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns: the float64 value rounded once to 8 significant bits,
    ties to even (numpy's round is half-to-even); normal range only (the values here are far
    from the float32 limits)."""
    f = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(f)                      # f = m * 2^e, 0.5 <= |m| < 1 (m = 0 for f = 0)
    out = np.ldexp(np.round(np.ldexp(m, 8)), e - 8).astype(np.float32)  # exact in float32
    return (out.view(np.uint32) >> 16).astype(np.uint16)


def sconv_write(k_new, v_new, w_k, w_v, k_cache, v_cache, k_state, v_state, block_table, ctx_lens, cu_seqlens):
    """Return (k_cache, v_cache, k_state, v_state, y_k, y_v): copies of the caches after the
    write, and the fp64 conv outputs of the new tokens in packed order [T, Hkv, 128].

    k_new, v_new  [T, Hkv, 128] bf16 bits; w_k, w_v [4, Hkv, 128] float (tap s multiplies
    x[p - s]); caches [num_blocks, 128, Hkv, 128] bf16 bits; block_table [B, mb]; ctx_lens
    [B] (keys after the write); cu_seqlens [B + 1] (new tokens of sequence b are rows
    cu_seqlens[b] .. cu_seqlens[b + 1] - 1)."""
    k_cache, v_cache = k_cache.copy(), v_cache.copy()
    k_state_in, v_state_in = k_state, v_state
    k_state, v_state = k_state.copy(), v_state.copy()
    y_k = np.zeros(k_new.shape, dtype=np.float64)
    y_v = np.zeros(v_new.shape, dtype=np.float64)
    wk = np.asarray(w_k, dtype=np.float64)
    wv = np.asarray(w_v, dtype=np.float64)
    for b in range(len(ctx_lens)):
        r0, r1 = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        n = r1 - r0
        start = int(ctx_lens[b]) - n  # position of the first new token

        def raw(new, state, pos):
            """x[pos] of sequence b as float64 (zero before position 0)."""
            if pos < 0:
                return np.zeros(new.shape[1:], dtype=np.float64)
            if pos >= start:
                return bf16_to_f64(new[r0 + pos - start])
            return bf16_to_f64(state[block_table[b, pos // BLOCK], pos % BLOCK])

        for t in range(n):
            p = start + t
            acc_k = np.zeros(k_new.shape[1:], dtype=np.float64)
            acc_v = np.zeros(v_new.shape[1:], dtype=np.float64)
            for s in range(TAPS):
                acc_k += wk[s] * raw(k_new, k_state_in, p - s)
                acc_v += wv[s] * raw(v_new, v_state_in, p - s)
            y_k[r0 + t], y_v[r0 + t] = acc_k, acc_v
            blk, slot = block_table[b, p // BLOCK], p % BLOCK
            k_cache[blk, slot] = f64_to_bf16(acc_k)
            v_cache[blk, slot] = f64_to_bf16(acc_v)
            k_state[blk, slot] = k_new[r0 + t]
            v_state[blk, slot] = v_new[r0 + t]
    return k_cache, v_cache, k_state, v_state, y_k, y_v
