"""fp64 CPU oracle for relative-bias grouped-query attention.

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the test suite, the smoke check and
the benchmark's CPU-baseline leg use it.  The arithmetic lives in
``rattn_oracle.c`` (plain definition, two-pass softmax in double); this module
only builds that file with gcc, marshals numpy arrays and, for sampled rows,
slices inputs.  It shares nothing with the HIP library.

Definition (vLLM recipes page "thinkingmachines/Inkling", Overview >
Architectural highlights > Attention; term fixed as r[h, min(i-j, R-1)]):
``logit[i,j] = q_i.k_j / sqrt(head_dim) + r[h, min(i-j, R-1)]`` over the causal
(and, for windowed sequences, sliding-window) visible keys.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rattn_oracle.c")
_SRC_BWD = os.path.join(_HERE, "rattn_oracle_bwd.c")
_INCLUDE = os.path.join(os.path.dirname(_HERE), "include")  # include/rattn_oracle.h
_LIB_PATH = os.path.join(_HERE, "librattn_oracle.so")
_lib = None

DTYPE_CODES = {"bf16": 0, "fp32": 1, "fp64": 2}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, fp64, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
               "-ffp-contract=off", "-Wall", "-Wextra", "-I", _INCLUDE, "-o", tmp, _SRC, _SRC_BWD, "-lm"]
        subprocess.run(cmd, check=True, cwd=_HERE)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def load_library(path: str):
    """Load an oracle build from ``path`` (the default build, or a test's own)."""
    lib = ctypes.CDLL(path)
    lib.rattn_ref_cpu.restype = ctypes.c_int
    lib.rattn_ref_cpu.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int] * 11
    if hasattr(lib, "rattn_ref_cpu_tokbias"):
        lib.rattn_ref_cpu_tokbias.restype = ctypes.c_int
        lib.rattn_ref_cpu_tokbias.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int] * 11
    if hasattr(lib, "rattn_ref_cpu_backward"):
        lib.rattn_ref_cpu_backward.restype = ctypes.c_int
        lib.rattn_ref_cpu_backward.argtypes = [ctypes.c_void_p] * 14 + [ctypes.c_double] + [ctypes.c_int] * 10
    return lib


def _load():
    global _lib
    if _lib is None:
        hdr = os.path.join(_INCLUDE, "rattn_oracle.h")
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < max(os.path.getmtime(_SRC),
                                                                             os.path.getmtime(_SRC_BWD),
                                                                             os.path.getmtime(hdr)):
            build(force=True)
        _lib = load_library(_LIB_PATH)
    return _lib


def _bias_f64(bias) -> np.ndarray:
    """A bias table as contiguous float64 (uint16 arrays are bf16 bit patterns: widened
    exactly by placing them in the high half of a float32)."""
    a = np.asarray(bias)
    if a.dtype == np.uint16:
        a = (a.astype(np.uint32) << 16).view(np.float32)
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_of(a: np.ndarray) -> str:
    if a.dtype == np.uint16:
        return "bf16"
    if a.dtype == np.float32:
        return "fp32"
    if a.dtype == np.float64:
        return "fp64"
    raise TypeError(f"unsupported oracle input dtype {a.dtype}")


def ref_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, bias: np.ndarray,
                  ctx_lens: Sequence[int], windows: Optional[Sequence[int]] = None,
                  block_table: Optional[np.ndarray] = None, block_size: int = 128,
                  want_probs: bool = False, num_threads: int = 0,
                  Lk_max: Optional[int] = None, lib=None,
                  token_bias: bool = False) -> Tuple[np.ndarray, np.ndarray, Optional[np.ndarray]]:
    """Run the oracle.

    q: [B, n_q, Hq, D]; k, v: contiguous [B, Lk, Hkv, D] (block_table None) or
    paged [num_blocks, block_size, Hkv, D].  dtype is taken from the arrays
    (uint16 = bf16 bit patterns, float32, float64).  bias: [Hq, R], or with
    token_bias [B, n_q, Hq, R] (one table per query row; uint16 = bf16 bits).
    Returns (out [B,n_q,Hq,D], lse [B,n_q,Hq], probs [B,n_q,Hq,Lk_max] or None),
    all float64.  ``lib`` selects another build of the same C source (default:
    the normal build).
    """
    lib = lib if lib is not None else _load()
    dt = _dtype_of(q)
    if _dtype_of(k) != dt or _dtype_of(v) != dt:
        raise TypeError("q, k, v must share a dtype")
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    B, n_q, Hq, D = q.shape
    Hkv = k.shape[2]
    ctx = np.ascontiguousarray(np.asarray(ctx_lens, dtype=np.int32).reshape(B))
    win = None if windows is None else np.ascontiguousarray(np.asarray(windows, dtype=np.int32).reshape(B))
    bias64 = _bias_f64(bias)
    if token_bias:
        assert bias64.shape[:3] == (B, n_q, Hq), (bias64.shape, (B, n_q, Hq))
        R = bias64.shape[3]
    else:
        Hq_b, R = bias64.shape
        assert Hq_b == Hq
    if block_table is None:
        Lk = k.shape[1]
        bt = None
        mbps = 0
    else:
        bt = np.ascontiguousarray(np.asarray(block_table, dtype=np.int32))
        mbps = bt.shape[1]
        Lk = int(ctx.max()) if B else 0
    if Lk_max is None:
        Lk_max = Lk if block_table is None else max(Lk, 1)
    out = np.empty((B, n_q, Hq, D), dtype=np.float64)
    lse = np.empty((B, n_q, Hq), dtype=np.float64)
    probs = np.empty((B, n_q, Hq, Lk_max), dtype=np.float64) if want_probs else None
    fn = lib.rattn_ref_cpu_tokbias if token_bias else lib.rattn_ref_cpu
    rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(bt), _ptr(ctx), _ptr(win), _ptr(bias64),
            _ptr(out), _ptr(lse), _ptr(probs), B, n_q, Lk_max, Hq, Hkv, D,
            block_size, R, mbps, DTYPE_CODES[dt], int(num_threads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return out, lse, probs


def ref_prefill(q, k, v, bias, window: int = 0, want_probs: bool = False, num_threads: int = 0):
    """Prefill: every sequence has Lk keys; query t sits at Lk - Lq + t."""
    B, Lq = q.shape[:2]
    Lk = k.shape[1]
    return ref_attention(q, k, v, bias, [Lk] * B, [window] * B, None, want_probs=want_probs,
                         num_threads=num_threads)


def ref_prefill_rows(q, k, v, bias, window: int, rows: Sequence[Tuple[int, int]], num_threads: int = 0):
    """Oracle output for selected query rows (b, t) of a prefill, one row at a time.

    Query t of a prefill with Lk keys sits at p = Lk - Lq + t; presenting only
    that query with p + 1 keys places it at the same position, so the oracle
    computes exactly the row the full call would.  Returns (out [n, Hq, D],
    lse [n, Hq])."""
    B, Lq = q.shape[:2]
    Lk = k.shape[1]
    outs, lses = [], []
    for (b, t) in rows:
        p = Lk - Lq + t
        o, l, _ = ref_attention(q[b:b + 1, t:t + 1], k[b:b + 1], v[b:b + 1], bias, [p + 1], [window],
                                None, num_threads=num_threads)
        outs.append(o[0, 0])
        lses.append(l[0, 0])
    return np.stack(outs), np.stack(lses)


def ref_decode(case, want_probs: bool = False, num_threads: int = 0, batch_index=None):
    """Paged decode on a synth DecodeCase (optionally for a subset of sequences)."""
    if batch_index is None:
        return ref_attention(case.q, case.k_cache, case.v_cache, case.bias, case.ctx_lens, case.windows,
                             case.block_table, want_probs=want_probs, num_threads=num_threads)
    idx = np.asarray(batch_index)
    return ref_attention(case.q[idx], case.k_cache, case.v_cache, case.bias, case.ctx_lens[idx],
                         case.windows[idx], case.block_table[idx], want_probs=want_probs,
                         num_threads=num_threads)


def ref_prefill_tokbias(q, k, v, bias_tok, window: int = 0, want_probs: bool = False, num_threads: int = 0,
                        lib=None):
    """Prefill with a token-dependent bias: bias_tok [B, Lq, Hq, R] (float32/64, or uint16
    bf16 bits), row (b, t, h) using its own table r_t[h, min(p - j, R - 1)]."""
    B = q.shape[0]
    Lk = k.shape[1]
    return ref_attention(q, k, v, bias_tok, [Lk] * B, [window] * B, None, want_probs=want_probs,
                         num_threads=num_threads, lib=lib, token_bias=True)


def ref_prefill_tokbias_rows(q, k, v, bias_tok, window: int, rows: Sequence[Tuple[int, int]],
                             num_threads: int = 0):
    """ref_prefill_tokbias for selected query rows (b, t), one at a time (each query placed
    alone at its own position, with its own table row).  Returns (out [n, Hq, D], lse [n, Hq])."""
    Lq = q.shape[1]
    Lk = k.shape[1]
    outs, lses = [], []
    for (b, t) in rows:
        p = Lk - Lq + t
        o, l, _ = ref_attention(q[b:b + 1, t:t + 1], k[b:b + 1], v[b:b + 1], bias_tok[b:b + 1, t:t + 1], [p + 1],
                                [window], None, num_threads=num_threads, token_bias=True)
        outs.append(o[0, 0])
        lses.append(l[0, 0])
    return np.stack(outs), np.stack(lses)


def ref_backward(q, k, v, bias, dout, window: int = 0, want_abs: bool = True, num_threads: int = 0, lib=None,
                 out=None, abs_weight: float = 1.0):
    """Gradients of a prefill (C oracle, one query row at a time in double).

    q, dout [B, Lq, Hq, D]; k, v [B, Lk, Hkv, D] (uint16 bf16 bits, float32 or float64, one
    dtype); bias [Hq, R]; out: None (D = sum_j P_j dP_j) or a forward output like q, same
    dtype (D = rowsum(dout * out)).  Returns (dq, dk, dv, dbias) and, with want_abs, the
    magnitude sums (dq_abs, dk_abs, dv_abs, dbias_abs) as a second tuple (else None), with
    dS_abs = P (|dP - D| + abs_weight (a_j + D_abs)); all float64."""
    lib = lib if lib is not None else _load()
    dt = _dtype_of(q)
    if any(_dtype_of(a) != dt for a in (k, v, dout) + ((out,) if out is not None else ())):
        raise TypeError("q, k, v, dout (and out) must share a dtype")
    q, k, v, dout = (np.ascontiguousarray(a) for a in (q, k, v, dout))
    out = None if out is None else np.ascontiguousarray(out)
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    bias64 = _bias_f64(bias)
    R = bias64.shape[1]
    grads = [np.empty(q.shape), np.empty(k.shape), np.empty(k.shape), np.empty((Hq, R))]
    absums = [np.empty(q.shape), np.empty(k.shape), np.empty(k.shape), np.empty((Hq, R))] if want_abs else [None] * 4
    rc = lib.rattn_ref_cpu_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(out), _ptr(bias64),
                                    *[_ptr(g) for g in grads], *[_ptr(a) for a in absums], float(abs_weight),
                                    B, Lq, Lk, Hq, Hkv, D, R, int(window), DTYPE_CODES[dt], int(num_threads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return tuple(grads), (tuple(absums) if want_abs else None)
