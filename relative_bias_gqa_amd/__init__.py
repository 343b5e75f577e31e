"""relative_bias_gqa_amd -- relative-bias grouped-query attention for MI355X (gfx950).

Thin ctypes binding over ``librattn.so`` (C ABI in ``include/rattn.h``).  The
functions named like the C entry points only marshal arguments: they read
shapes and device pointers off torch tensors and call the library on the
current (or given) HIP stream.  Every step of the computation runs in the HIP
kernels; there is no fallback.  If the library is missing or fails to load,
every call raises.

Operation (vLLM recipes page "thinkingmachines/Inkling", Overview >
Architectural highlights > Attention): GQA with head size 128 whose logits
carry a trained bias depending on the query-key distance, fixed here as
``logit[i,j] = q_i.k_j/sqrt(128) + r[h, min(i-j, R-1)]``; causal full or
sliding-window; prefill over contiguous K/V and paged (block 128) decode with
multi-query (MTP) verification.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librattn.so")

RATTN_OK, RATTN_ERR_INVALID_ARG, RATTN_ERR_UNSUPPORTED, RATTN_ERR_WORKSPACE, RATTN_ERR_HIP = 0, 1, 2, 3, 4
RATTN_BF16, RATTN_FP32 = 0, 1
ABI_VERSION = 9

EXPORTED = ("rattn_prefill_workspace_bytes", "rattn_prefill", "rattn_prefill_tokbias", "rattn_prefill_paged", "rattn_kv_sconv_write",
            "rattn_prefill_backward_workspace_bytes", "rattn_prefill_backward",
            "rattn_decode_num_splits", "rattn_decode_workspace_bytes", "rattn_decode_paged",
            "rattn_decode_paged_noalloc_max_scratch_bytes", "rattn_decode_paged_noalloc", "rattn_last_error",
            "rattn_abi_version")

_lib = None


class RattnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


def load(path: Optional[str] = None):
    """Load (once) and return the ctypes handle of librattn.so."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built: run `python -m relative_bias_gqa_amd.build` "
                           "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(p)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.rattn_prefill_workspace_bytes.restype = sz
    lib.rattn_prefill_workspace_bytes.argtypes = [i32] * 8
    lib.rattn_prefill.restype = i32
    lib.rattn_prefill.argtypes = [vp] * 6 + [i32] * 10 + [vp, sz, vp]
    lib.rattn_prefill_tokbias.restype = i32
    lib.rattn_prefill_tokbias.argtypes = [vp] * 6 + [i32] * 9 + [vp, sz, vp]
    lib.rattn_prefill_paged.restype = i32
    lib.rattn_prefill_paged.argtypes = [vp] * 9 + [i32] * 11 + [vp, sz, vp]
    lib.rattn_kv_sconv_write.restype = i32
    lib.rattn_kv_sconv_write.argtypes = [vp] * 11 + [i32] * 7 + [vp]
    lib.rattn_prefill_backward_workspace_bytes.restype = sz
    lib.rattn_prefill_backward_workspace_bytes.argtypes = [i32] * 5
    lib.rattn_prefill_backward.restype = i32
    lib.rattn_prefill_backward.argtypes = [vp] * 11 + [i32] * 8 + [vp, sz, vp]
    lib.rattn_decode_num_splits.restype = i32
    lib.rattn_decode_num_splits.argtypes = [i32] * 6
    lib.rattn_decode_workspace_bytes.restype = sz
    lib.rattn_decode_workspace_bytes.argtypes = [i32] * 6
    lib.rattn_decode_paged.restype = i32
    lib.rattn_decode_paged.argtypes = [vp] * 9 + [i32] * 11 + [vp, sz, vp]
    lib.rattn_decode_paged_noalloc_max_scratch_bytes.restype = sz
    lib.rattn_decode_paged_noalloc_max_scratch_bytes.argtypes = []
    lib.rattn_decode_paged_noalloc.restype = i32
    lib.rattn_decode_paged_noalloc.argtypes = [vp] * 9 + [i32] * 11 + [vp]
    lib.rattn_last_error.restype = ctypes.c_char_p
    lib.rattn_last_error.argtypes = []
    lib.rattn_abi_version.restype = i32
    lib.rattn_abi_version.argtypes = []
    if lib.rattn_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{p}: ABI version {lib.rattn_abi_version()} != {ABI_VERSION}")
    if path is None:
        _lib = lib
    return lib


def rattn_last_error() -> str:
    return load().rattn_last_error().decode()


def rattn_abi_version() -> int:
    return load().rattn_abi_version()


def _check(status: int):
    if status != RATTN_OK:
        raise RattnError(status, rattn_last_error())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to librattn must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return RATTN_BF16
    if t.dtype == torch.float32:
        return RATTN_FP32
    raise ValueError(f"unsupported dtype {t.dtype}")


def rattn_prefill_workspace_bytes(B: int, Lq: int, Lk: int, Hq: int, Hkv: int, window: int = 0,
                                  dtype: int = RATTN_BF16, kv_splits: int = 0) -> int:
    return load().rattn_prefill_workspace_bytes(B, Lq, Lk, Hq, Hkv, int(window), dtype, int(kv_splits))


def rattn_prefill(q, k, v, bias, out, lse=None, window: int = 0, kv_splits: int = 0, workspace=None,
                  stream=None) -> None:
    """q [B,Lq,Hq,128], k/v [B,Lk,Hkv,128] (bf16 or fp32), bias [Hq,R] fp32,
    out like q, lse [B,Lq,Hq] fp32 or None.  Query t sits at position Lk-Lq+t.
    workspace: a uint8 device tensor of at least rattn_prefill_workspace_bytes(...) bytes,
    zero-filled before its first use (calls leave it so), or None (no key-range split)."""
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    R = bias.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().rattn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(out), _ptr(lse),
                                B, Lq, Lk, Hq, Hkv, D, R, int(window), _dtype_code(q), int(kv_splits),
                                _ptr(workspace), ws_bytes, _stream(stream)))


def rattn_prefill_tokbias(q, k, v, bias_tok, out, lse=None, window: int = 0, kv_splits: int = 0, workspace=None,
                          stream=None) -> None:
    """q [B,Lq,Hq,128], k/v [B,Lk,Hkv,128] bf16, bias_tok [B,Lq,Hq,R] bf16 (query t's own
    table), out like q, lse [B,Lq,Hq] fp32 or None; workspace as for rattn_prefill."""
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    R = bias_tok.shape[3]
    if tuple(bias_tok.shape[:3]) != (B, Lq, Hq):
        raise ValueError(f"bias_tok shape {tuple(bias_tok.shape)} does not match q {tuple(q.shape)}")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().rattn_prefill_tokbias(_ptr(q), _ptr(k), _ptr(v), _ptr(bias_tok), _ptr(out), _ptr(lse),
                                        B, Lq, Lk, Hq, Hkv, D, R, int(window), int(kv_splits),
                                        _ptr(workspace), ws_bytes, _stream(stream)))


PREFILL_PAGED_WORKSPACE_BYTES = 256


def rattn_prefill_paged(q, k_cache, v_cache, block_table, ctx_lens, bias, out, lse, max_ctx_len: int,
                        window: int = 0, workspace=None, stream=None, cu_seqlens_q=None, max_q_len: int = 0) -> None:
    """q [B,Lq,Hq,128] bf16, or packed [total,Hq,128] with cu_seqlens_q [B+1] int32 and the
    longest chunk max_q_len; caches [num_blocks,128,Hkv,128] bf16; block_table [B,mb] int32;
    ctx_lens [B] int32 (keys in the cache including the chunk's own); bias [Hq,R] fp32; out
    like q; lse like q without its last dimension (fp32) or None.  Query t of sequence b
    (n_b queries) sits at ctx_lens[b]-n_b+t.  workspace: a zero-filled uint8 device tensor of
    at least PREFILL_PAGED_WORKSPACE_BYTES (a job queue; calls leave it zero-filled), or None
    (one workgroup per job)."""
    if _dtype_code(q) != RATTN_BF16:
        raise TypeError("rattn_prefill_paged takes bf16 q and caches")
    if cu_seqlens_q is None:
        B, Lq, Hq, D = q.shape
    else:
        B, Lq = block_table.shape[0], int(max_q_len)
        Hq, D = q.shape[1], q.shape[2]
    num_blocks, bs, Hkv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    mb = block_table.shape[1]
    R = bias.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().rattn_prefill_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(ctx_lens),
                                      _ptr(cu_seqlens_q), _ptr(bias), _ptr(out), _ptr(lse), B, Lq, Hq, Hkv, D, bs, R,
                                      int(window),
                                      num_blocks, mb, int(max_ctx_len), _ptr(workspace), ws_bytes,
                                      _stream(stream)))


def rattn_kv_sconv_write(k_new, v_new, w_k, w_v, k_cache, v_cache, k_state, v_state, block_table, ctx_lens,
                         cu_seqlens, max_new: int, stream=None) -> None:
    """k_new/v_new [T,Hkv,128] bf16 packed new tokens; w_k/w_v [4,Hkv,128] fp32; the attention
    caches and the state caches [num_blocks,128,Hkv,128] bf16 (one block table [B,mb] int32);
    ctx_lens [B] int32 keys after the write; cu_seqlens [B+1] int32; max_new >= every chunk."""
    B = block_table.shape[0]
    num_blocks, bs, Hkv, D = k_cache.shape
    mb = block_table.shape[1]
    _check(load().rattn_kv_sconv_write(_ptr(k_new), _ptr(v_new), _ptr(w_k), _ptr(w_v), _ptr(k_cache), _ptr(v_cache),
                                       _ptr(k_state), _ptr(v_state), _ptr(block_table), _ptr(ctx_lens),
                                       _ptr(cu_seqlens), B, Hkv, D, bs, num_blocks, mb, int(max_new),
                                       _stream(stream)))


def rattn_prefill_backward_workspace_bytes(B: int, Lq: int, Lk: int, Hq: int, Hkv: int) -> int:
    return load().rattn_prefill_backward_workspace_bytes(B, Lq, Lk, Hq, Hkv)


def rattn_prefill_backward(q, k, v, bias, out, dout, lse, dq, dk, dv, dbias, window: int, workspace,
                           stream=None) -> None:
    """q/out/dout [B,Lq,Hq,128] bf16; k/v [B,Lk,Hkv,128] bf16; bias [Hq,R] fp32; lse [B,Lq,Hq]
    fp32 (rattn_prefill's out and lse); dq like q, dk/dv like k, dbias like bias, all fp32;
    workspace a device tensor of at least rattn_prefill_backward_workspace_bytes(B, Lq, Lk, Hq,
    Hkv) bytes."""
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    R = bias.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().rattn_prefill_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(out), _ptr(dout), _ptr(lse),
                                         _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbias), B, Lq, Lk, Hq, Hkv, D, R,
                                         int(window), _ptr(workspace), ws_bytes, _stream(stream)))


def rattn_decode_num_splits(B: int, n_q: int, Hq: int, Hkv: int, max_ctx_len: int, num_splits: int = 0) -> int:
    return load().rattn_decode_num_splits(B, n_q, Hq, Hkv, max_ctx_len, num_splits)


def rattn_decode_workspace_bytes(B: int, n_q: int, Hq: int, Hkv: int, max_ctx_len: int,
                                 num_splits: int = 0) -> int:
    return load().rattn_decode_workspace_bytes(B, n_q, Hq, Hkv, max_ctx_len, num_splits)


def rattn_decode_paged(q, k_cache, v_cache, block_table, ctx_lens, windows, bias, out, lse,
                       max_ctx_len: int, num_splits: int = 0, workspace=None, stream=None) -> None:
    """q [B,n_q,Hq,128] bf16; caches [num_blocks,128,Hkv,128] bf16; block_table [B,mb] int32;
    ctx_lens [B] int32 (including the n_q queries); windows [B] int32 or None; bias [Hq,R]
    fp32; out like q; lse [B,n_q,Hq] fp32 or None; workspace a uint8 device tensor of at
    least rattn_decode_workspace_bytes(...) bytes."""
    B, n_q, Hq, D = q.shape
    num_blocks, bs, Hkv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    mb = block_table.shape[1]
    R = bias.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().rattn_decode_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(ctx_lens),
                                     _ptr(windows), _ptr(bias), _ptr(out), _ptr(lse), B, n_q, Hq, Hkv, D, bs, R,
                                     num_blocks, mb, int(max_ctx_len), int(num_splits), _ptr(workspace), ws_bytes,
                                     _stream(stream)))


def rattn_decode_paged_noalloc_max_scratch_bytes() -> int:
    return load().rattn_decode_paged_noalloc_max_scratch_bytes()


def rattn_decode_paged_noalloc(q, k_cache, v_cache, block_table, ctx_lens, windows, bias, out, lse,
                               max_ctx_len: int, num_splits: int = 0, stream=None) -> None:
    """rattn_decode_paged without a workspace: the split partials go to the library's static
    per-device scratch (calls that overlap on one device race); same arguments otherwise."""
    B, n_q, Hq, D = q.shape
    num_blocks, bs, Hkv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    mb = block_table.shape[1]
    R = bias.shape[1]
    _check(load().rattn_decode_paged_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                             _ptr(ctx_lens), _ptr(windows), _ptr(bias), _ptr(out), _ptr(lse), B,
                                             n_q, Hq, Hkv, D, bs, R, num_blocks, mb, int(max_ctx_len),
                                             int(num_splits), _stream(stream)))


# ---- conveniences that allocate the outputs (torch device memory) and call the above ----
_prefill_ws = {}


def prefill_workspace(nbytes: int, device, stream=None):
    """A zero-filled workspace of at least nbytes for calls on `stream` (default: the
    current stream of `device`), kept and reused by later calls on that stream (prefill
    calls leave it zero-filled).  One workspace per (device, stream): calls on one stream
    run in order, so they never share it concurrently; calls on different streams get
    different workspaces.  It is allocated on that stream, so growing it (the old one is
    released to torch's allocator) stays ordered after the calls that used it."""
    import torch
    device = torch.device(device)
    if stream is None:
        stream = torch.cuda.current_stream(device)
    handle = _stream(stream)
    key = (str(device), handle)
    ws = _prefill_ws.get(key)
    if ws is None or ws.numel() < nbytes:
        ctx = torch.cuda.stream(stream) if hasattr(stream, "cuda_stream") else torch.cuda.device(device)
        with ctx:
            ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=device)
        _prefill_ws[key] = ws
    return ws


def prefill(q, k, v, bias, window: int = 0, want_lse: bool = True, kv_splits: int = 0, workspace=None,
            stream=None) -> Tuple:
    import torch
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if want_lse else None
    if workspace is None:
        n = rattn_prefill_workspace_bytes(q.shape[0], q.shape[1], k.shape[1], q.shape[2], k.shape[2], window,
                                          _dtype_code(q), kv_splits)
        workspace = prefill_workspace(n, q.device, stream) if n > 0 else None
    rattn_prefill(q, k, v, bias, out, lse, window, kv_splits, workspace, stream)
    return out, lse


def prefill_tokbias(q, k, v, bias_tok, window: int = 0, want_lse: bool = True, kv_splits: int = 0,
                    workspace=None, stream=None) -> Tuple:
    import torch
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if want_lse else None
    if workspace is None:
        n = rattn_prefill_workspace_bytes(q.shape[0], q.shape[1], k.shape[1], q.shape[2], k.shape[2], window,
                                          RATTN_BF16, kv_splits)
        workspace = prefill_workspace(n, q.device, stream) if n > 0 else None
    rattn_prefill_tokbias(q, k, v, bias_tok, out, lse, window, kv_splits, workspace, stream)
    return out, lse


def prefill_backward(q, k, v, bias, out, lse, dout, window: int = 0, stream=None) -> Tuple:
    """Allocate fp32 gradients and a workspace, call rattn_prefill_backward; returns
    (dq, dk, dv, dbias)."""
    import torch
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    dk = torch.empty(k.shape, dtype=torch.float32, device=q.device)
    dv = torch.empty(v.shape, dtype=torch.float32, device=q.device)
    dbias = torch.empty(bias.shape, dtype=torch.float32, device=q.device)
    n = rattn_prefill_backward_workspace_bytes(q.shape[0], q.shape[1], k.shape[1], q.shape[2], k.shape[2])
    ws = torch.empty(n, dtype=torch.uint8, device=q.device)
    rattn_prefill_backward(q, k, v, bias, out, dout, lse, dq, dk, dv, dbias, window, ws, stream)
    return dq, dk, dv, dbias


def prefill_paged(q, k_cache, v_cache, block_table, ctx_lens, bias, max_ctx_len: int, window: int = 0,
                  want_lse: bool = True, workspace="auto", stream=None, cu_seqlens_q=None, max_q_len: int = 0) -> Tuple:
    """workspace "auto": the cached zero-filled prefill workspace of q's device and the call's
    stream (job queue); None: one workgroup per job; else a tensor as for rattn_prefill_paged."""
    import torch
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device) if want_lse else None
    if isinstance(workspace, str):
        workspace = prefill_workspace(PREFILL_PAGED_WORKSPACE_BYTES, q.device, stream)
    rattn_prefill_paged(q, k_cache, v_cache, block_table, ctx_lens, bias, out, lse, max_ctx_len, window, workspace,
                        stream, cu_seqlens_q, max_q_len)
    return out, lse


def decode_workspace(B, n_q, Hq, Hkv, max_ctx_len, num_splits=0, device="cuda"):
    import torch
    n = rattn_decode_workspace_bytes(B, n_q, Hq, Hkv, max_ctx_len, num_splits)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def decode_paged(q, k_cache, v_cache, block_table, ctx_lens, windows, bias, max_ctx_len: int,
                 num_splits: int = 0, want_lse: bool = True, workspace=None, stream=None) -> Tuple:
    import torch
    B, n_q, Hq, _ = q.shape
    Hkv = k_cache.shape[2]
    if workspace is None:
        workspace = decode_workspace(B, n_q, Hq, Hkv, max_ctx_len, num_splits, q.device)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if want_lse else None
    rattn_decode_paged(q, k_cache, v_cache, block_table, ctx_lens, windows, bias, out, lse, max_ctx_len,
                       num_splits, workspace, stream)
    return out, lse
