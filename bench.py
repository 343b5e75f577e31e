"""Throughput of relative-bias GQA attention on one MI355X.

One step is one call of the hot path on one batch of seeded synthetic input that is
already resident in HBM.  The headline line is the full-attention chunked prefill, the
largest single-GPU workload (batch 1, an 8192-token chunk at positions 24576..32767 over
32768 keys, 16 query / 2 KV heads, d 128, bias table 8192, bf16): attention TFLOP/s counted
over the visible (query, key) pairs only.  The same JSON line carries the other workloads
(fp32 tiny prefill, 8K sliding-window prefill, batch-64 paged decode, 1M-token 9-query
verify, paged prefill, K/V short convolution, backward, token-dependent bias), each timed the
same way: prefill in TFLOP/s against the bf16 MFMA peak, decode in KV GB/s (bytes the method
must move) against the HBM peak, and practical ceilings measured in the same process (a
large bf16 GEMM through torch, a device copy and a read stream).

Timing: the step repeated, untimed, for at least S ms of wall clock (the GPU raises its
clock over its first tens of milliseconds under load; S 0 skips this), then W untimed
warm-up steps, then exactly K steps between two hipEvents recorded on the stream the
kernels are launched on, with a device synchronisation on both sides.
The CPU oracle (fp64) is timed on a bounded sample of the headline workload (every n-th
query row, about 10-20 s of host time).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms S] [--workloads a,b,...]
                       [--no-cpu-baseline] [--only HEADLINE]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill attention TFLOP/s (% bf16 MFMA peak); decode KV GB/s (% HBM peak)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
HEADLINE = "chunked_prefill_32k"
ALL_WORKLOADS = ["tiny_prefill_fp32", "swa_prefill_8k", "chunked_prefill_32k", "paged_decode_b64", "mtp_verify_1m",
                 "paged_prefill_b4", "kv_sconv_32k", "swa_prefill_8k_bwd", "swa_prefill_8k_tokbias"]
HEAD_DIM = 128
KERNEL_SOURCES = {
    "prefill": ["relative_bias_gqa_amd/csrc/prefill.hip", "relative_bias_gqa_amd/csrc/prefill_bf16.hip",
                "relative_bias_gqa_amd/csrc/device_common.hpp", "relative_bias_gqa_amd/csrc/launch.hpp"],
    "decode": ["relative_bias_gqa_amd/csrc/decode.hip", "relative_bias_gqa_amd/csrc/device_common.hpp",
               "relative_bias_gqa_amd/csrc/launch.hpp"],
    "sconv": ["relative_bias_gqa_amd/csrc/sconv.hip", "relative_bias_gqa_amd/csrc/device_common.hpp",
              "relative_bias_gqa_amd/csrc/launch.hpp"],
    "backward": ["relative_bias_gqa_amd/csrc/backward.hip", "relative_bias_gqa_amd/csrc/backward.hpp",
                 "relative_bias_gqa_amd/csrc/device_common.hpp"],
}


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------------------
# algorithmic work
# ---------------------------------------------------------------------------------------
def visible_keys(p: np.ndarray, window: int) -> np.ndarray:
    """Keys visible to queries at absolute positions p (causal, optional window)."""
    n = p.astype(np.int64) + 1
    return np.minimum(n, window) if window > 0 else n


def prefill_flops(B: int, Lq: int, Lk: int, Hq: int, window: int) -> int:
    """4 * D * Hq * sum over query rows of visible keys (QK^T and PV, 2 flop per MAC)."""
    p = np.arange(Lq, dtype=np.int64) + (Lk - Lq)
    return int(4 * HEAD_DIM * Hq * B * visible_keys(p, window).sum())


def decode_bytes(ctx: np.ndarray, windows: np.ndarray, n_q: int, Hq: int, Hkv: int, R: int) -> int:
    """HBM bytes the paged decode must move: every K/V row some query can see (bf16), the
    queries, outputs (bf16) and lse (fp32), the bias entries the distances reach (fp32)
    and the block-table entries of the blocks holding visible keys."""
    total = 0
    max_dist = 0
    for c, w in zip(ctx.tolist(), windows.tolist()):
        lo = max(0, c - n_q - w + 1) if w > 0 else 0
        vis = c - lo
        total += vis * Hkv * HEAD_DIM * 2 * 2
        total += ((c - 1) // 128 - lo // 128 + 1) * 4
        max_dist = max(max_dist, c - 1 - lo)
    B = len(ctx)
    total += B * n_q * Hq * HEAD_DIM * 2 * 2 + B * n_q * Hq * 4
    total += Hq * min(R, max_dist + 1) * 4
    return total


# ---------------------------------------------------------------------------------------
# traffic recorded from rocprofv3 PMC runs
# ---------------------------------------------------------------------------------------
def source_digest(kind: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(kind: str, workload: str):
    """HBM bytes per launch measured with FETCH_SIZE / WRITE_SIZE (scaled by a copy-kernel
    calibration), read from profiles/<kind>_<workload>_traffic.txt; None if absent or if
    the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kind}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"^source_digest:\s*(\S+)", text, re.M)
    m_b = re.search(r"^traffic_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not m_src or not m_b or m_src.group(1) != source_digest(kind):
        return None
    return float(m_b.group(1))


# ---------------------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------------------
class PrefillRun:
    kind = "prefill"

    def __init__(self, name, torch, rb, synth, dev):
        self.name = name
        c = synth.WORKLOAD_FNS[name]()
        self.case = c
        self.q, self.k, self.v, self.bias = dev(c.q), dev(c.k), dev(c.v), dev(c.bias)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty(self.q.shape[:3], dtype=torch.float32, device=self.q.device)
        self.rb = rb
        self.work = prefill_flops(c.B, c.Lq, c.Lk, c.Hq, c.window)
        self.unit, self.peak, self.bound = "TFLOP/s", PEAK_BF16_TFLOPS, "mfma"
        self.config = {"workload": name, "batch": c.B, "q_len": c.Lq, "kv_len": c.Lk, "q_heads": c.Hq,
                       "kv_heads": c.Hkv, "head_dim": HEAD_DIM, "window": c.window, "bias_len": c.R,
                       "dtype": c.dtype}
        self.dtype = "bf16" if c.dtype == "bf16" else "f32"
        # the library's key-range split plan, with its (zero-filled) workspace allocated here,
        # outside the timed region
        nbytes = rb.rattn_prefill_workspace_bytes(c.B, c.Lq, c.Lk, c.Hq, c.Hkv, c.window,
                                                  rb.RATTN_BF16 if c.dtype == "bf16" else rb.RATTN_FP32)
        self.ws = torch.zeros(nbytes, dtype=torch.uint8, device=self.q.device) if nbytes else None
        self.config["kv_split_workspace_bytes"] = nbytes

    def step(self, stream):
        self.rb.rattn_prefill(self.q, self.k, self.v, self.bias, self.out, self.lse, self.case.window, 0, self.ws,
                              stream)

    def rate(self, seconds):
        return self.work / seconds / 1e12

    def finite(self):
        import torch
        return bool(torch.isfinite(self.out.float()).all()) and bool(torch.isfinite(self.lse).all())

    def free(self):
        del self.q, self.k, self.v, self.bias, self.out, self.lse, self.ws


class DecodeRun:
    kind = "decode"

    def __init__(self, name, torch, rb, synth, dev):
        self.name = name
        c = synth.WORKLOAD_FNS[name]()
        self.case = c
        self.q, self.kc, self.vc = dev(c.q), dev(c.k_cache), dev(c.v_cache)
        self.bt, self.ctx, self.win, self.bias = dev(c.block_table), dev(c.ctx_lens), dev(c.windows), dev(c.bias)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty(self.q.shape[:3], dtype=torch.float32, device=self.q.device)
        self.max_ctx = c.max_ctx_len
        self.ws = rb.decode_workspace(c.B, c.n_q, c.Hq, c.Hkv, self.max_ctx, 0, self.q.device)
        self.splits = rb.rattn_decode_num_splits(c.B, c.n_q, c.Hq, c.Hkv, self.max_ctx, 0)
        self.rb = rb
        self.work = decode_bytes(c.ctx_lens, c.windows, c.n_q, c.Hq, c.Hkv, c.R)
        self.unit, self.peak, self.bound = "GB/s", PEAK_HBM_GBS, "hbm"
        self.config = {"workload": name, "batch": c.B, "q_per_seq": c.n_q, "q_heads": c.Hq, "kv_heads": c.Hkv,
                       "head_dim": HEAD_DIM, "block_size": 128, "ctx_min": int(c.ctx_lens.min()),
                       "ctx_max": self.max_ctx, "ctx_sum": int(c.ctx_lens.sum()),
                       "windows": sorted(set(int(w) for w in c.windows)), "bias_len": c.R,
                       "kv_splits": self.splits, "dtype": "bf16"}
        self.dtype = "bf16"

    def step(self, stream):
        self.rb.rattn_decode_paged(self.q, self.kc, self.vc, self.bt, self.ctx, self.win, self.bias, self.out,
                                   self.lse, self.max_ctx, 0, self.ws, stream)

    def rate(self, seconds):
        return self.work / seconds / 1e9

    def finite(self):
        import torch
        return bool(torch.isfinite(self.out.float()).all()) and bool(torch.isfinite(self.lse).all())

    def free(self):
        del self.q, self.kc, self.vc, self.bt, self.ctx, self.win, self.bias, self.out, self.lse, self.ws


class PagedPrefillRun:
    """Chunked prefill over a paged KV cache: per-sequence contexts, one chunk length."""
    kind = "prefill"

    def __init__(self, name, torch, rb, synth, dev):
        self.name = name
        c = synth.WORKLOAD_FNS[name]()
        self.case = c
        self.q, self.kc, self.vc = dev(c.q), dev(c.k_cache), dev(c.v_cache)
        self.bt, self.ctx, self.bias = dev(c.block_table), dev(c.ctx_lens), dev(c.bias)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty(self.q.shape[:3], dtype=torch.float32, device=self.q.device)
        self.max_ctx = c.max_ctx_len
        self.window = int(c.windows[0])
        # the job queue's (zero-filled) workspace, allocated here, outside the timed region
        self.ws = torch.zeros(rb.PREFILL_PAGED_WORKSPACE_BYTES, dtype=torch.uint8, device=self.q.device)
        self.rb = rb
        self.work = sum(prefill_flops(1, c.n_q, int(ctx), c.Hq, self.window) for ctx in c.ctx_lens)
        self.unit, self.peak, self.bound = "TFLOP/s", PEAK_BF16_TFLOPS, "mfma"
        self.config = {"workload": name, "batch": c.B, "q_len": c.n_q, "ctx_lens": [int(x) for x in c.ctx_lens],
                       "q_heads": c.Hq, "kv_heads": c.Hkv, "head_dim": HEAD_DIM, "block_size": 128,
                       "window": self.window, "bias_len": c.R, "dtype": "bf16"}
        self.dtype = "bf16"

    def step(self, stream):
        self.rb.rattn_prefill_paged(self.q, self.kc, self.vc, self.bt, self.ctx, self.bias, self.out, self.lse,
                                    self.max_ctx, self.window, self.ws, stream)

    def rate(self, seconds):
        return self.work / seconds / 1e12

    def finite(self):
        import torch
        return bool(torch.isfinite(self.out.float()).all()) and bool(torch.isfinite(self.lse).all())

    def free(self):
        del self.q, self.kc, self.vc, self.bt, self.ctx, self.bias, self.out, self.lse, self.ws


class SconvRun:
    """Short convolution of new K/V tokens written into the paged caches (HBM-bound)."""
    kind = "sconv"

    def __init__(self, name, torch, rb, synth, dev):
        self.name = name
        c = synth.WORKLOAD_FNS[name]()
        self.case = c
        self.kn, self.vn, self.wk, self.wv = dev(c.k_new), dev(c.v_new), dev(c.w_k), dev(c.w_v)
        self.kc, self.vc, self.ks, self.vs = dev(c.k_cache), dev(c.v_cache), dev(c.k_state), dev(c.v_state)
        self.bt, self.ctx, self.cu = dev(c.block_table), dev(c.ctx_lens), dev(c.cu_seqlens)
        self.max_new = int(c.n_new.max())
        self.rb = rb
        Hkv = c.k_new.shape[1]
        row = Hkv * HEAD_DIM * 2
        # per new token: its K and V rows read, four cache rows written; per sequence the
        # state rows of up to three earlier positions read; the weights
        prior = sum(min(3, int(x) - int(n)) for x, n in zip(c.ctx_lens, c.n_new))
        self.work = int(6 * row * c.k_new.shape[0] + 2 * row * prior + 2 * 4 * Hkv * HEAD_DIM * 4)
        self.unit, self.peak, self.bound = "GB/s", PEAK_HBM_GBS, "hbm"
        self.config = {"workload": name, "batch": len(c.ctx_lens), "new_tokens": [int(x) for x in c.n_new],
                       "ctx_lens": [int(x) for x in c.ctx_lens], "kv_heads": Hkv, "head_dim": HEAD_DIM,
                       "block_size": 128, "taps": 4, "dtype": "bf16"}
        self.dtype = "bf16"

    def step(self, stream):
        self.rb.rattn_kv_sconv_write(self.kn, self.vn, self.wk, self.wv, self.kc, self.vc, self.ks, self.vs, self.bt,
                                     self.ctx, self.cu, self.max_new, stream)

    def rate(self, seconds):
        return self.work / seconds / 1e9

    def finite(self):
        import torch
        return bool(torch.isfinite(self.kc.float()).all())

    def free(self):
        del self.kn, self.vn, self.wk, self.wv, self.kc, self.vc, self.ks, self.vs, self.bt, self.ctx, self.cu


class BackwardRun:
    """Gradients of a bf16 prefill (dq, dk, dv, dr) for a given output gradient; the forward's
    out and lse are computed once, outside the timed region."""
    kind = "backward"

    def __init__(self, name, torch, rb, synth, dev):
        self.name = name
        bc = synth.WORKLOAD_FNS[name]()
        c = bc.fwd
        self.case = c
        self.q, self.k, self.v, self.bias, self.dout = dev(c.q), dev(c.k), dev(c.v), dev(c.bias), dev(bc.dout)
        self.out, self.lse = rb.prefill(self.q, self.k, self.v, self.bias, c.window)
        f32 = torch.float32
        self.dq = torch.empty(self.q.shape, dtype=f32, device=self.q.device)
        self.dk = torch.empty(self.k.shape, dtype=f32, device=self.q.device)
        self.dv = torch.empty(self.v.shape, dtype=f32, device=self.q.device)
        self.dbias = torch.empty(self.bias.shape, dtype=f32, device=self.q.device)
        self.ws = torch.empty(rb.rattn_prefill_backward_workspace_bytes(c.B, c.Lq, c.Lk, c.Hq, c.Hkv), dtype=torch.uint8,
                              device=self.q.device)
        self.rb = rb
        # five products per visible (query, key) pair and head: QK^T again, dO V^T, P^T dO,
        # dS^T Q, dS K (2 flop per multiply-add over the 128 dims)
        self.work = prefill_flops(c.B, c.Lq, c.Lk, c.Hq, c.window) * 5 // 2
        self.unit, self.peak, self.bound = "TFLOP/s", PEAK_BF16_TFLOPS, "mfma"
        self.config = {"workload": name, "batch": c.B, "q_len": c.Lq, "kv_len": c.Lk, "q_heads": c.Hq,
                       "kv_heads": c.Hkv, "head_dim": HEAD_DIM, "window": c.window, "bias_len": c.R,
                       "dtype": "bf16", "grads": "fp32"}
        self.dtype = "bf16"

    def step(self, stream):
        self.rb.rattn_prefill_backward(self.q, self.k, self.v, self.bias, self.out, self.dout, self.lse, self.dq,
                                       self.dk, self.dv, self.dbias, self.case.window, self.ws, stream)

    def rate(self, seconds):
        return self.work / seconds / 1e12

    def finite(self):
        import torch
        return all(bool(torch.isfinite(t).all()) for t in (self.dq, self.dk, self.dv, self.dbias))

    def free(self):
        del self.q, self.k, self.v, self.bias, self.dout, self.out, self.lse, self.dq, self.dk, self.dv
        del self.dbias, self.ws


class TokBiasRun(PrefillRun):
    """Prefill with a token-dependent table (bf16 [B, Lq, Hq, R], one per query row)."""

    def __init__(self, name, torch, rb, synth, dev):
        self.name = name
        tc = synth.WORKLOAD_FNS[name]()
        c = tc.fwd
        self.case = c
        self.q, self.k, self.v, self.bias = dev(c.q), dev(c.k), dev(c.v), dev(tc.bias_tok)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty(self.q.shape[:3], dtype=torch.float32, device=self.q.device)
        self.rb = rb
        self.work = prefill_flops(c.B, c.Lq, c.Lk, c.Hq, c.window)
        self.unit, self.peak, self.bound = "TFLOP/s", PEAK_BF16_TFLOPS, "mfma"
        nbytes = rb.rattn_prefill_workspace_bytes(c.B, c.Lq, c.Lk, c.Hq, c.Hkv, c.window, rb.RATTN_BF16)
        self.ws = torch.zeros(nbytes, dtype=torch.uint8, device=self.q.device) if nbytes else None
        self.config = {"workload": name, "batch": c.B, "q_len": c.Lq, "kv_len": c.Lk, "q_heads": c.Hq,
                       "kv_heads": c.Hkv, "head_dim": HEAD_DIM, "window": c.window, "bias_len": tc.R,
                       "bias": "token-dependent bf16 [B, Lq, Hq, R]", "dtype": "bf16",
                       "kv_split_workspace_bytes": nbytes}
        self.dtype = "bf16"

    def step(self, stream):
        self.rb.rattn_prefill_tokbias(self.q, self.k, self.v, self.bias, self.out, self.lse, self.case.window, 0,
                                      self.ws, stream)


RUN_CLASSES = {"paged_decode_b64": DecodeRun, "mtp_verify_1m": DecodeRun, "paged_prefill_b4": PagedPrefillRun,
               "kv_sconv_32k": SconvRun, "swa_prefill_8k_bwd": BackwardRun, "swa_prefill_8k_tokbias": TokBiasRun}


def settle_clock(run, torch, stream, ms: float) -> int:
    """Repeat the step, untimed, for at least `ms` milliseconds of wall clock."""
    if ms <= 0:
        return 0
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < ms / 1e3:
        for _ in range(8):
            run.step(stream)
        n += 8
        torch.cuda.synchronize()
    return n


def time_steps(run, torch, steps: int, warmup: int, settle_ms: float = 0.0):
    """Average seconds per step over exactly `steps` steps, hipEvents on the launch stream."""
    stream = torch.cuda.current_stream()
    settle_clock(run, torch, stream, settle_ms)
    for _ in range(warmup):
        run.step(stream)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        run.step(stream)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3 / steps


def result_of(run, sec: float):
    a = run.rate(sec)
    return {"workload": run.name, "ms_per_step": round(sec * 1e3, 4), "value": round(a, 3), "unit": run.unit,
            "frac_of_peak": round(a / run.peak, 4), "bound": run.bound, "work_per_step": run.work,
            "config": run.config}


# ---------------------------------------------------------------------------------------
# CPU oracle baseline on a bounded sample of the headline workload
# ---------------------------------------------------------------------------------------
def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def practical_ceilings(torch):
    """Context for the roofline, measured in this process: a large bf16 GEMM through torch
    (hipBLASLt), a device-to-device copy (read + write) and a read stream (sum of a large
    tensor), each timed with hipEvents after a warm-up."""
    dev = "cuda:0"
    res = {}
    n = 8192
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    reps = 20
    for _ in range(reps):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / reps
    res["bf16_gemm_tflops"] = round(2.0 * n ** 3 / sec / 1e12, 1)
    res["bf16_gemm_shape"] = f"{n}x{n}x{n}"
    del a, b
    nbytes = 2 << 30
    src = torch.empty(nbytes // 4, device=dev, dtype=torch.float32).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0.record()
    reps = 10
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    res["hbm_copy_gbs"] = round(2.0 * nbytes / (e0.elapsed_time(e1) / 1e3 / reps) / 1e9, 1)
    out = torch.empty((), device=dev, dtype=torch.float32)
    for _ in range(2):
        torch.sum(src, dim=0, out=out)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        torch.sum(src, dim=0, out=out)
    e1.record()
    torch.cuda.synchronize()
    res["hbm_read_gbs"] = round(nbytes / (e0.elapsed_time(e1) / 1e3 / reps) / 1e9, 1)
    res["note"] = "practical ceilings for context (torch matmul bf16, device copy counted as read + write, " \
                  "torch.sum over 2 GiB); the roofline peaks are the published ones"
    del src, dst
    torch.cuda.empty_cache()
    return res


def cpu_baseline(case, stride: int):
    import oracle
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    rows = list(range(stride - 1, case.Lq, stride))
    p = np.array(rows, dtype=np.int64) + (case.Lk - case.Lq)
    flops = int(4 * HEAD_DIM * case.Hq * case.B * visible_keys(p, case.window).sum())
    t0 = time.perf_counter()
    oracle.ref_prefill_rows(case.q, case.k, case.v, case.bias, case.window, [(0, t) for t in rows],
                            num_threads=threads)
    sec = time.perf_counter() - t0
    return {"value": round(flops / sec / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"{case.name}: every {stride}th query row ({len(rows)} of {case.Lq} rows x {case.Hq} heads, "
                      f"{flops:.4e} algorithmic flop) in {sec:.2f} s, fp64 on {threads} threads"}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed repetition of the step before the warm-up, in ms of wall clock")
    ap.add_argument("--workloads", default=",".join(ALL_WORKLOADS),
                    help="comma-separated workloads to time besides the headline")
    ap.add_argument("--only-headline", action="store_true", help="time only the headline workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-stride", type=int, default=4, help="oracle sample: every n-th query row")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the GEMM / copy ceiling measurements")
    ap.add_argument("--only", default=None,
                    help="time just this workload and print its own result line (for profiler runs)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="also run 4 device-to-device copies of this many MiB (byte-counter calibration)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the attention path has no "
              "multi-GPU mode: a tensor-parallel layout gives each GPU its own share of the heads.",
              file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    import relative_bias_gqa_amd as rb
    from relative_bias_gqa_amd import synth
    rb.load()
    torch.cuda.set_device(0)

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to("cuda:0").view(torch.bfloat16)
        return torch.from_numpy(a).to("cuda:0")

    if args.copy_calib_mib > 0:
        n = args.copy_calib_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: 4 copies of {n} bytes")
        del src, dst
    if args.only:
        if args.only not in ALL_WORKLOADS:
            raise SystemExit(f"unknown workload {args.only}")
        cls = RUN_CLASSES.get(args.only, PrefillRun)
        run = cls(args.only, torch, rb, synth, dev)
        torch.cuda.synchronize()
        sec = time_steps(run, torch, args.steps, args.warmup, args.settle_ms)
        res = result_of(run, sec)
        log(f"[bench] {args.only}: {res['ms_per_step']:.4f} ms/step, {res['value']} {run.unit}")
        print(json.dumps(res), flush=True)
        return 0

    names = [HEADLINE] if args.only_headline else [w for w in args.workloads.split(",") if w]
    if HEADLINE not in names:
        names = [HEADLINE] + names
    results = {}
    headline = None
    for name in names:
        cls = RUN_CLASSES.get(name, PrefillRun)
        t0 = time.time()
        run = cls(name, torch, rb, synth, dev)
        log(f"[bench] {name}: inputs on device in {time.time() - t0:.1f} s; timing {args.steps} steps")
        torch.cuda.synchronize()
        sec = time_steps(run, torch, args.steps, args.warmup, args.settle_ms)
        if not run.finite():
            raise RuntimeError(f"{name}: non-finite output")
        res = result_of(run, sec)
        traffic = recorded_traffic(run.kind, name)
        res["roofline"] = {"bound": run.bound, "achieved": res["value"], "peak": run.peak, "unit": run.unit,
                           "frac": res["frac_of_peak"], "traffic": traffic}
        results[name] = res
        log(f"[bench] {name}: {res['ms_per_step']:.4f} ms/step, {res['value']} {run.unit} "
            f"({100 * res['frac_of_peak']:.1f}% of peak)")
        if name == HEADLINE:
            headline = (run, sec)
            hcase = run.case
        run.free()
        torch.cuda.empty_cache()

    run, sec = headline
    h = results[HEADLINE]
    line = {
        "metric": METRIC,
        "value": h["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle_ms": args.settle_ms,
        "ms_per_step": h["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": run.dtype,
        "data": "synthetic (seeded numpy PCG64: N(0,1) rounded to bf16, bias 0.5*N(0,1) fp32)",
        "config": h["config"],
        "roofline": h["roofline"],
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample of the headline workload")
        line["cpu_baseline"] = cpu_baseline(hcase, args.cpu_stride)
    else:
        line["cpu_baseline"] = None
    if not args.no_ceilings:
        log("[bench] practical ceilings: bf16 GEMM, device copy, read stream")
        try:
            line["practical_ceilings"] = practical_ceilings(torch)
        except Exception as exc:  # context only: never let it cost the measurement
            line["practical_ceilings"] = {"error": f"{type(exc).__name__}: {exc}"}
    line["workloads"] = [results[n] for n in names if n != HEADLINE]
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
