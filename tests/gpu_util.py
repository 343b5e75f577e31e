"""Helpers for the GPU tests: move synthetic inputs to the device, compare with the oracle."""
from __future__ import annotations

import numpy as np

# Parity bar (bf16 inputs, fp32 accumulation) against the fp64 oracle, for every workload:
O_MAX_ABS = 2e-2     # max |gpu - oracle| over all output elements
O_MEAN_ABS = 2e-3    # mean |gpu - oracle| over all output elements
LSE_MAX_ABS = 1e-3   # max |gpu - oracle| of the natural-log log-sum-exp


def dev(a: np.ndarray, device="cuda"):
    """numpy -> torch device tensor; uint16 arrays are bf16 bit patterns."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def host(t) -> np.ndarray:
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def compare(out_gpu: np.ndarray, lse_gpu: np.ndarray, out_ref: np.ndarray, lse_ref: np.ndarray, what: str = ""):
    assert out_gpu.shape == out_ref.shape, (out_gpu.shape, out_ref.shape)
    assert np.isfinite(out_gpu).all(), f"{what}: non-finite output"
    err = np.abs(out_gpu - out_ref)
    lerr = np.abs(lse_gpu - lse_ref)
    msg = f"{what}: O max {err.max():.3e} mean {err.mean():.3e}; LSE max {lerr.max():.3e}"
    print(msg, flush=True)
    assert err.max() <= O_MAX_ABS, msg
    assert err.mean() <= O_MEAN_ABS, msg
    assert lerr.max() <= LSE_MAX_ABS, msg
    return err.max(), err.mean(), lerr.max()


def decode_to_device(case):
    import torch
    return dict(q=dev(case.q), k_cache=dev(case.k_cache), v_cache=dev(case.v_cache),
                block_table=dev(case.block_table), ctx_lens=dev(case.ctx_lens),
                windows=dev(case.windows), bias=dev(case.bias))
