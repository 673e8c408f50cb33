"""Helpers shared by the GPU tests: move seeded bf16 bits to the device, run
the HIP path, and compare with the oracle at the stated tolerances."""
from __future__ import annotations

import os
import sys

import numpy as np

# Parity bar for the attention forward (fp32 accumulation, bf16 P and O):
# max |O err| <= 2e-2, mean |O err| <= 2e-3, max |LSE err| <= 1e-3, each
# measured against the fp64 oracle (not an oracle rounded to bf16).
O_MAX_TOL = 2e-2
O_MEAN_TOL = 2e-3
LSE_MAX_TOL = 1e-3

ORACLE_THREADS = max(1, min(16, os.cpu_count() or 1))


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(bits: np.ndarray, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def to_host_f64(t) -> np.ndarray:
    import torch
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_gpu(q_bits, k_bits, v_bits, causal, scale):
    import torch
    import attention_attn_fwd_08_amd as af
    q, k, v = (to_device(x) for x in (q_bits, k_bits, v_bits))
    o, lse = af.attn_fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def errors(o_gpu: np.ndarray, lse_gpu: np.ndarray, o_ref: np.ndarray, lse_ref: np.ndarray):
    eo = np.abs(o_gpu - o_ref)
    el = np.abs(lse_gpu - lse_ref)
    return float(eo.max()), float(eo.mean()), float(el.max())


def assert_parity(o_gpu, lse_gpu, o_ref, lse_ref, what=""):
    assert np.isfinite(o_gpu).all() and np.isfinite(lse_gpu).all(), f"{what}: non-finite output"
    omax, omean, lmax = errors(o_gpu, lse_gpu, o_ref, lse_ref)
    log(f"  {what}: O max {omax:.3e} mean {omean:.3e}  LSE max {lmax:.3e}")
    assert omax <= O_MAX_TOL, f"{what}: O max err {omax}"
    assert omean <= O_MEAN_TOL, f"{what}: O mean err {omean}"
    assert lmax <= LSE_MAX_TOL, f"{what}: LSE max err {lmax}"
