"""Shared helpers of the GPU tests: upload the seeded inputs, compare with
the oracle.  The oracle never sees a value produced by the HIP library."""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from block_causal_linear_phi_amd import workloads as wl

DEV = torch.device("cuda:0")
TOL = {"f32": 1e-5, "bf16": 1e-2}


def to_device(raw: np.ndarray, dtype: str) -> torch.Tensor:
    raw = np.ascontiguousarray(raw)
    if dtype == "bf16":
        return torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(raw).to(DEV)


def rand(shape, seed: int, dtype: str, scale: float = 1.0):
    """(host fp32 values, device tensor) holding the same numbers."""
    vals, raw = wl.draw(shape, seed, scale, dtype)
    return vals, to_device(raw, dtype)


def relerr(gpu, ref) -> float:
    g = gpu.detach().float().cpu().numpy().astype(np.float64) if isinstance(gpu, torch.Tensor) else gpu
    return float(np.max(np.abs(g - ref)) / max(float(np.max(np.abs(ref))), 1e-300))


def device_workload(w: wl.Workload, step: int = 0, keep=(), n_tokens=None):
    """Device q, k, v of workload w (slice by slice, threaded draws), plus the
    host fp32 values of the (b, h) slices listed in `keep`."""
    n = w.N if n_tokens is None else n_tokens
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = {t: torch.empty((w.B, w.H, n, w.d), dtype=tdt, device=DEV) for t in ("q", "k", "v")}
    host = {}
    jobs = [(t, b, h) for t in ("q", "k", "v") for b in range(w.B) for h in range(w.H)]

    def one(job):
        t, b, h = job
        return job, wl.slice_qkv(w, t, b, h, step, n)

    with ThreadPoolExecutor(8) as ex:
        for (t, b, h), (vals, raw) in ex.map(one, jobs):
            dev[t][b, h].copy_(to_device(raw, w.dtype))
            if (b, h) in keep:
                host[(t, b, h)] = vals
    return dev, host


def host_bits(t: torch.Tensor) -> np.ndarray:
    """A device tensor's values on the host: fp32 as is, bf16 widened to fp32
    exactly (one copy of the whole tensor)."""
    if t.dtype == torch.bfloat16:
        raw = t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
        return wl.bf16_bits_to_f32(raw)
    return t.detach().float().cpu().numpy()


def compare_slices(slices, check, workers: int = 8):
    """Runs check(b, h) -> relative error for every (b, h) in `slices` in a
    thread pool (numpy releases the GIL; BLAS limited to one thread per
    worker) and returns the worst error and its slice."""
    from threadpoolctl import threadpool_limits

    def one(bh):
        return check(*bh), bh

    with threadpool_limits(limits=1), ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(one, list(slices)))
    return max(results)
