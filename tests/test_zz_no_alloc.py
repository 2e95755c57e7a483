"""The workspace-free block-cache apply (sva_block_cache_apply_noalloc),
called through the C ABI: its output equals sva_block_cache_apply's on the
cached-step workload (16 heads, one 3 x 30 x 52 block against a 6-block fp32
cache), and again on a second, smaller call right after it (4 heads, a
2 x 9 x 13 block), whose reduction grid and scratch layout differ; both
outputs are also within the bf16 bar of the oracle.  Neither call allocates
device memory."""
import ctypes
import sys

import numpy as np
import pytest
import torch

from block_causal_linear_phi_amd import sva
from block_causal_linear_phi_amd import workloads as wl
from gpu_helpers import DEV, rand, relerr
from oracle import sva_oracle as orc

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _call_noalloc(S, z, q, k, v, out, fg, t0, split):
    desc = sva.make_desc(q.shape[0], q.shape[1], q.shape[3], fg, fg[0], t0=t0, rope=True, split=split,
                         eps=1e-6, dtype=sva.SVA_BF16)
    return sva.lib().sva_block_cache_apply_noalloc(ctypes.byref(desc), S.data_ptr(), z.data_ptr(), q.data_ptr(),
                                                   k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                                   torch.cuda.current_stream().cuda_stream)


def _case(B, H, fg, t0, seed):
    d, split = 64, (16, 24, 24)
    n = fg[0] * fg[1] * fg[2]
    q, qd = rand((B, H, n, d), seed, "bf16")
    k, kd = rand((B, H, n, d), seed + 1, "bf16")
    v, vd = rand((B, H, n, d), seed + 2, "bf16")
    S0 = wl.draw((B, H, d, d), seed + 3, 30.0, "f32")[0]
    z0 = np.abs(wl.draw((B, H, d), seed + 4, 60.0, "f32")[0])
    return (q, k, v, S0, z0), (qd, kd, vd, torch.from_numpy(S0).to(DEV), torch.from_numpy(z0).to(DEV)), split


@pytest.mark.parametrize("order", ["large_then_small", "small_then_large"])
def test_noalloc_equals_the_workspace_apply(order):
    cases = [(1, 16, (3, 30, 52), 18, 501), (1, 4, (2, 9, 13), 4, 601)]
    if order == "small_then_large":
        cases = cases[::-1]
    prepared = []
    for B, H, fg, t0, seed in cases:
        host, dev, split = _case(B, H, fg, t0, seed)
        out_ref = sva.sva_block_cache_apply(dev[3], dev[4], dev[0], dev[1], dev[2], fg, t0=t0, rope=True,
                                            split=split, eps=1e-6)
        outs = torch.full_like(out_ref, 3.0)
        prepared.append((B, H, fg, t0, host, dev, split, out_ref, outs))
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    for B, H, fg, t0, host, dev, split, out_ref, out in prepared:  # back to back, no sync between
        _say(f"noalloc B={B} H={H} block {fg} t0={t0}")
        st = _call_noalloc(dev[3], dev[4], dev[0], dev[1], dev[2], out, fg, t0, split)
        assert st == sva.SVA_OK, sva.status_string(st)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    for B, H, fg, t0, host, dev, split, out_ref, out in prepared:
        assert torch.equal(out.view(torch.int16), out_ref.view(torch.int16))
        q, k, v, S0, z0 = host
        ref = orc.block_cache_apply(S0.astype(np.float64), z0.astype(np.float64), q, k, v, fg, t0=t0, rope=True,
                                    split=split, eps=1e-6)
        assert relerr(out, ref) <= 1e-2


def test_noalloc_rejects_a_descriptor_beyond_the_scratch():
    """(R + B*H) pieces of 16.6 KB and B*H prefix operands past 16 MiB:
    SVA_ERR_WORKSPACE before any launch (the pointers are never touched)."""
    fg = (1, 2, 8)
    n = fg[0] * fg[1] * fg[2]
    q = torch.zeros((1, 1024, n, 64), dtype=torch.bfloat16, device=DEV)
    S = torch.zeros((1, 1024, 64, 64), dtype=torch.float32, device=DEV)
    z = torch.zeros((1, 1024, 64), dtype=torch.float32, device=DEV)
    out = torch.empty_like(q)
    st = _call_noalloc(S, z, q, q, q, out, fg, 0, (16, 24, 24))
    assert st == sva.SVA_ERR_WORKSPACE
