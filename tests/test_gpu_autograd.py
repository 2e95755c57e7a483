"""GPU parity of the torch.autograd wrapper (forward with saved states,
backward through sva_lin_attn_bwd) against the fp64 oracle's gradients, for
L = sum(out * dout); bar 1e-2 (bf16), as for the backward itself."""
import sys

import numpy as np
import pytest
import torch

from block_causal_linear_phi_amd import block_causal_linear_attention
from block_causal_linear_phi_amd import workloads as wl
from gpu_helpers import DEV, TOL, rand, relerr
from oracle import sva_oracle as orc

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("with_cache", [False, True], ids=["no_cache", "initial_cache"])
def test_autograd_matches_oracle(with_cache):
    print(f"autograd with_cache={with_cache}", flush=True)
    sys.stdout.flush()
    B, H, d, grid, F, split = 1, 2, 64, (6, 5, 7), 2, (16, 24, 24)
    N = grid[0] * grid[1] * grid[2]
    q, qd = rand((B, H, N, d), 61, "bf16")
    k, kd = rand((B, H, N, d), 62, "bf16")
    v, vd = rand((B, H, N, d), 63, "bf16")
    do, dod = rand((B, H, N, d), 64, "bf16")
    S0 = z0 = S0d = z0d = None
    if with_cache:
        S0 = wl.draw((B, H, d, d), 65, 4.0, "f32")[0]
        z0 = np.abs(wl.draw((B, H, d), 66, 8.0, "f32")[0])
        S0d = torch.from_numpy(S0).to(DEV).requires_grad_()
        z0d = torch.from_numpy(z0).to(DEV).requires_grad_()
    for t in (qd, kd, vd):
        t.requires_grad_()
    kw = dict(t0=1, rope=True, split=split, eps=1e-6)
    out = block_causal_linear_attention(qd, kd, vd, grid, F, S0=S0d, z0=z0d, **kw)
    (out.float() * dod.float()).sum().backward()
    torch.cuda.synchronize()
    rq, rk, rv, rS0, rz0 = orc.lin_attn_bwd(q, k, v, do, grid, F, S0=S0, z0=z0, **kw)
    errs = {"dq": relerr(qd.grad, rq), "dk": relerr(kd.grad, rk), "dv": relerr(vd.grad, rv)}
    if with_cache:
        errs["dS0"] = relerr(S0d.grad, rS0)
        errs["dz0"] = relerr(z0d.grad, rz0)
    print(f"  {errs}", flush=True)
    for name, e in errs.items():
        assert e <= TOL["bf16"], (name, e)
