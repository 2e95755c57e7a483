"""GPU parity of the backward (sva_lin_attn_bwd, bf16) against the fp64
oracle's lin_attn_bwd on identical seeded inputs.

The library forms the forward's output again inside the backward (its
denominator term needs dout . out); the oracle recomputes everything in
fp64.  Bar: max|gpu - oracle| / max|oracle| <= 1e-2
for every gradient (bf16 inputs and outputs).  Sizes span several 16-token
tiles, ragged tails, several blocks, both head dims, every RoPE mode, an
initial cache and a final-state gradient; the 720p workload runs at full size
and every head is compared.
"""
import sys

import numpy as np
import pytest
import torch

from block_causal_linear_phi_amd import sva
from block_causal_linear_phi_amd import workloads as wl
from gpu_helpers import DEV, compare_slices, device_workload, host_bits, rand, relerr
from oracle import sva_oracle as orc

pytestmark = pytest.mark.gpu
TOL = 1e-2


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# (name, B, H, d, (T, Hs, Ws), F, split or None, t0, initial cache, final-state gradient)
CASES = [
    ("norope_d32", 1, 2, 32, (4, 5, 7), 2, None, 0, False, False),
    ("grouped_d64", 1, 2, 64, (6, 5, 7), 2, (16, 24, 24), 4, True, True),
    ("paired_d32", 2, 1, 32, (4, 3, 11), 4, (8, 12, 12), 0, False, True),
    ("general_d64", 1, 2, 64, (4, 5, 6), 2, (6, 26, 32), 3, True, False),
    ("one_block_d64", 1, 1, 64, (3, 9, 9), 3, (16, 24, 24), 7, True, True),
    ("lt16_tokens", 1, 1, 64, (3, 1, 1), 1, (16, 24, 24), 2, False, False),
    # one 20,000-token block per sequence: the suffix scan's block-lanes share
    # the pieces of that block (more than 32 of them)
    ("one_long_block", 1, 4, 64, (2, 100, 100), 2, (16, 24, 24), 5, True, True),
    # 100 blocks of 700 tokens: the recomputed forward takes one reduction
    # range fewer per block
    ("fewer_ranges_per_block", 1, 4, 64, (25, 20, 35), 1, (16, 24, 24), 0, True, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bwd_small(case):
    name, B, H, d, grid, F, split, t0, with_cache, with_final = case
    _say(f"bwd_small {name}")
    N = grid[0] * grid[1] * grid[2]
    rope = split is not None
    q, qd = rand((B, H, N, d), 31, "bf16")
    k, kd = rand((B, H, N, d), 32, "bf16")
    v, vd = rand((B, H, N, d), 33, "bf16")
    do, dod = rand((B, H, N, d), 34, "bf16")
    kw = dict(t0=t0, rope=rope, split=split, eps=1e-6)
    S0 = z0 = dSo = dzo = None
    S0d = z0d = dSod = dzod = None
    if with_cache:
        S0 = wl.draw((B, H, d, d), 35, 10.0, "f32")[0]
        z0 = np.abs(wl.draw((B, H, d), 36, 20.0, "f32")[0])
        S0d, z0d = torch.from_numpy(S0).to(DEV), torch.from_numpy(z0).to(DEV)
    if with_final:
        dSo = wl.draw((B, H, d, d), 37, 1.0, "f32")[0]
        dzo = wl.draw((B, H, d), 38, 1.0, "f32")[0]
        dSod, dzod = torch.from_numpy(dSo).to(DEV), torch.from_numpy(dzo).to(DEV)
    dS0 = torch.empty((B, H, d, d), dtype=torch.float32, device=DEV)
    dz0 = torch.empty((B, H, d), dtype=torch.float32, device=DEV)
    dq, dk, dv = sva.sva_lin_attn_bwd(qd, kd, vd, dod, grid, F, S0=S0d, z0=z0d, dS_out=dSod, dz_out=dzod,
                                      dS0=dS0, dz0=dz0, **kw)
    torch.cuda.synchronize()
    rq, rk, rv, rS0, rz0 = orc.lin_attn_bwd(q, k, v, do, grid, F, S0=S0, z0=z0, dS_final=dSo, dz_final=dzo, **kw)
    errs = {"dq": relerr(dq, rq), "dk": relerr(dk, rk), "dv": relerr(dv, rv), "dS0": relerr(dS0, rS0),
            "dz0": relerr(dz0, rz0)}
    _say(f"  {errs}")
    for key, e in errs.items():
        assert e <= TOL, (key, e)


def test_bwd_gradients_land_only_in_outputs():
    """Every element of dq, dk, dv is written: a second call with the
    gradient buffers pre-filled with garbage gives identical bits."""
    B, H, d, grid, F, split = 1, 2, 64, (6, 4, 8), 2, (16, 24, 24)
    N = grid[0] * grid[1] * grid[2]
    _say("bwd_repeat")
    _, qd = rand((B, H, N, d), 41, "bf16")
    _, kd = rand((B, H, N, d), 42, "bf16")
    _, vd = rand((B, H, N, d), 43, "bf16")
    _, dod = rand((B, H, N, d), 44, "bf16")
    kw = dict(t0=0, rope=True, split=split)
    a = sva.sva_lin_attn_bwd(qd, kd, vd, dod, grid, F, **kw)
    a = [x.clone() for x in a]
    junk = [torch.full_like(x, 7.0) for x in a]
    b = sva.sva_lin_attn_bwd(qd, kd, vd, dod, grid, F, dq=junk[0], dk=junk[1], dv=junk[2], **kw)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_720p_all_heads():
    """The 720p workload at full size; dq, dk, dv of every head compared
    with the oracle's backward."""
    w = wl.WORKLOADS["720p"]
    _say("bwd 720p: generating")
    dev, _ = device_workload(w)
    dod = torch.empty_like(dev["q"])
    for h in range(w.H):
        _, raw = wl.draw((w.N, w.d), wl.seed_for("720p", "dout", 0, h), 1.0, "bf16")
        dod[0, h].copy_(torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16).to(DEV))
    kw = dict(t0=w.t0, rope=w.rope, split=w.split, base=w.base, eps=w.eps)
    grid = (w.T, w.Hs, w.Ws)
    _say("bwd 720p: running")
    dq, dk, dv = sva.sva_lin_attn_bwd(dev["q"], dev["k"], dev["v"], dod, grid, w.F, **kw)
    torch.cuda.synchronize()
    for g in (dq, dk, dv):
        assert bool(torch.isfinite(g).all())
    got = [host_bits(g) for g in (dq, dk, dv)]
    del dev, dod, dq, dk, dv

    def check(b, h):
        q, k, v = (wl.slice_qkv(w, t, b, h)[0][None, None] for t in ("q", "k", "v"))
        do = wl.draw((w.N, w.d), wl.seed_for("720p", "dout", b, h), 1.0, "bf16")[0][None, None]
        refs = orc.lin_attn_bwd(q, k, v, do, grid, w.F, **kw)[:3]
        return max(relerr(g[b, h].astype(np.float64), r[0, 0]) for g, r in zip(got, refs))

    _say(f"bwd 720p: oracle on all {w.H} heads")
    worst, where = compare_slices([(0, h) for h in range(w.H)], check)
    _say(f"bwd 720p: worst rel err over dq, dk, dv {worst:.3e} at {where}")
    assert worst <= TOL


def test_saved_states_match_recompute():
    """sva_lin_attn_fwd_save gives the forward's output bit for bit, and the
    backward from its saved states equals the recomputing backward bit for
    bit (the same fixed-order sums), with an initial cache."""
    B, H, d, grid, F, split = 1, 3, 64, (6, 5, 9), 2, (16, 24, 24)
    N = grid[0] * grid[1] * grid[2]
    _say("bwd saved states")
    _, qd = rand((B, H, N, d), 51, "bf16")
    _, kd = rand((B, H, N, d), 52, "bf16")
    _, vd = rand((B, H, N, d), 53, "bf16")
    _, dod = rand((B, H, N, d), 54, "bf16")
    S0 = torch.from_numpy(wl.draw((B, H, d, d), 55, 5.0, "f32")[0]).to(DEV)
    z0 = torch.from_numpy(np.abs(wl.draw((B, H, d), 56, 9.0, "f32")[0])).to(DEV)
    kw = dict(t0=2, rope=True, split=split)
    out = sva.sva_lin_attn_fwd(qd, kd, vd, grid, F, S0=S0, z0=z0, **kw)
    out2, states = sva.sva_lin_attn_fwd_save(qd, kd, vd, grid, F, S0=S0, z0=z0, **kw)
    a = sva.sva_lin_attn_bwd(qd, kd, vd, dod, grid, F, S0=S0, z0=z0, **kw)
    a = [x.clone() for x in a]
    b = sva.sva_lin_attn_bwd(qd, kd, vd, dod, grid, F, S0=S0, z0=z0, states=states, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
