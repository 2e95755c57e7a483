"""GPU parity: the HIP library (called through its C ABI) against the fp64
oracle on identical seeded inputs.

Bar: max|gpu - oracle| / max|oracle| <= 1e-5 for fp32 inputs and <= 1e-2 for
bf16 inputs.  Sizes span several 16/32-token tiles, ragged tails, several
blocks, both head dims and every RoPE axis; the video-shaped workloads run
at full size in the launch configuration the benchmark times, with every
(b, h) slice compared element by element.
"""
import sys

import numpy as np
import pytest
import torch

from block_causal_linear_phi_amd import sva
from block_causal_linear_phi_amd import workloads as wl
from gpu_helpers import DEV, TOL, compare_slices, device_workload, host_bits, rand, relerr
from oracle import sva_oracle as orc

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# (name, B, H, d, (T, Hs, Ws), F, rope split or None, t0)
SMALL = [
    ("tiny_cfg", 1, 2, 32, (4, 8, 8), 1, None, 0),
    ("ragged_d64", 2, 3, 64, (6, 5, 7), 2, (16, 24, 24), 4),
    ("ragged_d32", 1, 2, 32, (4, 3, 11), 4, (8, 12, 12), 0),
    ("lt16_tokens", 1, 1, 64, (3, 1, 1), 1, (16, 24, 24), 2),
    ("one_block_norope", 1, 2, 64, (2, 9, 9), 2, None, 0),
    ("h_only_axis", 1, 2, 64, (2, 6, 4), 1, (0, 64, 0), 0),
    ("w_frame_axes", 2, 1, 32, (6, 2, 17), 3, (16, 0, 16), 11),
    # axis widths that are not multiples of 4: the unpaired table-lookup path
    ("odd_split_d64", 1, 2, 64, (4, 5, 6), 2, (6, 26, 32), 3),
    ("odd_split_d32", 2, 1, 32, (3, 4, 9), 3, (10, 10, 12), 0),
    # 32 or more blocks a sequence: the prefix is formed inside the reduction
    # (the last workgroup of each sequence), not by a scan launch
    ("many_blocks_d64", 2, 2, 64, (40, 3, 5), 1, (16, 24, 24), 7),
    ("many_blocks_d32", 1, 3, 32, (64, 2, 4), 2, (8, 12, 12), 0),
    # one 20,000-token block per sequence: every block cut into equal ranges
    # (its length padded on the split axis), and the scan's block-lanes share
    # more than 32 pieces of one block
    ("one_long_block", 1, 4, 64, (2, 100, 100), 2, (16, 24, 24), 5),
    # 100 blocks of 700 tokens: ceil(700 / L) ranges a block would not fit in
    # one round, so the reduction takes one range fewer per block
    ("fewer_ranges_per_block", 1, 4, 64, (25, 20, 35), 1, (16, 24, 24), 0),
    # 32 blocks of 2,001 tokens in one sequence: the prefix formed inside the
    # reduction, on equal ranges of a padded block length
    ("folded_padded_ranges", 1, 1, 64, (32, 23, 87), 1, (16, 24, 24), 3),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_fwd_small(case, dtype):
    name, B, H, d, grid, F, split, t0 = case
    _say(f"fwd_small {name} {dtype}")
    N = grid[0] * grid[1] * grid[2]
    q, qd = rand((B, H, N, d), 1, dtype)
    k, kd = rand((B, H, N, d), 2, dtype)
    v, vd = rand((B, H, N, d), 3, dtype)
    rope = split is not None
    S_out = torch.empty((B, H, d, d), dtype=torch.float32, device=DEV)
    z_out = torch.empty((B, H, d), dtype=torch.float32, device=DEV)
    out = sva.sva_lin_attn_fwd(qd, kd, vd, grid, F, t0=t0, rope=rope, split=split, eps=1e-6,
                               S_out=S_out, z_out=z_out)
    torch.cuda.synchronize()
    ref, S_ref, z_ref = orc.lin_attn_fwd(q, k, v, grid, F, t0=t0, rope=rope, split=split, eps=1e-6)
    assert relerr(out, ref) <= TOL[dtype]
    assert relerr(S_out, S_ref) <= TOL[dtype]
    assert relerr(z_out, z_ref) <= 1e-5


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("base,eps,t0", [(500.0, 1e-3, 0), (1e6, 1e-6, 0), (10000.0, 1e-6, 5000)],
                         ids=["base500_eps1e-3", "base1e6", "t0_5000"])
def test_fwd_other_base_eps_and_positions(base, eps, t0, dtype):
    """Descriptor values other than the workloads': the RoPE base (angles
    base^(-2i/d_a)), a larger eps, and large absolute frame positions (the
    angle's reduction to one turn)."""
    B, H, d, grid, F, split = 1, 2, 64, (6, 5, 7), 3, (16, 24, 24)
    _say(f"fwd base={base} eps={eps} t0={t0} {dtype}")
    N = grid[0] * grid[1] * grid[2]
    q, qd = rand((B, H, N, d), 11, dtype)
    k, kd = rand((B, H, N, d), 12, dtype)
    v, vd = rand((B, H, N, d), 13, dtype)
    out = sva.sva_lin_attn_fwd(qd, kd, vd, grid, F, t0=t0, rope=True, split=split, base=base, eps=eps)
    torch.cuda.synchronize()
    ref, _, _ = orc.lin_attn_fwd(q, k, v, grid, F, t0=t0, rope=True, split=split, base=base, eps=eps)
    assert relerr(out, ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("grid,F", [((4, 6, 10), 2), ((36, 2, 3), 1)], ids=["scan", "folded_prefix"])
def test_fwd_with_initial_cache_in_place(dtype, grid, F):
    """S0/z0 given and S_out/z_out the same buffers: the final cache is
    written in place (by the scan kernel, or by the reduction's last
    workgroup when a sequence has 32 or more blocks)."""
    B, H, d, split, t0 = 1, 4, 64, (16, 24, 24), 6
    _say(f"fwd_initial_cache {dtype} {grid} F={F}")
    N = grid[0] * grid[1] * grid[2]
    q, qd = rand((B, H, N, d), 11, dtype)
    k, kd = rand((B, H, N, d), 12, dtype)
    v, vd = rand((B, H, N, d), 13, dtype)
    S0 = (wl.draw((B, H, d, d), 14, 20.0, "f32")[0])
    z0 = np.abs(wl.draw((B, H, d), 15, 30.0, "f32")[0])
    S = torch.from_numpy(S0).to(DEV)
    z = torch.from_numpy(z0).to(DEV)
    out = sva.sva_lin_attn_fwd(qd, kd, vd, grid, F, t0=t0, rope=True, split=split, S0=S, z0=z,
                               S_out=S, z_out=z)
    torch.cuda.synchronize()
    ref, S_ref, z_ref = orc.lin_attn_fwd(q, k, v, grid, F, t0=t0, rope=True, split=split, S0=S0, z0=z0)
    assert relerr(out, ref) <= TOL[dtype]
    assert relerr(S, S_ref) <= TOL[dtype]
    assert relerr(z, z_ref) <= 1e-5


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d,split", [(64, (16, 24, 24)), (32, (8, 12, 12)), (64, None)])
def test_prep_stage(dtype, d, split):
    """phi + 3D RoPE stage alone against the oracle's phi and rotation."""
    B, H, grid, t0 = 1, 2, (5, 7, 9), 13
    _say(f"prep {dtype} d={d} split={split}")
    N = grid[0] * grid[1] * grid[2]
    x, xd = rand((B, H, N, d), 21, dtype)
    rope = split is not None
    xr, xp = sva.sva_phi_rope_prep(xd, grid, t0=t0, rope=rope, split=split)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            ph = orc.phi(x[b, h].astype(np.float64))
            np.testing.assert_array_equal(xp[b, h].cpu().numpy(), ph.astype(np.float32))
            if rope:
                t, hh, ww = orc.token_coords(*grid, t0)
                ref = orc.rope_rotate(ph, t, hh, ww, split, 10000.0)
            else:
                ref = ph
            # fp32 rotation of fp32 values: a few ulps; same bar for both paths
            assert relerr(xr[b, h], ref) <= 2e-6


def test_tiny_workload():
    w = wl.WORKLOADS["tiny"]
    _say("tiny workload")
    dev, host = device_workload(w, keep={(0, h) for h in range(w.H)})
    out = sva.sva_lin_attn_fwd(dev["q"], dev["k"], dev["v"], (w.T, w.Hs, w.Ws), w.F, rope=False, eps=w.eps)
    torch.cuda.synchronize()
    q = np.stack([host[("q", 0, h)] for h in range(w.H)])[None]
    k = np.stack([host[("k", 0, h)] for h in range(w.H)])[None]
    v = np.stack([host[("v", 0, h)] for h in range(w.H)])[None]
    ref, _, _ = orc.lin_attn_fwd(q, k, v, (w.T, w.Hs, w.Ws), w.F, eps=w.eps)
    assert relerr(out, ref) <= 1e-5


def _full_workload_check(name):
    """The workload at full size, in the launch configuration the benchmark
    times; every (b, h) slice of the output compared element by element with
    the oracle on the same seeded inputs (regenerated slice by slice)."""
    w = wl.WORKLOADS[name]
    _say(f"{name}: generating")
    dev, _ = device_workload(w)
    _say(f"{name}: running")
    out = sva.sva_lin_attn_fwd(dev["q"], dev["k"], dev["v"], (w.T, w.Hs, w.Ws), w.F, t0=w.t0, rope=w.rope,
                               split=w.split, base=w.base, eps=w.eps)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    got = host_bits(out)
    del dev

    def check(b, h):
        q, k, v = (wl.slice_qkv(w, t, b, h)[0][None, None] for t in "qkv")
        ref, _, _ = orc.lin_attn_fwd(q, k, v, (w.T, w.Hs, w.Ws), w.F, t0=w.t0, rope=w.rope,
                                     split=w.split, base=w.base, eps=w.eps)
        return relerr(got[b, h].astype(np.float64), ref[0, 0])

    _say(f"{name}: oracle on all {w.B * w.H} (b, h) slices")
    worst, where = compare_slices([(b, h) for b in range(w.B) for h in range(w.H)], check)
    _say(f"{name}: worst rel err {worst:.3e} at (b, h) = {where}")
    assert worst <= TOL[w.dtype]


def test_480p_all_heads():
    _full_workload_check("480p")


def test_720p_all_heads():
    _full_workload_check("720p")


def test_minute_all_heads():
    _full_workload_check("minute")


def test_cached_step_workload():
    """Cache from 6 prior 3-frame blocks (oracle, rounded to fp32), then one
    block at t0 = 18 re-evaluated for 4 denoising steps with fresh q, k, v,
    then the last step committed.  Apply never changes the cache."""
    w = wl.WORKLOADS["cached_step"]
    fg = (w.F, w.Hs, w.Ws)
    _say("cached step: building cache with the oracle")
    S = np.zeros((w.B, w.H, w.d, w.d))
    z = np.zeros((w.B, w.H, w.d))
    for pb in range(w.prior_blocks):
        kk = np.stack([[wl.slice_qkv(w, "k_prior", b, h, pb)[0] for h in range(w.H)] for b in range(w.B)])
        vv = np.stack([[wl.slice_qkv(w, "v_prior", b, h, pb)[0] for h in range(w.H)] for b in range(w.B)])
        S, z = orc.block_cache_commit(S, z, kk, vv, fg, t0=pb * w.F, rope=w.rope, split=w.split, base=w.base)
    S32, z32 = S.astype(np.float32), z.astype(np.float32)
    Sd, zd = torch.from_numpy(S32).to(DEV), torch.from_numpy(z32).to(DEV)
    keep = {(b, h) for b in range(w.B) for h in range(w.H)}
    for step in range(w.steps):
        _say(f"cached step: step {step}")
        dev, host = device_workload(w, step=step, keep=keep)
        out = sva.sva_block_cache_apply(Sd, zd, dev["q"], dev["k"], dev["v"], fg, t0=w.t0, rope=w.rope,
                                        split=w.split, base=w.base, eps=w.eps)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(Sd.cpu().numpy(), S32)
        np.testing.assert_array_equal(zd.cpu().numpy(), z32)
        q, k, v = (np.stack([[host[(t, b, h)] for h in range(w.H)] for b in range(w.B)]) for t in "qkv")
        ref = orc.block_cache_apply(S32.astype(np.float64), z32.astype(np.float64), q, k, v, fg, t0=w.t0,
                                    rope=w.rope, split=w.split, base=w.base, eps=w.eps)
        assert relerr(out, ref) <= 1e-2
    sva.sva_block_cache_commit(Sd, zd, dev["k"], dev["v"], fg, t0=w.t0, rope=w.rope, split=w.split,
                               base=w.base)
    torch.cuda.synchronize()
    S_ref, z_ref = orc.block_cache_commit(S32.astype(np.float64), z32.astype(np.float64), k, v, fg, t0=w.t0,
                                          rope=w.rope, split=w.split, base=w.base)
    assert relerr(Sd, S_ref) <= 1e-2
    assert relerr(zd, z_ref) <= 1e-5
