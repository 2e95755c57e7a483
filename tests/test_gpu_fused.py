"""GPU parity of the fused projection + attention (sva_proj_lin_attn_fwd)
against the oracles composed: q, k, v = the fp64 projection oracle rounded
to bf16 (round to nearest even, as the stored tensors of the unfused path
are), then the fp64 attention oracle.  Bar 1e-2 (bf16), as for both parts.
Cases cover ragged 64-token tiles inside a range, ranges inside blocks,
two samples, no RoPE, no bias, an initial cache with the final cache
written in place, and every head at the 720p size."""
import sys

import numpy as np
import pytest
import torch

from block_causal_linear_phi_amd import sva
from block_causal_linear_phi_amd import workloads as wl
from gpu_helpers import DEV, TOL, compare_slices, host_bits, relerr, to_device
from oracle import proj_oracle as porc
from oracle import sva_oracle as orc

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bf16(a: np.ndarray) -> np.ndarray:
    """fp64 -> nearest-even bf16 -> fp64 (torch on the host)."""
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).to(torch.float64).numpy()


def _weights(n_out, C, seed):
    codes, scales = wl.mxfp4_weights(n_out, C, seed)
    cd = torch.from_numpy(wl.pack_nibbles(codes)).to(DEV)
    sd = torch.from_numpy(scales).to(DEV)
    return codes, scales, cd, sd


# (name, B, H, grid, F, C, split or None, t0, bias, initial cache)
CASES = [
    ("ragged_tiles", 1, 2, (6, 5, 7), 3, 256, (16, 24, 24), 3, True, False),
    ("two_samples", 2, 4, (4, 8, 9), 2, 256, (16, 24, 24), 0, False, False),
    ("no_rope", 1, 2, (3, 10, 10), 1, 512, None, 0, True, False),
    ("cache_in_place", 1, 2, (4, 6, 7), 2, 768, (8, 28, 28), 6, True, True),
    ("long_ranges", 1, 2, (2, 40, 41), 2, 256, (16, 24, 24), 0, True, False),
    # RoPE table (F dt/2 + Hs dh/2 + Ws dw/2 entries) past the kernel's LDS
    # budget: angles on the fly
    ("wide_rows", 1, 2, (2, 3, 280), 1, 256, (16, 24, 24), 11, True, False),
    # the same on-the-fly angles at a frame index in the hundred thousands
    # (the block's first-frame turn is reduced in fp64)
    ("wide_rows_far_frames", 1, 2, (2, 3, 280), 1, 256, (16, 24, 24), 123457, True, False),
]


def _long_range(Nb):
    """The largest divisor of the block length up to 2048 tokens: ranges of
    many 64-token tiles, the last one ragged where 64 does not divide it."""
    return max(L for L in range(1, min(Nb, 2048) + 1) if Nb % L == 0)


@pytest.mark.parametrize("ranges", ["auto", "long"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fused_small(case, ranges):
    name, B, H, grid, F, C, split, t0, with_bias, cache = case
    N = grid[0] * grid[1] * grid[2]
    range_tokens = _long_range(F * grid[1] * grid[2]) if ranges == "long" else 0
    _say(f"fused {name} ranges {ranges}")
    xv, xraw = wl.draw((B, N, C), 301, 1.0, "bf16")
    codes, scales, cd, sd = _weights(3 * H * 64, C, 302)
    wp = sva.sva_mxfp4_pack_weights(cd, sd, H, 64)
    bias = bd = None
    if with_bias:
        bias = wl.draw((3 * H * 64,), 303, 0.1, "f32")[0]
        bd = torch.from_numpy(bias).to(DEV)
    S0 = z0 = S0d = z0d = None
    if cache:
        S0 = np.abs(wl.draw((B, H, 64, 64), 304, 2.0, "f32")[0])
        z0 = np.abs(wl.draw((B, H, 64), 305, 8.0, "f32")[0])
        S0d = torch.from_numpy(S0).to(DEV)
        z0d = torch.from_numpy(z0).to(DEV)
    rope = split is not None
    kw = dict(t0=t0, rope=rope, split=split, eps=1e-6)
    out = sva.sva_proj_lin_attn_fwd(to_device(xraw, "bf16"), wp, bd, H, grid, F, S0=S0d, z0=z0d, S_out=S0d,
                                    z_out=z0d, range_tokens=range_tokens, **kw)
    torch.cuda.synchronize()
    q, k, v = (_bf16(t) for t in porc.qkv_project(xv, codes, scales, bias, H, 64))
    ref, S_ref, z_ref = orc.lin_attn_fwd(q, k, v, grid, F, S0=S0, z0=z0, **kw)
    err = relerr(out, ref)
    _say(f"  out err {err:.3g}")
    assert err <= TOL["bf16"]
    if cache:
        eS, ez = relerr(S0d, S_ref), relerr(z0d, z_ref)
        _say(f"  cache errs {eS:.3g} {ez:.3g}")
        assert eS <= TOL["bf16"] and ez <= TOL["bf16"]


def test_fused_matches_unfused_gpu_path():
    """The fused and the two-call paths (projection, then the attention on
    its stored q, k, v) agree within the bf16 bar."""
    B, H, grid, F, C, split = 1, 4, (6, 9, 13), 3, 256, (16, 24, 24)
    _say("fused vs unfused")
    N = grid[0] * grid[1] * grid[2]
    _, xraw = wl.draw((B, N, C), 311, 1.0, "bf16")
    xd = to_device(xraw, "bf16")
    codes, scales, cd, sd = _weights(3 * H * 64, C, 312)
    wp = sva.sva_mxfp4_pack_weights(cd, sd, H, 64)
    fused = sva.sva_proj_lin_attn_fwd(xd, wp, None, H, grid, F, rope=True, split=split, t0=9)
    q, k, v = sva.sva_qkv_proj_mxfp4(xd, wp, None, H, 64)
    two = sva.sva_lin_attn_fwd(q, k, v, grid, F, rope=True, split=split, t0=9)
    torch.cuda.synchronize()
    err = relerr(fused, two.float().cpu().numpy().astype(np.float64))
    _say(f"  err {err:.3g}")
    assert err <= TOL["bf16"]


def test_fused_720p_all_heads():
    """The 720p grid (75,600 tokens, 16 heads, C = 1024) in full; every head
    compared with the composed oracles."""
    w = wl.WORKLOADS["720p"]
    pw = wl.PROJ_WORKLOADS["proj_720p"]
    _say("fused 720p: generating")
    xd = torch.empty((1, pw.N, pw.C), dtype=torch.bfloat16, device=DEV)
    xs = np.empty((pw.N, pw.C), dtype=np.float64)
    for j, s0 in enumerate(range(0, pw.N, 4096)):
        n = min(4096, pw.N - s0)
        vals, raw = wl.draw((n, pw.C), wl.seed_for(pw.name, "x", 0, j), 1.0, "bf16")
        xd[0, s0:s0 + n].copy_(to_device(raw, "bf16"))
        xs[s0:s0 + n] = vals
    codes, scales, cd, sd = _weights(pw.n_out, pw.C, wl.seed_for(pw.name, "w", 0, 0))
    wp = sva.sva_mxfp4_pack_weights(cd, sd, pw.H, pw.d)
    bias = wl.draw((pw.n_out,), wl.seed_for(pw.name, "bias", 0, 0), 0.1, "f32")[0]
    _say("fused 720p: running")
    out = sva.sva_proj_lin_attn_fwd(xd, wp, torch.from_numpy(bias).to(DEV), pw.H, (w.T, w.Hs, w.Ws), w.F,
                                    rope=True, split=w.split, t0=w.t0, eps=w.eps)
    torch.cuda.synchronize()
    got = host_bits(out)
    HD = pw.H * pw.d
    x64 = xs[None]

    def check(b, h):
        rows = np.concatenate([np.arange(h * 64, h * 64 + 64) + j * HD for j in range(3)])
        q, k, v = (_bf16(t) for t in porc.qkv_project(x64, codes[rows], scales[rows], bias[rows], 1, 64))
        ref, _, _ = orc.lin_attn_fwd(q, k, v, (w.T, w.Hs, w.Ws), w.F, rope=True, split=w.split, t0=w.t0,
                                     eps=w.eps)
        return relerr(got[b, h:h + 1].astype(np.float64), ref[0])

    _say(f"fused 720p: oracle on all {pw.H} heads")
    worst, where = compare_slices([(0, h) for h in range(pw.H)], check)
    _say(f"fused 720p: worst rel err {worst:.3e} at {where}")
    assert worst <= TOL["bf16"]
