"""Properties of the HIP path that hold at any size: determinism, block
causality, streaming == one-shot, the V = 1 identity, cache size constant
over an 80-block stream."""
import sys

import numpy as np
import pytest
import torch

from block_causal_linear_phi_amd import sva
from block_causal_linear_phi_amd import workloads as wl
from gpu_helpers import DEV, compare_slices, device_workload, host_bits, rand, relerr
from oracle import sva_oracle as orc

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_two_runs_are_bit_identical_720p():
    w = wl.WORKLOADS["720p"]
    _say("determinism 720p")
    dev, _ = device_workload(w)
    args = ((w.T, w.Hs, w.Ws), w.F)
    kw = dict(t0=w.t0, rope=True, split=w.split, eps=w.eps)
    a = sva.sva_lin_attn_fwd(dev["q"], dev["k"], dev["v"], *args, **kw)
    b = sva.sva_lin_attn_fwd(dev["q"], dev["k"], dev["v"], *args, **kw)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_later_blocks_do_not_change_earlier_outputs(dtype):
    """[talk] block causal segment: block 1 cannot see block 2."""
    B, H, d, grid, F, split = 1, 4, 64, (8, 6, 9), 2, (16, 24, 24)
    _say(f"causality {dtype}")
    N = grid[0] * grid[1] * grid[2]
    Nb = F * grid[1] * grid[2]
    _, qd = rand((B, H, N, d), 31, dtype)
    _, kd = rand((B, H, N, d), 32, dtype)
    _, vd = rand((B, H, N, d), 33, dtype)
    kw = dict(t0=0, rope=True, split=split)
    base = sva.sva_lin_attn_fwd(qd, kd, vd, grid, F, **kw)
    k2, v2 = kd.clone(), vd.clone()
    k2[:, :, 2 * Nb:] = k2[:, :, 2 * Nb:] * 3 + 1
    v2[:, :, 2 * Nb:] = -v2[:, :, 2 * Nb:]
    out = sva.sva_lin_attn_fwd(qd, k2, v2, grid, F, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out[:, :, :2 * Nb], base[:, :, :2 * Nb])
    assert not torch.equal(out[:, :, 2 * Nb:], base[:, :, 2 * Nb:])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_streaming_equals_one_shot(dtype):
    """[talk] block KV cache segment: apply block c against the cache of
    blocks < c, then commit it; outputs and final cache match the one-shot
    forward.  Both are the library's, so this checks the cache path's plumbing
    (t0 handling, in-place commit) rather than numerics against the oracle."""
    B, H, d, F, Hs, Ws, split = 2, 3, 64, 3, 7, 9, (16, 24, 24)
    nblk = 5
    T = nblk * F
    _say(f"streaming {dtype}")
    N = T * Hs * Ws
    Nb = F * Hs * Ws
    _, qd = rand((B, H, N, d), 41, dtype)
    _, kd = rand((B, H, N, d), 42, dtype)
    _, vd = rand((B, H, N, d), 43, dtype)
    S_ref = torch.empty((B, H, d, d), dtype=torch.float32, device=DEV)
    z_ref = torch.empty((B, H, d), dtype=torch.float32, device=DEV)
    one = sva.sva_lin_attn_fwd(qd, kd, vd, (T, Hs, Ws), F, rope=True, split=split, S_out=S_ref, z_out=z_ref)
    S = torch.zeros((B, H, d, d), dtype=torch.float32, device=DEV)
    z = torch.zeros((B, H, d), dtype=torch.float32, device=DEV)
    tol = 1e-5 if dtype == "f32" else 1e-2
    for c in range(nblk):
        sl = slice(c * Nb, (c + 1) * Nb)
        qb, kb, vb = (x[:, :, sl].contiguous() for x in (qd, kd, vd))
        o = sva.sva_block_cache_apply(S, z, qb, kb, vb, (F, Hs, Ws), t0=c * F, rope=True, split=split)
        sva.sva_block_cache_commit(S, z, kb, vb, (F, Hs, Ws), t0=c * F, rope=True, split=split)
        torch.cuda.synchronize()
        assert relerr(o, one[:, :, sl].float().cpu().numpy().astype(np.float64)) <= tol
    assert relerr(S, S_ref.cpu().numpy().astype(np.float64)) <= 1e-5
    assert relerr(z, z_ref.cpu().numpy().astype(np.float64)) <= 1e-5
    # The last denoising step of a block can output and commit in one call: a
    # one-block forward with the cache as both S0 and S_out.
    S2 = torch.zeros_like(S)
    z2 = torch.zeros_like(z)
    for c in range(nblk):
        sl = slice(c * Nb, (c + 1) * Nb)
        qb, kb, vb = (x[:, :, sl].contiguous() for x in (qd, kd, vd))
        o = sva.sva_lin_attn_fwd(qb, kb, vb, (F, Hs, Ws), F, t0=c * F, rope=True, split=split, S0=S2, z0=z2,
                                 S_out=S2, z_out=z2)
        torch.cuda.synchronize()
        assert relerr(o, one[:, :, sl].float().cpu().numpy().astype(np.float64)) <= tol
    assert relerr(S2, S_ref.cpu().numpy().astype(np.float64)) <= 1e-5
    assert relerr(z2, z_ref.cpu().numpy().astype(np.float64)) <= 1e-5


def test_v_ones_gives_one_without_rope():
    """RoPE-free denominator: with V = 1 and no RoPE the output is
    den / (den + eps), i.e. 1 up to eps/den."""
    B, H, d, grid, F = 1, 2, 64, (4, 8, 12), 2
    N = grid[0] * grid[1] * grid[2]
    _, qd = rand((B, H, N, d), 51, "f32")
    _, kd = rand((B, H, N, d), 52, "f32")
    vd = torch.ones((B, H, N, d), dtype=torch.float32, device=DEV)
    out = sva.sva_lin_attn_fwd(qd, kd, vd, grid, F, rope=False, eps=1e-6)
    torch.cuda.synchronize()
    assert float((out - 1).abs().max()) < 1e-5
    out2 = sva.sva_lin_attn_fwd(qd, kd, vd, grid, F, rope=True, split=(16, 24, 24), eps=1e-6)
    torch.cuda.synchronize()
    assert float((out2 - 1).abs().max()) > 1e-2


def test_cache_memory_constant_over_80_block_stream():
    """[talk]: constant memory regardless of length.  An 80-block stream of
    the minute-long workload's shape (B=2, H=16, 3 x 30 x 52 blocks) runs
    apply + commit per block on one fixed cache without any growth in device
    memory; the workspace is one-block sized and reused.  The final cache and
    the last block's output match the oracle's stream of the same blocks on
    every (b, h) slice."""
    w = wl.WORKLOADS["minute"]
    fg = (w.F, w.Hs, w.Ws)
    _say("80-block stream")
    blocks = [device_workload(w, step=s, n_tokens=w.block_tokens)[0] for s in range(2)]
    S = torch.zeros((w.B, w.H, w.d, w.d), dtype=torch.float32, device=DEV)
    z = torch.zeros((w.B, w.H, w.d), dtype=torch.float32, device=DEV)
    desc = sva.make_desc(w.B, w.H, w.d, fg, w.F, t0=0, rope=True, split=w.split)
    ws = torch.zeros(sva.sva_block_cache_workspace(desc), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(blocks[0]["q"])
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    for c in range(w.nb):
        x = blocks[c % 2]
        sva.sva_block_cache_apply(S, z, x["q"], x["k"], x["v"], fg, t0=c * w.F, rope=True, split=w.split,
                                  out=out, ws=ws)
        sva.sva_block_cache_commit(S, z, x["k"], x["v"], fg, t0=c * w.F, rope=True, split=w.split, ws=ws)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(S).all())
    assert S.numel() * 4 + z.numel() * 4 == w.B * w.H * (w.d * w.d + w.d) * 4
    got_out, got_S, got_z = host_bits(out), S.cpu().numpy(), z.cpu().numpy()
    kw = dict(rope=True, split=w.split, base=w.base)

    def check(b, h):
        data = [[wl.slice_qkv(w, t, b, h, s, w.block_tokens)[0][None, None] for t in "qkv"] for s in range(2)]
        Sr, zr = np.zeros((1, 1, w.d, w.d)), np.zeros((1, 1, w.d))
        for c in range(w.nb):
            q, k, v = data[c % 2]
            if c == w.nb - 1:
                ref_out = orc.block_cache_apply(Sr, zr, q, k, v, fg, t0=c * w.F, eps=w.eps, **kw)
            Sr, zr = orc.block_cache_commit(Sr, zr, k, v, fg, t0=c * w.F, **kw)
        eo = relerr(got_out[b, h].astype(np.float64), ref_out[0, 0])
        eS = relerr(got_S[b, h].astype(np.float64), Sr[0, 0])
        ez = relerr(got_z[b, h].astype(np.float64), zr[0, 0])
        assert ez <= 1e-5, (b, h, ez)
        return max(eo, eS)

    _say("80-block stream: oracle stream on every (b, h) slice")
    worst, where = compare_slices([(b, h) for b in range(w.B) for h in range(w.H)], check)
    _say(f"80-block stream: worst rel err (last output, final S) {worst:.3e} at {where}")
    assert worst <= 1e-2
