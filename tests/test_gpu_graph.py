"""Library calls captured in a HIP graph (torch's CUDAGraph) and replayed
three times, with eager library calls of another shape, torch work and a
synchronization between replays; the outputs are overwritten with garbage
before each replay, and every replay must reproduce the eager call's outputs
bit for bit.  Covered: the forward with the prefix from the scan kernel and
with the prefix folded into the reduction (32 blocks per sequence: its
arrival counters must be back at zero for each replay), the block-cache apply
with a workspace and the workspace-free one, and the commit, whose replays
add to the cache as repeated eager commits do.  The library launches kernels
only (no memset or copy nodes in the graphs)."""
import sys

import pytest
import torch

from block_causal_linear_phi_amd import sva
from gpu_helpers import DEV, rand

pytestmark = pytest.mark.gpu

SPLIT = (16, 24, 24)
REPLAYS = 3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


def _qkv(B, H, n, seed, d=64):
    return [rand((B, H, n, d), seed + i, "bf16")[1] for i in range(3)]


def _cache(B, H, seed, d=64):
    S = rand((B, H, d, d), seed, "f32", 30.0)[1]
    z = rand((B, H, d), seed + 1, "f32", 60.0)[1].abs()
    return S, z


def _other_work():
    """Eager work of another shape between two replays."""
    q, k, v = _qkv(1, 2, 2 * 4 * 6, 907)
    sva.sva_lin_attn_fwd(q, k, v, (2, 4, 6), 1, t0=3, rope=True, split=SPLIT)
    torch.randn(1 << 20, device=DEV).mul_(2.0).sum()
    torch.cuda.synchronize()


def _replay_and_check(g, outs, refs, label):
    for r in range(REPLAYS):
        for o in outs:
            o.fill_(7.0)
        _other_work()
        _say(f"graph replay {r} of {label}")
        g.replay()
        torch.cuda.synchronize()
        for o, ref in zip(outs, refs):
            assert _same(o, ref), (label, r)


@pytest.mark.parametrize("grid,F,H", [((6, 6, 10), 2, 4), ((32, 4, 8), 1, 2)], ids=["scan", "folded"])
def test_forward_graph_replays_match_eager(grid, F, H):
    B, n = 1, grid[0] * grid[1] * grid[2]
    q, k, v = _qkv(B, H, n, 301)
    S0, z0 = _cache(B, H, 311)
    kw = dict(t0=5, rope=True, split=SPLIT, eps=1e-6)
    desc = sva.make_desc(B, H, 64, grid, F, t0=5, rope=True, split=SPLIT)
    ws = torch.zeros(sva.sva_lin_attn_fwd_workspace(desc), dtype=torch.uint8, device=DEV)
    _say(f"eager forward grid={grid} F={F} H={H}")
    out_e, S_e, z_e = torch.empty_like(q), torch.empty_like(S0), torch.empty_like(z0)
    sva.sva_lin_attn_fwd(q, k, v, grid, F, S0=S0, z0=z0, out=out_e, S_out=S_e, z_out=z_e, ws=ws, **kw)
    torch.cuda.synchronize()
    out_g, S_g, z_g = torch.empty_like(q), torch.empty_like(S0), torch.empty_like(z0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sva.sva_lin_attn_fwd(q, k, v, grid, F, S0=S0, z0=z0, out=out_g, S_out=S_g, z_out=z_g, ws=ws, **kw)
    _replay_and_check(g, [out_g, S_g, z_g], [out_e, S_e, z_e], f"forward {grid}")
    # the workspace starts with the folded prefix's B*H arrival counters
    # (then padding to 256 bytes): zero again after the replays
    assert int(ws[:256].count_nonzero()) == 0


@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
def test_block_cache_apply_graph_replays_match_eager(noalloc):
    B, H, fg, t0 = 1, 16, (3, 30, 52), 18
    n = fg[0] * fg[1] * fg[2]
    q, k, v = _qkv(B, H, n, 401)
    S, z = _cache(B, H, 411)
    S_keep, z_keep = S.clone(), z.clone()
    kw = dict(t0=t0, rope=True, split=SPLIT, eps=1e-6)
    desc = sva.make_desc(B, H, 64, fg, fg[0], **kw)
    ws = torch.zeros(sva.sva_block_cache_workspace(desc), dtype=torch.uint8, device=DEV)

    def call(out):
        if noalloc:
            sva.sva_block_cache_apply_noalloc(S, z, q, k, v, fg, out=out, **kw)
        else:
            sva.sva_block_cache_apply(S, z, q, k, v, fg, out=out, ws=ws, **kw)

    _say(f"eager block-cache apply noalloc={noalloc}")
    out_e = torch.empty_like(q)
    call(out_e)
    torch.cuda.synchronize()
    out_g = torch.empty_like(q)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out_g)
    _replay_and_check(g, [out_g], [out_e], f"block-cache apply noalloc={noalloc}")
    assert torch.equal(S, S_keep) and torch.equal(z, z_keep)  # the cache is read only


def test_commit_graph_replays_match_repeated_eager_commits():
    B, H, fg, t0 = 1, 4, (3, 12, 20), 9
    n = fg[0] * fg[1] * fg[2]
    _, k, v = _qkv(B, H, n, 501)
    S0, z0 = _cache(B, H, 511)
    kw = dict(t0=t0, rope=True, split=SPLIT)
    desc = sva.make_desc(B, H, 64, fg, fg[0], **kw)
    ws = torch.zeros(sva.sva_block_cache_workspace(desc), dtype=torch.uint8, device=DEV)
    _say("eager commits")
    S_e, z_e = S0.clone(), z0.clone()
    snaps = []
    for _ in range(REPLAYS):
        sva.sva_block_cache_commit(S_e, z_e, k, v, fg, ws=ws, **kw)
        torch.cuda.synchronize()
        snaps.append((S_e.clone(), z_e.clone()))
    S_g, z_g = S0.clone(), z0.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sva.sva_block_cache_commit(S_g, z_g, k, v, fg, ws=ws, **kw)
    assert torch.equal(S_g, S0)  # capture runs nothing
    for r in range(REPLAYS):
        _other_work()
        _say(f"graph replay {r} of the commit")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(S_g, snaps[r][0]) and torch.equal(z_g, snaps[r][1]), r
