"""The prepared forward call (sva.prepare_lin_attn_fwd): its calls give the
checking wrapper's outputs bit for bit, follow new contents of the same
input buffers, and are captured like any call under a HIP graph."""
import sys

import pytest
import torch

from block_causal_linear_phi_amd import sva
from gpu_helpers import DEV, rand

pytestmark = pytest.mark.gpu

SPLIT = (16, 24, 24)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16)) if a.dtype == torch.bfloat16 else torch.equal(a, b)


@pytest.mark.parametrize("grid,F,H,with_cache", [((6, 6, 10), 2, 4, False), ((3, 30, 52), 3, 16, True)],
                         ids=["multi_block", "one_block_cache"])
def test_prepared_forward_matches_the_wrapper(grid, F, H, with_cache):
    B, n = 1, grid[0] * grid[1] * grid[2]
    q, k, v = (rand((B, H, n, 64), 701 + i, "bf16")[1] for i in range(3))
    kw = dict(t0=6, rope=True, split=SPLIT, eps=1e-6)
    cache = {}
    if with_cache:
        cache = dict(S0=rand((B, H, 64, 64), 711, "f32", 30.0)[1], z0=rand((B, H, 64), 712, "f32", 60.0)[1].abs(),
                     S_out=torch.empty((B, H, 64, 64), dtype=torch.float32, device=DEV),
                     z_out=torch.empty((B, H, 64), dtype=torch.float32, device=DEV))
    _say(f"prepared forward grid={grid} H={H}")
    call = sva.prepare_lin_attn_fwd(q, k, v, grid, F, **kw, **cache)
    for rnd in range(3):
        if rnd:
            # new contents in the same buffers
            for t, seed in ((q, 720 + rnd), (k, 730 + rnd), (v, 740 + rnd)):
                t.copy_(rand(tuple(t.shape), seed, "bf16")[1])
        ref_cache = {}
        if with_cache:
            ref_cache = dict(S0=cache["S0"], z0=cache["z0"], S_out=torch.empty_like(cache["S_out"]),
                             z_out=torch.empty_like(cache["z_out"]))
        ref = sva.sva_lin_attn_fwd(q, k, v, grid, F, **kw, **ref_cache)
        out = call()
        torch.cuda.synchronize()
        assert out is call.out and _same(out, ref), rnd
        if with_cache:
            assert torch.equal(cache["S_out"], ref_cache["S_out"]) and torch.equal(cache["z_out"], ref_cache["z_out"])
    # captured under a graph: the replay writes the same output
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    call.out.fill_(5.0)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert _same(call.out, ref)
