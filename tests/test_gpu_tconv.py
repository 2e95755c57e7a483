"""GPU parity of the causal temporal convolution (sva_tconv_fwd, _apply,
_commit) against the fp64 oracle (oracle/tconv_oracle.py) on identical
seeded inputs.

Bar: max|gpu - oracle| / max|oracle| <= 1e-5 for fp32 (fp32 fused
multiply-adds on exact inputs) and <= 1e-2 for bf16 (one output rounding);
the carried cache is a copy and must match bit for bit.  Small cases span a
ragged number of frames against the four-frame load chunk, one-frame and
one-block splits, channel rows of 1..65 vectors, an initial cache and no
bias; the 720p and minute workloads run at full size and are compared at
sampled spatial positions (the op is independent per position).
"""
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from block_causal_linear_phi_amd import sva
from block_causal_linear_phi_amd import workloads as wl
from gpu_helpers import DEV, TOL, relerr, to_device
from oracle import tconv_oracle as orc

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _draw(shape, seed, dtype, scale=1.0):
    vals, raw = wl.draw(shape, seed, scale, dtype)
    return vals, to_device(raw, dtype)


def _params(C, seed):
    w = wl.draw((C, 3), seed, float(np.sqrt(1.0 / 3.0)), "f32")[0]
    b = wl.draw((C,), seed + 1, 0.1, "f32")[0]
    return w, b, torch.from_numpy(w).to(DEV), torch.from_numpy(b).to(DEV)


# (name, B, T, Hs, Ws, C, F, dtype, initial cache, bias)
CASES = [
    ("tiny_f32", 1, 4, 8, 8, 32, 1, "f32", False, True),
    ("ragged_bf16", 2, 9, 3, 5, 24, 3, "bf16", True, True),
    ("one_block_bf16", 1, 5, 2, 7, 8, 5, "bf16", True, False),
    ("one_frame_blocks_f32", 1, 6, 1, 3, 4, 1, "f32", True, True),
    ("long_f32", 1, 42, 2, 2, 12, 6, "f32", False, True),
    ("wide_bf16", 1, 6, 4, 4, 520, 2, "bf16", True, True),
    ("single_frame_bf16", 3, 1, 2, 3, 16, 1, "bf16", True, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_tconv_small(case):
    name, B, T, Hs, Ws, C, F, dtype, with_cache, with_bias = case
    _say(f"tconv_small {name}")
    x, xd = _draw((B, T, Hs, Ws, C), 101, dtype)
    w, b, wd, bd = _params(C, 102)
    cache = cached = None
    if with_cache:
        cache, cached = _draw((B, Hs, Ws, C), 104, dtype)
    if not with_bias:
        b = bd = None
    cache_out = torch.full((B, Hs, Ws, C), 7.0, dtype=xd.dtype, device=DEV)
    y = sva.sva_tconv_fwd(xd, wd, bd, F, cache_in=cached, cache_out=cache_out)
    torch.cuda.synchronize()
    ref, ref_last = orc.tconv_fwd(x, w, b, F, cache=cache)
    err = relerr(y, ref)
    _say(f"  err {err:.3g}")
    assert err <= TOL[dtype]
    assert torch.equal(cache_out, xd[:, -1])


def test_tconv_cache_out_may_be_cache_in():
    """cache_out == cache_in updates the cache in place: the output is the
    same as with separate buffers, and the cache ends as the last frame."""
    B, T, Hs, Ws, C, F = 1, 6, 3, 4, 16, 3
    _say("tconv in-place cache")
    _, xd = _draw((B, T, Hs, Ws, C), 111, "bf16")
    _, _, wd, bd = _params(C, 112)
    _, cd = _draw((B, Hs, Ws, C), 114, "bf16")
    y1 = sva.sva_tconv_fwd(xd, wd, bd, F, cache_in=cd)
    c2 = cd.clone()
    y2 = sva.sva_tconv_fwd(xd, wd, bd, F, cache_in=c2, cache_out=c2)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.equal(c2, xd[:, -1])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tconv_streaming_equals_one_shot(dtype):
    """Block by block -- apply against the cache, then commit -- gives the
    one-shot output bit for bit (the same arithmetic per element), apply
    leaves the cache untouched, and the final cache is the last frame."""
    B, F, nb, Hs, Ws, C = 2, 3, 5, 5, 6, 40
    _say(f"tconv streaming {dtype}")
    x, xd = _draw((B, F * nb, Hs, Ws, C), 121, dtype)
    w, b, wd, bd = _params(C, 122)
    c0, c0d = _draw((B, Hs, Ws, C), 124, dtype)
    y_full = sva.sva_tconv_fwd(xd, wd, bd, F, cache_in=c0d)
    cache = c0d.clone()
    for c in range(nb):
        blk = xd[:, c * F:(c + 1) * F].contiguous()
        before = cache.clone()
        yc = sva.sva_tconv_apply(cache, blk, wd, bd)
        torch.cuda.synchronize()
        assert torch.equal(cache, before)
        assert torch.equal(yc, y_full[:, c * F:(c + 1) * F])
        sva.sva_tconv_commit(cache, blk)
    torch.cuda.synchronize()
    assert torch.equal(cache, xd[:, -1])
    ref, _ = orc.tconv_fwd(x, w, b, F, cache=c0)
    assert relerr(y_full, ref) <= TOL[dtype]


def _full_size(name, n_pos, seed):
    w = wl.TCONV_WORKLOADS[name]
    _say(f"tconv {name}: generating")
    xd = torch.empty((w.B, w.T, w.Hs, w.Ws, w.C), dtype=torch.bfloat16, device=DEV)
    rng = np.random.default_rng(seed)
    pos = [(int(h), int(q)) for h, q in zip(rng.integers(0, w.Hs, n_pos), rng.integers(0, w.Ws, n_pos))]
    host = np.empty((w.B, w.T, n_pos, 1, w.C), dtype=np.float32)

    def one(job):
        b, t = job
        return job, wl.tconv_frame(w, b, t)

    with ThreadPoolExecutor(8) as ex:
        for (b, t), (vals, raw) in ex.map(one, [(b, t) for b in range(w.B) for t in range(w.T)]):
            xd[b, t].copy_(to_device(raw, "bf16"))
            for i, (h, q) in enumerate(pos):
                host[b, t, i, 0] = vals[h, q]
    taps, bias = wl.tconv_params(w)
    _say(f"tconv {name}: running")
    last = torch.empty((w.B, w.Hs, w.Ws, w.C), dtype=torch.bfloat16, device=DEV)
    y = sva.sva_tconv_fwd(xd, torch.from_numpy(taps).to(DEV), torch.from_numpy(bias).to(DEV), w.F,
                          cache_out=last)
    torch.cuda.synchronize()
    assert torch.equal(last, xd[:, -1])
    _say(f"tconv {name}: oracle at {n_pos} positions")
    ref, _ = orc.tconv_fwd(host, taps, bias, w.F)
    got = torch.stack([y[:, :, h, q] for h, q in pos], dim=2)[:, :, :, None]
    err = relerr(got, ref)
    _say(f"  err {err:.3g}")
    assert err <= TOL["bf16"]


def test_tconv_720p_sampled_positions():
    _full_size("tconv_720p", 64, 7)


def test_tconv_minute_sampled_positions():
    _full_size("tconv_minute", 32, 8)
