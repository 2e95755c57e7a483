"""GPU parity of the QKV projection with MXFP4 weights (sva_qkv_proj_mxfp4)
against the fp64 oracle (oracle/proj_oracle.py) on identical seeded inputs.

Bar: max|gpu - oracle| / max|oracle| <= 1e-2 per output tensor (bf16
inputs and outputs; the weights decode exactly and the products accumulate
in fp32, so the bf16 output rounding dominates).  The weights go through
sva_mxfp4_pack_weights first.  Small cases cover a ragged last token tile,
sample boundaries inside a tile, several channel stages, partial feature
tiles, d = 32 and 64, no bias, and extreme E8M0 scales (denormal weights,
and weights up to 6 * 2^125); the 720p-sized projection runs in full and is
compared on sampled tokens.
"""
import sys

import numpy as np
import pytest
import torch

from block_causal_linear_phi_amd import sva
from block_causal_linear_phi_amd import workloads as wl
from gpu_helpers import DEV, TOL, relerr, to_device
from oracle import proj_oracle as orc

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _weights(n_out, C, seed, lo=120, hi=125):
    codes, scales = wl.mxfp4_weights(n_out, C, seed)
    if (lo, hi) != (120, 125):
        scales = np.random.default_rng(seed + 7).integers(lo, hi, scales.shape, dtype=np.uint8)
    cd = torch.from_numpy(wl.pack_nibbles(codes)).to(DEV)
    sd = torch.from_numpy(scales).to(DEV)
    return codes, scales, cd, sd


# (name, B, N, C, H, d, bias): ragged token tiles, partial feature tiles
# (3 H d = 192, 384, 576), sample boundaries inside a tile, 1 to 3 stages.
CASES = [
    ("ragged_tile", 1, 100, 128, 2, 64, True),
    ("samples_in_tile", 2, 300, 128, 4, 32, True),
    ("three_stages", 1, 513, 384, 2, 64, False),
    ("several_tiles", 3, 700, 256, 8, 32, True),
    ("one_block_rows", 2, 130, 256, 1, 64, True),
    ("three_blocks", 1, 257, 128, 3, 64, True),
    ("one_token", 1, 1, 128, 1, 64, True),
    ("whole_tiles", 2, 128, 256, 4, 64, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_proj_small(case):
    name, B, N, C, H, d, with_bias = case
    _say(f"proj_small {name}")
    xv, xraw = wl.draw((B, N, C), 201, 1.0, "bf16")
    xd = to_device(xraw, "bf16")
    codes, scales, cd, sd = _weights(3 * H * d, C, 202)
    wp = sva.sva_mxfp4_pack_weights(cd, sd, H, d)
    bias = bd = None
    if with_bias:
        bias = wl.draw((3 * H * d,), 203, 0.1, "f32")[0]
        bd = torch.from_numpy(bias).to(DEV)
    q, k, v = sva.sva_qkv_proj_mxfp4(xd, wp, bd, H, d)
    torch.cuda.synchronize()
    ref = orc.qkv_project(xv, codes, scales, bias, H, d)
    errs = [relerr(g_, r_) for g_, r_ in zip((q, k, v), ref)]
    _say(f"  errs {errs}")
    assert max(errs) <= TOL["bf16"]


@pytest.mark.parametrize("lo,hi,x_scale", [(0, 2, 2.0 ** 100), (248, 253, 2.0 ** -100)],
                         ids=["denormal_weights", "huge_weights"])
def test_proj_extreme_scales(lo, hi, x_scale):
    """E8M0 bytes 0 and 1 (2^-127, 2^-126: denormal weights) against 2^100
    activations, and bytes 248..252 (weights up to 6 * 2^125, the largest
    below the bf16 and fp32 limit) against 2^-100 activations: every product
    and sum stays in range, and the weights decode exactly."""
    B, N, C, H, d = 1, 64, 128, 2, 64
    _say(f"proj extreme scales {lo}..{hi - 1}")
    codes, scales, cd, sd = _weights(3 * H * d, C, 211, lo, hi)
    wp = sva.sva_mxfp4_pack_weights(cd, sd, H, d)
    xv, xraw = wl.draw((B, N, C), 213, x_scale, "bf16")
    q, k, v = sva.sva_qkv_proj_mxfp4(to_device(xraw, "bf16"), wp, None, H, d)
    torch.cuda.synchronize()
    ref = orc.qkv_project(xv, codes, scales, None, H, d)
    for g_, r_ in zip((q, k, v), ref):
        assert bool(torch.isfinite(g_.float()).all())
        err = relerr(g_, r_)
        _say(f"  err {err:.3g}")
        assert err <= TOL["bf16"]


def test_proj_720p_sampled_tokens():
    w = wl.PROJ_WORKLOADS["proj_720p"]
    _say("proj 720p: generating")
    xd = torch.empty((w.B, w.N, w.C), dtype=torch.bfloat16, device=DEV)
    blocks = {}
    for j, s0 in enumerate(range(0, w.N, 4096)):
        n = min(4096, w.N - s0)
        vals, raw = wl.draw((n, w.C), wl.seed_for(w.name, "x", 0, j), 1.0, "bf16")
        xd[0, s0:s0 + n].copy_(to_device(raw, "bf16"))
        blocks[s0] = vals
    codes, scales = wl.mxfp4_weights(w.n_out, w.C, wl.seed_for(w.name, "w", 0, 0))
    bias = wl.draw((w.n_out,), wl.seed_for(w.name, "bias", 0, 0), 0.1, "f32")[0]
    _say("proj 720p: running")
    wp = sva.sva_mxfp4_pack_weights(torch.from_numpy(wl.pack_nibbles(codes)).to(DEV),
                                    torch.from_numpy(scales).to(DEV), w.H, w.d)
    q, k, v = sva.sva_qkv_proj_mxfp4(xd, wp, torch.from_numpy(bias).to(DEV), w.H, w.d)
    torch.cuda.synchronize()
    toks = np.random.default_rng(5).choice(w.N, 96, replace=False)
    toks.sort()
    xs = np.stack([blocks[t // 4096 * 4096][t % 4096] for t in toks])[None]
    ref = orc.qkv_project(xs, codes, scales, bias, w.H, w.d)
    idx = torch.from_numpy(toks).to(DEV)
    errs = [relerr(g_[:, :, idx], r_) for g_, r_ in zip((q, k, v), ref)]
    _say(f"  errs {errs}")
    assert max(errs) <= TOL["bf16"]


def test_pack_layout_matches_header():
    """sva_mxfp4_pack_weights writes the layout include/sva_proj.h spells
    out: with P = 3 H d / 64 row blocks and S = C / 128 stages, codes entry
    (p, s, t, l) = the 16 code bytes of channels 128 s + 32 (l / 16) .. + 31
    of row 64 p + r(t, l % 16), then scale word (p, s, l) with byte t the
    scale of that block; r(t, i) = 32 (t / 2) + 8 (i / 4) + 4 (t % 2) + i % 4.
    The expected bytes are rebuilt here with numpy from that text."""
    H, d, C = 2, 96, 384
    n_out = 3 * H * d
    _say("pack layout")
    codes, scales, cd, sd = _weights(n_out, C, 221)
    packed = sva.sva_mxfp4_pack_weights(cd, sd, H, d).cpu().numpy()
    nib = wl.pack_nibbles(codes)  # [n_out, C / 2]
    P, S = n_out // 64, C // 128
    t = np.arange(4)[:, None]
    i = np.arange(64)[None, :] % 16
    rows = 32 * (t // 2) + 8 * (i // 4) + 4 * (t % 2) + i % 4  # [4, 64]
    lg = np.arange(64) // 16
    exp_c = np.empty((P, S, 4, 64, 16), np.uint8)
    exp_s = np.empty((P, S, 64, 4), np.uint8)
    for p in range(P):
        for s in range(S):
            for tt in range(4):
                for l in range(64):
                    n = 64 * p + rows[tt, l]
                    ch0 = 128 * s + 32 * lg[l]
                    exp_c[p, s, tt, l] = nib[n, ch0 // 2: ch0 // 2 + 16]
                    exp_s[p, s, l, tt] = scales[n, ch0 // 32]
    nc = n_out * C // 2
    assert packed.shape == (nc + n_out * C // 32,)
    assert np.array_equal(packed[:nc], exp_c.reshape(-1))
    assert np.array_equal(packed[nc:], exp_s.reshape(-1))
