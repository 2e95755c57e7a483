"""Seeded synthetic inputs for block-causal linear attention.

This module only draws and rounds numbers; it holds none of the method's
arithmetic.  The same bits feed the HIP library (uploaded by torch) and the
fp64 oracle (upcast), so parity compares the two on identical inputs.

Every (workload, tensor, batch, head, step) slice has its own seed, drawn with
numpy's PCG64 as float32 N(0, 1), scaled where the workload says so, then
rounded to bf16 (round-to-nearest-even) for bf16 workloads.  Any slice can be
regenerated alone, which keeps the oracle's memory bounded at large sizes.

The latent grids are video-shaped: a 480p clip of 81 frames becomes a
21 x 30 x 52 latent grid and a 720p clip a 21 x 45 x 80 grid (75,600 tokens,
the ">75000 tokens" the cstia.com SANA-Video article quotes for a 5-second
720p video); blocks are 3 latent frames.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    d: int
    T: int
    Hs: int
    Ws: int
    F: int
    dtype: str                      # "f32" or "bf16"
    rope: bool
    split: Tuple[int, int, int] = (0, 0, 0)
    base: float = 10000.0
    eps: float = 1e-6
    k_scale: float = 1.0
    t0: int = 0
    steps: int = 1                  # denoising steps (cached-step workload)
    prior_blocks: int = 0           # committed blocks before the current one

    @property
    def N(self) -> int:
        return self.T * self.Hs * self.Ws

    @property
    def nb(self) -> int:
        return self.T // self.F

    @property
    def block_tokens(self) -> int:
        return self.F * self.Hs * self.Ws


WORKLOADS = {
    # 4 blocks x 64 tokens, fp32, no RoPE; grid 4 x 8 x 8 with 1 frame a block
    "tiny": Workload("tiny", B=1, H=2, d=32, T=4, Hs=8, Ws=8, F=1, dtype="f32", rope=False),
    "480p": Workload("480p", B=1, H=16, d=64, T=21, Hs=30, Ws=52, F=3, dtype="bf16",
                     rope=True, split=(16, 24, 24)),
    # one 3-frame block at t0 = 18 against a cache of 6 prior blocks, 4 steps
    "cached_step": Workload("cached_step", B=1, H=16, d=64, T=3, Hs=30, Ws=52, F=3,
                            dtype="bf16", rope=True, split=(16, 24, 24), t0=18, steps=4,
                            prior_blocks=6),
    "720p": Workload("720p", B=1, H=16, d=64, T=21, Hs=45, Ws=80, F=3, dtype="bf16",
                     rope=True, split=(16, 24, 24), k_scale=0.5),
    "minute": Workload("minute", B=2, H=16, d=64, T=240, Hs=30, Ws=52, F=3, dtype="bf16",
                       rope=True, split=(16, 24, 24)),
}


def seed_for(workload: str, tensor: str, b: int, h: int, step: int = 0) -> int:
    return zlib.crc32(f"{workload}/{tensor}/{b}/{h}/{step}".encode()) & 0x7FFFFFFF


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round-to-nearest-even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def draw(shape, seed: int, scale: float = 1.0, dtype: str = "bf16"):
    """N(0,1) * scale as float32 values exactly representable in `dtype`.
    Returns (values_f32, raw) where raw is uint16 bf16 bits or float32."""
    x = np.random.default_rng(np.random.PCG64(seed)).standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x = (x * np.float32(scale)).astype(np.float32)
    if dtype == "bf16":
        bits = round_to_bf16_bits(x)
        return bf16_bits_to_f32(bits), bits
    return x, x


def slice_qkv(w: Workload, tensor: str, b: int, h: int, step: int = 0, n_tokens: Optional[int] = None):
    """One [N, d] slice of Q, K or V for (b, h, step)."""
    n = w.N if n_tokens is None else n_tokens
    scale = w.k_scale if tensor == "k" else 1.0
    return draw((n, w.d), seed_for(w.name, tensor, b, h, step), scale, w.dtype)


def full_qkv(w: Workload, step: int = 0, n_tokens: Optional[int] = None, heads=None):
    """Stacked [B, H, N, d] host arrays for q, k, v: returns dict of
    (values_f32, raw) per tensor.  `heads` restricts to a list of (b, h)."""
    n = w.N if n_tokens is None else n_tokens
    out = {}
    for tensor in ("q", "k", "v"):
        vals = np.empty((w.B, w.H, n, w.d), dtype=np.float32)
        raw = np.empty((w.B, w.H, n, w.d), dtype=np.uint16 if w.dtype == "bf16" else np.float32)
        for b in range(w.B):
            for h in range(w.H):
                if heads is not None and (b, h) not in heads:
                    vals[b, h] = 0
                    raw[b, h] = 0
                    continue
                vals[b, h], raw[b, h] = slice_qkv(w, tensor, b, h, step, n)
        out[tensor] = (vals, raw)
    return out


# Causal temporal convolution of the Mix-FFN.  The pages give no FFN width;
# the channel count here is the attention workloads' model width, H * d =
# 16 * 64 = 1024, on the same latent grids.  Activations are drawn per
# (workload, b, frame) slice [Hs * Ws, C]; taps N(0, 1/3) and bias N(0, 0.01)
# in fp32; the cache (a carried frame) like one activation frame.

@dataclass(frozen=True)
class TconvWorkload:
    name: str
    B: int
    T: int
    Hs: int
    Ws: int
    C: int
    F: int
    dtype: str                      # "f32" or "bf16"

    @property
    def nb(self) -> int:
        return self.T // self.F

    @property
    def elems(self) -> int:
        return self.B * self.T * self.Hs * self.Ws * self.C


TCONV_WORKLOADS = {
    "tconv_tiny": TconvWorkload("tconv_tiny", B=1, T=4, Hs=8, Ws=8, C=32, F=1, dtype="f32"),
    "tconv_720p": TconvWorkload("tconv_720p", B=1, T=21, Hs=45, Ws=80, C=1024, F=3, dtype="bf16"),
    "tconv_minute": TconvWorkload("tconv_minute", B=2, T=240, Hs=30, Ws=52, C=1024, F=3, dtype="bf16"),
}


def tconv_frame(w: TconvWorkload, b: int, t: int, tensor: str = "x"):
    """One activation frame [Hs, Ws, C] of (b, t): (values_f32, raw)."""
    vals, raw = draw((w.Hs * w.Ws * w.C,), seed_for(w.name, tensor, b, t), 1.0, w.dtype)
    shape = (w.Hs, w.Ws, w.C)
    return vals.reshape(shape), raw.reshape(shape)


def tconv_params(w: TconvWorkload):
    """(taps [C, 3], bias [C]) as float32."""
    taps, _ = draw((w.C, 3), seed_for(w.name, "w", 0, 0), float(np.sqrt(1.0 / 3.0)), "f32")
    bias, _ = draw((w.C,), seed_for(w.name, "bias", 0, 0), 0.1, "f32")
    return taps, bias


# QKV projection with MXFP4 weights.  The pages give no model width; the
# input channels are the attention workloads' H * d = 1024 (as for the
# temporal convolution), the outputs [q | k | v] for 16 heads of 64.  Codes
# are uniform over the 16 E2M1 values; block scales are E8M0 bytes 120..124
# (2^-7 .. 2^-3); activations N(0, 1) bf16, drawn per (workload, b, token
# block of 4096) slice; bias N(0, 0.01) fp32.

@dataclass(frozen=True)
class ProjWorkload:
    name: str
    B: int
    N: int
    C: int
    H: int
    d: int

    @property
    def n_out(self) -> int:
        return 3 * self.H * self.d


PROJ_WORKLOADS = {
    "proj_720p": ProjWorkload("proj_720p", B=1, N=75600, C=1024, H=16, d=64),
    "proj_480p": ProjWorkload("proj_480p", B=1, N=32760, C=1024, H=16, d=64),
    "proj_minute": ProjWorkload("proj_minute", B=2, N=374400, C=1024, H=16, d=64),
}


def mxfp4_weights(n_out: int, C: int, seed: int):
    """(codes [n_out, C] uint8 in 0..15, scales [n_out, C // 32] uint8)."""
    rng = np.random.default_rng(np.random.PCG64(seed))
    codes = rng.integers(0, 16, (n_out, C), dtype=np.uint8)
    scales = rng.integers(120, 125, (n_out, C // 32), dtype=np.uint8)
    return codes, scales


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[rows, C] 4-bit codes -> [rows, C // 2] bytes, channel 2j in the low
    nibble of byte j and channel 2j + 1 in the high nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
