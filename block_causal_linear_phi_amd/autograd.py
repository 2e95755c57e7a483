"""torch.autograd wrapper of the block-causal linear attention, for block-
causal training: the forward runs sva_lin_attn_fwd_save (keeping its prefix
states), the backward runs sva_lin_attn_bwd on those states.  Argument
marshalling only: every step runs in libsva's kernels.  bf16 inputs.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import torch

from . import sva


class BlockCausalLinearAttention(torch.autograd.Function):
    """out = block-causal ReLU linear attention with numerator-only 3D RoPE
    (see sva.sva_lin_attn_fwd); gradients for q, k, v and, when given, the
    initial cache S0, z0."""

    @staticmethod
    def forward(ctx, q, k, v, grid, frames_per_block, t0, rope, split, base, eps, S0, z0):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        out, states = sva.sva_lin_attn_fwd_save(q, k, v, grid, frames_per_block, t0=t0, rope=rope, split=split,
                                                base=base, eps=eps, S0=S0, z0=z0)
        ctx.save_for_backward(q, k, v, states, S0, z0)  # the output is formed again in the backward
        ctx.cfg = dict(grid=grid, frames_per_block=frames_per_block, t0=t0, rope=rope, split=split, base=base,
                       eps=eps)
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, states, S0, z0 = ctx.saved_tensors
        c = ctx.cfg
        dS0 = dz0 = None
        if S0 is not None and (ctx.needs_input_grad[10] or ctx.needs_input_grad[11]):
            dS0 = torch.empty_like(S0)
            dz0 = torch.empty_like(z0)
        dq, dk, dv = sva.sva_lin_attn_bwd(q, k, v, dout.contiguous(), c["grid"], c["frames_per_block"],
                                          t0=c["t0"], rope=c["rope"], split=c["split"], base=c["base"],
                                          eps=c["eps"], S0=S0, z0=z0, states=states, dS0=dS0, dz0=dz0)
        return dq, dk, dv, None, None, None, None, None, None, None, dS0, dz0


def block_causal_linear_attention(q, k, v, grid: Tuple[int, int, int], frames_per_block: int, *, t0: int = 0,
                                  rope: bool = False, split: Optional[Sequence[int]] = None,
                                  base: float = 10000.0, eps: float = 1e-6, S0=None, z0=None):
    """Differentiable forward: q, k, v [B, H, N, d] bf16 (N = T*Hs*Ws),
    optional initial cache S0 [B, H, d, d], z0 [B, H, d] fp32."""
    return BlockCausalLinearAttention.apply(q, k, v, tuple(grid), frames_per_block, t0, rope,
                                            None if split is None else tuple(split), base, eps, S0, z0)
