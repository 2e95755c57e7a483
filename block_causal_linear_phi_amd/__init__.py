"""Block-causal ReLU linear attention with numerator-only 3D RoPE and a
constant-size block KV cache (SANA-Video) on AMD MI355X (gfx950).

The computation lives in libsva.so (hand-written HIP kernels behind the C ABI
in include/sva.h, include/sva_tconv.h and include/sva_proj.h); `sva` is its thin
ctypes binding and `autograd` wraps the attention's forward and backward for
torch training.
"""
from .sva import (  # noqa: F401
    SVA_BF16, SVA_F32, SvaDesc, SvaError, make_desc, sva_block_cache_apply, sva_block_cache_commit,
    sva_block_cache_workspace, sva_lin_attn_bwd, sva_lin_attn_bwd_workspace, sva_lin_attn_fwd,
    sva_lin_attn_fwd_save, sva_lin_attn_fwd_workspace, sva_lin_attn_states_bytes, sva_phi_rope_prep,
    SvaTconvDesc, make_tconv_desc, sva_tconv_apply, sva_tconv_commit, sva_tconv_fwd,
    SvaProjDesc, sva_qkv_proj_mxfp4, sva_mxfp4_pack_weights, mxfp4_packed_bytes, sva_proj_lin_attn_fwd,
    mxfp4_acts_bytes, sva_mxfp4_quant_acts, sva_qkv_proj_w4a4, sva_proj_lin_attn_fwd_w4a4,
)
from .autograd import BlockCausalLinearAttention, block_causal_linear_attention  # noqa: F401
