"""Thin ctypes binding of libsva (include/sva.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libsva.so.  torch supplies device memory and the current stream.
If the library is not built, every call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

SVA_F32 = 0
SVA_BF16 = 1

SVA_OK = 0
SVA_ERR_INVALID_ARG = -1
SVA_ERR_UNSUPPORTED = -2
SVA_ERR_WORKSPACE = -3
SVA_ERR_HIP = -4

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsva.so")


class SvaDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int), ("H", ctypes.c_int), ("d", ctypes.c_int),
        ("T", ctypes.c_int), ("Hs", ctypes.c_int), ("Ws", ctypes.c_int),
        ("frames_per_block", ctypes.c_int), ("t0", ctypes.c_int), ("rope", ctypes.c_int),
        ("rope_dt", ctypes.c_int), ("rope_dh", ctypes.c_int), ("rope_dw", ctypes.c_int),
        ("rope_base", ctypes.c_float), ("eps", ctypes.c_float), ("dtype", ctypes.c_int),
    ]


class SvaTconvDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int), ("T", ctypes.c_int), ("Hs", ctypes.c_int), ("Ws", ctypes.c_int),
        ("C", ctypes.c_int), ("frames_per_block", ctypes.c_int), ("dtype", ctypes.c_int),
    ]


class SvaProjDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("N", ctypes.c_int), ("C", ctypes.c_int), ("H", ctypes.c_int),
                ("d", ctypes.c_int)]


class SvaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None

_VP = ctypes.c_void_p
_SIG = {
    "sva_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "sva_version": (ctypes.c_int, []),
    "sva_lin_attn_fwd_workspace": (ctypes.c_int, [ctypes.POINTER(SvaDesc), ctypes.POINTER(ctypes.c_size_t)]),
    "sva_lin_attn_fwd": (ctypes.c_int, [ctypes.POINTER(SvaDesc), _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                        _VP, ctypes.c_size_t, _VP]),
    "sva_lin_attn_fwd_traced": (ctypes.c_int, [ctypes.POINTER(SvaDesc), _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                               _VP, _VP, ctypes.c_size_t, _VP, ctypes.POINTER(_VP)]),
    "sva_lin_attn_bwd_workspace": (ctypes.c_int, [ctypes.POINTER(SvaDesc), ctypes.POINTER(ctypes.c_size_t)]),
    "sva_lin_attn_bwd": (ctypes.c_int, [ctypes.POINTER(SvaDesc)] + [_VP] * 16 + [ctypes.c_size_t, _VP]),
    "sva_lin_attn_states_bytes": (ctypes.c_int, [ctypes.POINTER(SvaDesc), ctypes.POINTER(ctypes.c_size_t)]),
    "sva_lin_attn_fwd_save": (ctypes.c_int, [ctypes.POINTER(SvaDesc)] + [_VP] * 10 + [ctypes.c_size_t, _VP]),
    "sva_block_cache_workspace": (ctypes.c_int, [ctypes.POINTER(SvaDesc), ctypes.POINTER(ctypes.c_size_t)]),
    "sva_block_cache_apply": (ctypes.c_int, [ctypes.POINTER(SvaDesc), _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                             ctypes.c_size_t, _VP]),
    "sva_block_cache_commit": (ctypes.c_int, [ctypes.POINTER(SvaDesc), _VP, _VP, _VP, _VP, _VP,
                                              ctypes.c_size_t, _VP]),
    "sva_phi_rope_prep": (ctypes.c_int, [ctypes.POINTER(SvaDesc), _VP, _VP, _VP, _VP]),
    "sva_tconv_fwd": (ctypes.c_int, [ctypes.POINTER(SvaTconvDesc)] + [_VP] * 7),
    "sva_tconv_apply": (ctypes.c_int, [ctypes.POINTER(SvaTconvDesc)] + [_VP] * 6),
    "sva_tconv_commit": (ctypes.c_int, [ctypes.POINTER(SvaTconvDesc)] + [_VP] * 3),
    "sva_mxfp4_pack_weights": (ctypes.c_int, [ctypes.POINTER(SvaProjDesc)] + [_VP] * 4),
    "sva_qkv_proj_mxfp4": (ctypes.c_int, [ctypes.POINTER(SvaProjDesc)] + [_VP] * 7),
    "sva_proj_lin_attn_fwd_workspace": (ctypes.c_int, [ctypes.POINTER(SvaDesc), ctypes.POINTER(SvaProjDesc),
                                                        ctypes.POINTER(ctypes.c_size_t)]),
    "sva_proj_lin_attn_fwd": (ctypes.c_int, [ctypes.POINTER(SvaDesc), ctypes.POINTER(SvaProjDesc)] + [_VP] * 9
                              + [ctypes.c_size_t, _VP]),
}


def lib():
    """The loaded libsva.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libsva.so is not built ({LIB_PATH}); run __graft_entry__.build()")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIG.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().sva_status_string(status).decode()


def make_desc(B: int, H: int, d: int, grid: Sequence[int], frames_per_block: int, *, t0: int = 0,
              rope: bool = False, split: Optional[Sequence[int]] = None, base: float = 10000.0,
              eps: float = 1e-6, dtype: int = SVA_BF16) -> SvaDesc:
    T, Hs, Ws = grid
    dt, dh, dw = split if (rope and split is not None) else (0, 0, 0)
    return SvaDesc(B, H, d, T, Hs, Ws, frames_per_block, t0, 1 if rope else 0, dt, dh, dw,
                   float(base), float(eps), dtype)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return SVA_BF16
    if t.dtype == torch.float32:
        return SVA_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")


def _check(status: int, where: str):
    if status != SVA_OK:
        raise SvaError(status, where)


def _desc_from(q, grid, F, t0, rope, split, base, eps) -> SvaDesc:
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, H, N, d = q.shape
    return make_desc(B, H, d, grid, F, t0=t0, rope=rope, split=split, base=base, eps=eps,
                     dtype=_dtype_code(q))


def sva_lin_attn_fwd_workspace(desc: SvaDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().sva_lin_attn_fwd_workspace(ctypes.byref(desc), ctypes.byref(n)), "sva_lin_attn_fwd_workspace")
    return n.value


def sva_lin_attn_bwd_workspace(desc: SvaDesc) -> int:
    n = ctypes.c_size_t()
    _check(lib().sva_lin_attn_bwd_workspace(ctypes.byref(desc), ctypes.byref(n)), "sva_lin_attn_bwd_workspace")
    return n.value


def sva_block_cache_workspace(desc: SvaDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().sva_block_cache_workspace(ctypes.byref(desc), ctypes.byref(n)), "sva_block_cache_workspace")
    return n.value


def _workspace(nbytes: int, like, ws):
    import torch
    if ws is not None:
        return ws
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=like.device)


def sva_lin_attn_fwd(q, k, v, grid: Tuple[int, int, int], frames_per_block: int, *, t0: int = 0,
                     rope: bool = False, split=None, base: float = 10000.0, eps: float = 1e-6,
                     S0=None, z0=None, out=None, S_out=None, z_out=None, ws=None, stream=None,
                     events=None):
    """One-shot block-causal forward (sva_lin_attn_fwd).  Returns `out`."""
    import torch
    desc = _desc_from(q, grid, frames_per_block, t0, rope, split, base, eps)
    if out is None:
        out = torch.empty_like(q)
    nbytes = sva_lin_attn_fwd_workspace(desc)
    ws = _workspace(nbytes, q, ws)
    args = (ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(S0), _ptr(z0), _ptr(S_out),
            _ptr(z_out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    if events is None:
        st = lib().sva_lin_attn_fwd(*args)
    else:
        arr = (_VP * 4)(*[ctypes.c_void_p(e) for e in events])
        st = lib().sva_lin_attn_fwd_traced(*args, arr)
    _check(st, "sva_lin_attn_fwd")
    return out


def sva_lin_attn_states_bytes(desc: SvaDesc) -> int:
    n = ctypes.c_size_t()
    _check(lib().sva_lin_attn_states_bytes(ctypes.byref(desc), ctypes.byref(n)), "sva_lin_attn_states_bytes")
    return n.value


def sva_lin_attn_fwd_save(q, k, v, grid: Tuple[int, int, int], frames_per_block: int, *, t0: int = 0,
                          rope: bool = False, split=None, base: float = 10000.0, eps: float = 1e-6,
                          S0=None, z0=None, out=None, S_out=None, z_out=None, states=None, ws=None,
                          stream=None):
    """Forward that keeps its prefix states for the backward
    (sva_lin_attn_fwd_save).  Returns (out, states)."""
    import torch
    desc = _desc_from(q, grid, frames_per_block, t0, rope, split, base, eps)
    if out is None:
        out = torch.empty_like(q)
    if states is None:
        states = torch.empty(sva_lin_attn_states_bytes(desc), dtype=torch.uint8, device=q.device)
    ws = _workspace(sva_lin_attn_fwd_workspace(desc), q, ws)
    st = lib().sva_lin_attn_fwd_save(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(S0),
                                     _ptr(z0), _ptr(S_out), _ptr(z_out), _ptr(states), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "sva_lin_attn_fwd_save")
    return out, states


def sva_lin_attn_bwd(q, k, v, out, dout, grid: Tuple[int, int, int], frames_per_block: int, *, t0: int = 0,
                     rope: bool = False, split=None, base: float = 10000.0, eps: float = 1e-6,
                     S0=None, z0=None, dS_out=None, dz_out=None, states=None, dq=None, dk=None, dv=None,
                     dS0=None, dz0=None, ws=None, stream=None):
    """Gradients of the forward (sva_lin_attn_bwd), bf16.  Returns (dq, dk, dv);
    dS0/dz0 are filled when given.  `states` from sva_lin_attn_fwd_save
    skips recomputing the forward's prefix states."""
    import torch
    desc = _desc_from(q, grid, frames_per_block, t0, rope, split, base, eps)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    ws = _workspace(sva_lin_attn_bwd_workspace(desc), q, ws)
    st = lib().sva_lin_attn_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout),
                                _ptr(S0), _ptr(z0), _ptr(dS_out), _ptr(dz_out), _ptr(states), _ptr(dq),
                                _ptr(dk), _ptr(dv),
                                _ptr(dS0), _ptr(dz0), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "sva_lin_attn_bwd")
    return dq, dk, dv


def sva_block_cache_apply(S, z, q, k, v, frame_grid: Tuple[int, int, int], *, t0: int, rope: bool = False,
                          split=None, base: float = 10000.0, eps: float = 1e-6, out=None, ws=None,
                          stream=None):
    """Output of one block against the committed cache (S, z); the cache is
    not modified.  frame_grid = (F, Hs, Ws).  Returns `out`."""
    import torch
    desc = _desc_from(q, frame_grid, frame_grid[0], t0, rope, split, base, eps)
    if out is None:
        out = torch.empty_like(q)
    ws = _workspace(sva_block_cache_workspace(desc), q, ws)
    st = lib().sva_block_cache_apply(ctypes.byref(desc), _ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "sva_block_cache_apply")
    return out


def sva_block_cache_commit(S, z, k, v, frame_grid: Tuple[int, int, int], *, t0: int, rope: bool = False,
                           split=None, base: float = 10000.0, ws=None, stream=None):
    """Adds one block's K, V to the cache (S, z) in place."""
    desc = _desc_from(k, frame_grid, frame_grid[0], t0, rope, split, base, 0.0)
    ws = _workspace(sva_block_cache_workspace(desc), k, ws)
    st = lib().sva_block_cache_commit(ctypes.byref(desc), _ptr(S), _ptr(z), _ptr(k), _ptr(v), _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "sva_block_cache_commit")


def sva_phi_rope_prep(x, grid: Tuple[int, int, int], *, t0: int = 0, rope: bool = False, split=None,
                      base: float = 10000.0, want_phi: bool = True, stream=None):
    """The phi + RoPE stage alone: returns (RoPE(phi x), phi x) as fp32."""
    import torch
    desc = _desc_from(x, grid, grid[0], t0, rope, split, base, 0.0)
    xr = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    xp = torch.empty_like(xr) if want_phi else None
    st = lib().sva_phi_rope_prep(ctypes.byref(desc), _ptr(x), _ptr(xr), _ptr(xp), _stream(stream))
    _check(st, "sva_phi_rope_prep")
    return xr, xp


# Causal temporal convolution with a one-token block cache (include/sva_tconv.h).

def make_tconv_desc(B: int, T: int, Hs: int, Ws: int, C: int, frames_per_block: int,
                    dtype: int = SVA_BF16) -> SvaTconvDesc:
    return SvaTconvDesc(B, T, Hs, Ws, C, frames_per_block, dtype)


def _tconv_desc_from(x, F) -> SvaTconvDesc:
    if x.dim() != 5:
        raise ValueError("x must be [B, T, Hs, Ws, C]")
    B, T, Hs, Ws, C = x.shape
    return make_tconv_desc(B, T, Hs, Ws, C, F, _dtype_code(x))


def sva_tconv_fwd(x, w, bias, frames_per_block: int, *, cache_in=None, y=None, cache_out=None,
                  stream=None):
    """Block-causal temporal convolution over all blocks of x [B, T, Hs, Ws, C]
    with taps w [C, 3] and bias [C] (fp32; bias may be None).  cache_in is the
    frame carried into block 0 (None: zero); cache_out, if given, receives the
    last frame.  Returns y."""
    import torch
    desc = _tconv_desc_from(x, frames_per_block)
    if y is None:
        y = torch.empty_like(x)
    st = lib().sva_tconv_fwd(ctypes.byref(desc), _ptr(x), _ptr(w), _ptr(bias), _ptr(cache_in), _ptr(y),
                             _ptr(cache_out), _stream(stream))
    _check(st, "sva_tconv_fwd")
    return y


def sva_tconv_apply(cache, x, w, bias, *, y=None, stream=None):
    """Output of one block x [B, F, Hs, Ws, C] against the cache [B, Hs, Ws, C];
    the cache is not modified.  Returns y."""
    import torch
    desc = _tconv_desc_from(x, x.shape[1])
    if y is None:
        y = torch.empty_like(x)
    st = lib().sva_tconv_apply(ctypes.byref(desc), _ptr(cache), _ptr(x), _ptr(w), _ptr(bias), _ptr(y),
                               _stream(stream))
    _check(st, "sva_tconv_apply")
    return y


def sva_tconv_commit(cache, x, *, stream=None):
    """cache <- the last frame of one block x [B, F, Hs, Ws, C], in place."""
    desc = _tconv_desc_from(x, x.shape[1])
    st = lib().sva_tconv_commit(ctypes.byref(desc), _ptr(cache), _ptr(x), _stream(stream))
    _check(st, "sva_tconv_commit")


# QKV projection with MXFP4 weights (include/sva_proj.h).

def mxfp4_packed_bytes(n_out: int, C: int) -> int:
    """Size of the packed weights: that of the codes plus the scales."""
    return n_out * C // 2 + n_out * C // 32


def sva_mxfp4_pack_weights(codes, scales, H: int, d: int, *, out=None, stream=None):
    """codes [3 H d, C / 2] uint8 (two 4-bit codes a byte, low nibble first),
    scales [3 H d, C / 32] uint8 (E8M0) -> the packed weights (uint8 tensor)
    that sva_qkv_proj_mxfp4 takes.  Weights are constant: pack them once."""
    import torch
    n_out, half = codes.shape
    C = 2 * half
    if out is None:
        out = torch.empty((mxfp4_packed_bytes(n_out, C),), dtype=torch.uint8, device=codes.device)
    desc = SvaProjDesc(1, 1, C, H, d)
    st = lib().sva_mxfp4_pack_weights(ctypes.byref(desc), _ptr(codes), _ptr(scales), _ptr(out), _stream(stream))
    _check(st, "sva_mxfp4_pack_weights")
    return out


def sva_qkv_proj_mxfp4(x, wpack, bias, H: int, d: int, *, q=None, k=None, v=None, stream=None):
    """x [B, N, C] bf16; wpack from sva_mxfp4_pack_weights; bias [3 H d]
    fp32 or None.  Returns (q, k, v), each [B, H, N, d] bf16."""
    import torch
    if x.dim() != 3 or x.dtype != torch.bfloat16:
        raise ValueError("x must be [B, N, C] bf16")
    B, N, C = x.shape
    desc = SvaProjDesc(B, N, C, H, d)
    outs = []
    for t in (q, k, v):
        outs.append(torch.empty((B, H, N, d), dtype=torch.bfloat16, device=x.device) if t is None else t)
    st = lib().sva_qkv_proj_mxfp4(ctypes.byref(desc), _ptr(x), _ptr(wpack), _ptr(bias),
                                  _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]), _stream(stream))
    _check(st, "sva_qkv_proj_mxfp4")
    return tuple(outs)


def sva_proj_lin_attn_fwd(x, wpack, bias, H: int, grid: Tuple[int, int, int], frames_per_block: int, *,
                          t0: int = 0, rope: bool = False, split=None, base: float = 10000.0, eps: float = 1e-6,
                          S0=None, z0=None, S_out=None, z_out=None, out=None, ws=None, stream=None):
    """Projection and attention fused (sva_proj_lin_attn_fwd): x [B, N, C]
    bf16 with N = T * Hs * Ws; wpack from sva_mxfp4_pack_weights for H heads
    of d = 64; bias [3 H 64] fp32 or None.  Returns out [B, H, N, 64] bf16."""
    import torch
    if x.dim() != 3 or x.dtype != torch.bfloat16:
        raise ValueError("x must be [B, N, C] bf16")
    B, N, C = x.shape
    q_like = torch.empty((B, H, N, 64), dtype=torch.bfloat16, device=x.device) if out is None else out
    desc = _desc_from(q_like, grid, frames_per_block, t0, rope, split, base, eps)
    pdesc = SvaProjDesc(B, N, C, H, 64)
    n = ctypes.c_size_t()
    _check(lib().sva_proj_lin_attn_fwd_workspace(ctypes.byref(desc), ctypes.byref(pdesc), ctypes.byref(n)),
           "sva_proj_lin_attn_fwd_workspace")
    ws = _workspace(n.value, x, ws)
    st = lib().sva_proj_lin_attn_fwd(ctypes.byref(desc), ctypes.byref(pdesc), _ptr(x), _ptr(wpack), _ptr(bias),
                                     _ptr(q_like), _ptr(S0), _ptr(z0), _ptr(S_out), _ptr(z_out), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "sva_proj_lin_attn_fwd")
    return q_like
