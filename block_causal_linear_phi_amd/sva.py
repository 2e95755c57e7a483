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

SVA_STAGE_REDUCE = 1
SVA_STAGE_SCAN = 2
SVA_STAGE_APPLY = 4
SVA_STAGE_ALL = 7

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
    # range_tokens: the fused entry point's reduction range length (0 = chosen
    # by the library); the pack and projection calls ignore it
    _fields_ = [("B", ctypes.c_int), ("N", ctypes.c_int), ("C", ctypes.c_int), ("H", ctypes.c_int),
                ("d", ctypes.c_int), ("range_tokens", ctypes.c_int)]


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
    "sva_lin_attn_fwd_stages": (ctypes.c_int, [ctypes.POINTER(SvaDesc), _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                               _VP, _VP, ctypes.c_size_t, _VP, ctypes.c_int]),
    "sva_lin_attn_bwd_workspace": (ctypes.c_int, [ctypes.POINTER(SvaDesc), ctypes.POINTER(ctypes.c_size_t)]),
    "sva_lin_attn_bwd": (ctypes.c_int, [ctypes.POINTER(SvaDesc)] + [_VP] * 15 + [ctypes.c_size_t, _VP]),
    "sva_lin_attn_states_bytes": (ctypes.c_int, [ctypes.POINTER(SvaDesc), ctypes.POINTER(ctypes.c_size_t)]),
    "sva_lin_attn_fwd_save": (ctypes.c_int, [ctypes.POINTER(SvaDesc)] + [_VP] * 10 + [ctypes.c_size_t, _VP]),
    "sva_block_cache_workspace": (ctypes.c_int, [ctypes.POINTER(SvaDesc), ctypes.POINTER(ctypes.c_size_t)]),
    "sva_block_cache_apply": (ctypes.c_int, [ctypes.POINTER(SvaDesc), _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                             ctypes.c_size_t, _VP]),
    "sva_block_cache_commit": (ctypes.c_int, [ctypes.POINTER(SvaDesc), _VP, _VP, _VP, _VP, _VP,
                                              ctypes.c_size_t, _VP]),
    "sva_block_cache_apply_noalloc": (ctypes.c_int, [ctypes.POINTER(SvaDesc), _VP, _VP, _VP, _VP, _VP, _VP,
                                                     _VP]),
    "sva_phi_rope_prep": (ctypes.c_int, [ctypes.POINTER(SvaDesc), _VP, _VP, _VP, _VP]),
    "sva_tconv_fwd": (ctypes.c_int, [ctypes.POINTER(SvaTconvDesc)] + [_VP] * 7),
    "sva_tconv_apply": (ctypes.c_int, [ctypes.POINTER(SvaTconvDesc)] + [_VP] * 6),
    "sva_tconv_commit": (ctypes.c_int, [ctypes.POINTER(SvaTconvDesc)] + [_VP] * 3),
    "sva_mxfp4_pack_weights": (ctypes.c_int, [ctypes.POINTER(SvaProjDesc)] + [_VP] * 4),
    "sva_qkv_proj_mxfp4": (ctypes.c_int, [ctypes.POINTER(SvaProjDesc)] + [_VP] * 7),
    "sva_mxfp4_acts_bytes": (ctypes.c_int, [ctypes.POINTER(SvaProjDesc), ctypes.POINTER(ctypes.c_size_t)]),
    "sva_mxfp4_quant_acts": (ctypes.c_int, [ctypes.POINTER(SvaProjDesc)] + [_VP] * 3),
    "sva_qkv_proj_w4a4": (ctypes.c_int, [ctypes.POINTER(SvaProjDesc)] + [_VP] * 7),
    "sva_proj_lin_attn_fwd_workspace": (ctypes.c_int, [ctypes.POINTER(SvaDesc), ctypes.POINTER(SvaProjDesc),
                                                        ctypes.POINTER(ctypes.c_size_t)]),
    "sva_proj_lin_attn_fwd": (ctypes.c_int, [ctypes.POINTER(SvaDesc), ctypes.POINTER(SvaProjDesc)] + [_VP] * 9
                              + [ctypes.c_size_t, _VP]),
    "sva_proj_lin_attn_fwd_w4a4": (ctypes.c_int, [ctypes.POINTER(SvaDesc), ctypes.POINTER(SvaProjDesc)] + [_VP] * 9
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
    """The HIP stream handle of `stream`, else of the current device's current
    stream (torch's raw getter: 0.1 us against 2.7 us for
    torch.cuda.current_stream(), which a tiny call would otherwise spend)."""
    import torch
    if stream is not None:
        return stream.cuda_stream
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    dev = getattr(torch._C, "_cuda_getDevice", None)
    if raw is None or dev is None:
        return torch.cuda.current_stream().cuda_stream
    return raw(dev())


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


# Argument checks.  The C ABI sees only pointers, so the binding is where
# tensor shapes, dtypes, contiguity and devices are checked; every check runs
# before the library is called and raises ValueError (TypeError for a
# non-tensor or an unsupported dtype).  Shapes, dtypes and contiguity are
# checked for every argument first, then the device of every argument.

def _as_tensor(name, t):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    return t


def _check_layout(name, t, shape, dtype):
    _as_tensor(name, t)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_devices(ref_name, ref, named):
    if ref.device.type != "cuda":
        raise ValueError(f"{ref_name} must be on a GPU (cuda) device, got {ref.device}")
    for name, t in named:
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, expected {ref.device} (the device of {ref_name})")


def _check_bytes(name, t):
    """A byte buffer (workspace, saved states, packed weights): contiguous."""
    _as_tensor(name, t)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_attn(q, grid, like_q=(), caches=(), buffers=(), qname="q"):
    """q [B, H, T*Hs*Ws, d] (bf16 or fp32); like_q: (name, tensor) pairs
    with q's shape and dtype (None skipped); caches: (name, tensor, kind)
    with kind "S" [B, H, d, d] or "z" [B, H, d], fp32 (None skipped);
    buffers: (name, byte tensor) pairs (None skipped)."""
    import torch
    _as_tensor(qname, q)
    if q.dim() != 4:
        raise ValueError(f"{qname} must be [B, H, N, d], got shape {tuple(q.shape)}")
    _dtype_code(q)
    B, H, N, d = q.shape
    T, Hs, Ws = grid
    if N != T * Hs * Ws:
        raise ValueError(f"{qname} holds {N} tokens per sequence but the grid {T}x{Hs}x{Ws} has {T * Hs * Ws}")
    _check_layout(qname, q, None, None)
    for name, t in like_q:
        if t is not None:
            _check_layout(name, t, q.shape, q.dtype)
    for name, t, kind in caches:
        if t is not None:
            _check_layout(name, t, (B, H, d, d) if kind == "S" else (B, H, d), torch.float32)
    for name, t in buffers:
        if t is not None:
            _check_bytes(name, t)
    _check_devices(qname, q, [(n, t) for n, t in like_q] + [(n, t) for n, t, _ in caches] + list(buffers))


def _pair(name_a, a, name_b, b):
    if (a is None) != (b is None):
        raise ValueError(f"{name_a} and {name_b} must be given together")


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
    """The caller's workspace, or a new zero-filled one (a workspace must be
    zero-filled before its first use: its arrival counters start at zero, and
    every call leaves them zero again)."""
    import torch
    if ws is not None:
        return ws
    return torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=like.device)


def sva_lin_attn_fwd(q, k, v, grid: Tuple[int, int, int], frames_per_block: int, *, t0: int = 0,
                     rope: bool = False, split=None, base: float = 10000.0, eps: float = 1e-6,
                     S0=None, z0=None, out=None, S_out=None, z_out=None, ws=None, stream=None,
                     stages: int = 7):
    """One-shot block-causal forward (sva_lin_attn_fwd).  Returns `out`.
    stages (a mask of SVA_STAGE_*) restricts the call to some of its kernels
    (sva_lin_attn_fwd_stages), for timing them one at a time."""
    import torch
    _pair("S0", S0, "z0", z0)
    _pair("S_out", S_out, "z_out", z_out)
    _check_attn(q, grid, like_q=[("k", k), ("v", v), ("out", out)],
                caches=[("S0", S0, "S"), ("z0", z0, "z"), ("S_out", S_out, "S"), ("z_out", z_out, "z")],
                buffers=[("ws", ws)])
    desc = _desc_from(q, grid, frames_per_block, t0, rope, split, base, eps)
    if out is None:
        out = torch.empty_like(q)
    nbytes = sva_lin_attn_fwd_workspace(desc)
    ws = _workspace(nbytes, q, ws)
    args = (ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(S0), _ptr(z0), _ptr(S_out),
            _ptr(z_out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    if stages == SVA_STAGE_ALL:
        st = lib().sva_lin_attn_fwd(*args)
    else:
        st = lib().sva_lin_attn_fwd_stages(*args, int(stages))
    _check(st, "sva_lin_attn_fwd")
    return out


class PreparedCall:
    """One library call whose arguments were checked and marshalled once:
    calling it issues the C call alone (about a microsecond of host time,
    against tens for a call through the checking wrappers), for loops that
    repeat a call on the same buffers.  It keeps references to its tensors;
    their storage must not be resized or freed, and their contents may
    change between calls.  The stream is the one given at preparation, else
    the current stream at each call (so a call made under graph capture is
    captured).  Raises SvaError on a nonzero status."""

    __slots__ = ("_fn", "_args", "_stream", "_keep", "_where", "out")

    def __init__(self, fn_name, args, stream, keep, where, out=None):
        self._fn = getattr(lib(), fn_name)
        self._args = tuple(args)
        self._stream = None if stream is None else stream.cuda_stream
        self._keep = keep
        self._where = where
        self.out = out

    def __call__(self):
        st = self._fn(*self._args, self._stream if self._stream is not None else _stream(None))
        if st != SVA_OK:
            raise SvaError(st, self._where)
        return self.out


def prepare_lin_attn_fwd(q, k, v, grid: Tuple[int, int, int], frames_per_block: int, *, t0: int = 0,
                         rope: bool = False, split=None, base: float = 10000.0, eps: float = 1e-6,
                         S0=None, z0=None, out=None, S_out=None, z_out=None, ws=None, stream=None) -> PreparedCall:
    """sva_lin_attn_fwd with its checks done now: returns a PreparedCall
    whose calls run the forward on these buffers (out and the workspace
    are allocated here when not given, and kept)."""
    import torch
    _pair("S0", S0, "z0", z0)
    _pair("S_out", S_out, "z_out", z_out)
    _check_attn(q, grid, like_q=[("k", k), ("v", v), ("out", out)],
                caches=[("S0", S0, "S"), ("z0", z0, "z"), ("S_out", S_out, "S"), ("z_out", z_out, "z")],
                buffers=[("ws", ws)])
    desc = _desc_from(q, grid, frames_per_block, t0, rope, split, base, eps)
    if out is None:
        out = torch.empty_like(q)
    nbytes = sva_lin_attn_fwd_workspace(desc)
    if ws is not None and ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"ws holds {ws.numel() * ws.element_size()} bytes, the call needs {nbytes}")
    ws = _workspace(nbytes, q, ws)
    ptrs = [ctypes.c_void_p(_ptr(t)) for t in (q, k, v, out, S0, z0, S_out, z_out, ws)]
    args = [ctypes.byref(desc)] + ptrs[:9] + [ctypes.c_size_t(ws.numel() * ws.element_size())]
    return PreparedCall("sva_lin_attn_fwd", args, stream,
                        (desc, q, k, v, out, S0, z0, S_out, z_out, ws), "sva_lin_attn_fwd", out)


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
    _pair("S0", S0, "z0", z0)
    _pair("S_out", S_out, "z_out", z_out)
    _check_attn(q, grid, like_q=[("k", k), ("v", v), ("out", out)],
                caches=[("S0", S0, "S"), ("z0", z0, "z"), ("S_out", S_out, "S"), ("z_out", z_out, "z")],
                buffers=[("ws", ws), ("states", states)])
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


def sva_lin_attn_bwd(q, k, v, dout, grid: Tuple[int, int, int], frames_per_block: int, *, t0: int = 0,
                     rope: bool = False, split=None, base: float = 10000.0, eps: float = 1e-6,
                     S0=None, z0=None, dS_out=None, dz_out=None, states=None, dq=None, dk=None, dv=None,
                     dS0=None, dz0=None, ws=None, stream=None):
    """Gradients of the forward (sva_lin_attn_bwd), bf16.  Returns (dq, dk, dv);
    dS0/dz0 are filled when given.  `states` from sva_lin_attn_fwd_save
    skips recomputing the forward's prefix states.  The forward's output is
    not needed: the kernels form it again from q and the states."""
    import torch
    for na, ta, nb_, tb in (("S0", S0, "z0", z0), ("dS_out", dS_out, "dz_out", dz_out), ("dS0", dS0, "dz0", dz0)):
        _pair(na, ta, nb_, tb)
    if dout is None:
        raise ValueError("dout is required")
    _check_attn(q, grid, like_q=[("k", k), ("v", v), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)],
                caches=[("S0", S0, "S"), ("z0", z0, "z"), ("dS_out", dS_out, "S"), ("dz_out", dz_out, "z"),
                        ("dS0", dS0, "S"), ("dz0", dz0, "z")],
                buffers=[("ws", ws), ("states", states)])
    desc = _desc_from(q, grid, frames_per_block, t0, rope, split, base, eps)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    ws = _workspace(sva_lin_attn_bwd_workspace(desc), q, ws)
    st = lib().sva_lin_attn_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(dout),
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
    _check_attn(q, frame_grid, like_q=[("k", k), ("v", v), ("out", out)], caches=[("S", S, "S"), ("z", z, "z")],
                buffers=[("ws", ws)])
    if S is None or z is None:
        raise ValueError("the cache S, z is required")
    desc = _desc_from(q, frame_grid, frame_grid[0], t0, rope, split, base, eps)
    if out is None:
        out = torch.empty_like(q)
    ws = _workspace(sva_block_cache_workspace(desc), q, ws)
    st = lib().sva_block_cache_apply(ctypes.byref(desc), _ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "sva_block_cache_apply")
    return out


def sva_block_cache_apply_noalloc(S, z, q, k, v, frame_grid: Tuple[int, int, int], *, t0: int,
                                  rope: bool = False, split=None, base: float = 10000.0, eps: float = 1e-6,
                                  out, stream=None):
    """sva_block_cache_apply on the library's static scratch: nothing is
    allocated, `out` included (the caller passes it).  Calls on one GPU
    share the scratch and must not overlap."""
    _check_attn(q, frame_grid, like_q=[("k", k), ("v", v), ("out", out)], caches=[("S", S, "S"), ("z", z, "z")])
    if S is None or z is None or out is None:
        raise ValueError("the cache S, z and out are required")
    desc = _desc_from(q, frame_grid, frame_grid[0], t0, rope, split, base, eps)
    st = lib().sva_block_cache_apply_noalloc(ctypes.byref(desc), _ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v),
                                             _ptr(out), _stream(stream))
    _check(st, "sva_block_cache_apply_noalloc")
    return out


def sva_block_cache_commit(S, z, k, v, frame_grid: Tuple[int, int, int], *, t0: int, rope: bool = False,
                           split=None, base: float = 10000.0, ws=None, stream=None):
    """Adds one block's K, V to the cache (S, z) in place."""
    _check_attn(k, frame_grid, like_q=[("v", v)], caches=[("S", S, "S"), ("z", z, "z")], buffers=[("ws", ws)],
                qname="k")
    if S is None or z is None:
        raise ValueError("the cache S, z is required")
    desc = _desc_from(k, frame_grid, frame_grid[0], t0, rope, split, base, 0.0)
    ws = _workspace(sva_block_cache_workspace(desc), k, ws)
    st = lib().sva_block_cache_commit(ctypes.byref(desc), _ptr(S), _ptr(z), _ptr(k), _ptr(v), _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "sva_block_cache_commit")


def sva_phi_rope_prep(x, grid: Tuple[int, int, int], *, t0: int = 0, rope: bool = False, split=None,
                      base: float = 10000.0, want_phi: bool = True, stream=None):
    """The phi + RoPE stage alone: returns (RoPE(phi x), phi x) as fp32."""
    import torch
    _check_attn(x, grid, qname="x")
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


def _check_tconv(x, w=None, bias=None, caches=(), y=None):
    """x [B, T, Hs, Ws, C] (bf16 or fp32), taps w [C, 3] and bias [C] fp32,
    caches [B, Hs, Ws, C] in x's dtype, y like x (None skipped)."""
    import torch
    _as_tensor("x", x)
    if x.dim() != 5:
        raise ValueError(f"x must be [B, T, Hs, Ws, C], got shape {tuple(x.shape)}")
    _dtype_code(x)
    B, T, Hs, Ws, C = x.shape
    _check_layout("x", x, None, None)
    named = []
    if w is not None:
        _check_layout("w", w, (C, 3), torch.float32)
        named.append(("w", w))
    if bias is not None:
        _check_layout("bias", bias, (C,), torch.float32)
        named.append(("bias", bias))
    for name, t in caches:
        if t is not None:
            _check_layout(name, t, (B, Hs, Ws, C), x.dtype)
            named.append((name, t))
    if y is not None:
        _check_layout("y", y, x.shape, x.dtype)
        named.append(("y", y))
    _check_devices("x", x, named)


def sva_tconv_fwd(x, w, bias, frames_per_block: int, *, cache_in=None, y=None, cache_out=None,
                  stream=None):
    """Block-causal temporal convolution over all blocks of x [B, T, Hs, Ws, C]
    with taps w [C, 3] and bias [C] (fp32; bias may be None).  cache_in is the
    frame carried into block 0 (None: zero); cache_out, if given, receives the
    last frame.  Returns y."""
    import torch
    if w is None:
        raise ValueError("the taps w are required")
    _check_tconv(x, w, bias, [("cache_in", cache_in), ("cache_out", cache_out)], y)
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
    if w is None or cache is None:
        raise ValueError("the taps w and the cache are required")
    _check_tconv(x, w, bias, [("cache", cache)], y)
    desc = _tconv_desc_from(x, x.shape[1])
    if y is None:
        y = torch.empty_like(x)
    st = lib().sva_tconv_apply(ctypes.byref(desc), _ptr(cache), _ptr(x), _ptr(w), _ptr(bias), _ptr(y),
                               _stream(stream))
    _check(st, "sva_tconv_apply")
    return y


def sva_tconv_commit(cache, x, *, stream=None):
    """cache <- the last frame of one block x [B, F, Hs, Ws, C], in place."""
    if cache is None:
        raise ValueError("the cache is required")
    _check_tconv(x, caches=[("cache", cache)])
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
    _as_tensor("codes", codes)
    if codes.dim() != 2:
        raise ValueError(f"codes must be [3 H d, C / 2], got shape {tuple(codes.shape)}")
    n_out, half = codes.shape
    C = 2 * half
    if n_out != 3 * H * d:
        raise ValueError(f"codes has {n_out} rows, expected 3 H d = {3 * H * d}")
    if C % 32:
        raise ValueError(f"C = {C} is not a whole number of 32-channel scale blocks")
    _check_layout("codes", codes, None, torch.uint8)
    _check_layout("scales", scales, (n_out, C // 32), torch.uint8)
    if out is not None:
        _check_layout("out", out, (mxfp4_packed_bytes(n_out, C),), torch.uint8)
    _check_devices("codes", codes, [("scales", scales), ("out", out)])
    if out is None:
        out = torch.empty((mxfp4_packed_bytes(n_out, C),), dtype=torch.uint8, device=codes.device)
    desc = SvaProjDesc(1, 1, C, H, d, 0)
    st = lib().sva_mxfp4_pack_weights(ctypes.byref(desc), _ptr(codes), _ptr(scales), _ptr(out), _stream(stream))
    _check(st, "sva_mxfp4_pack_weights")
    return out


def _check_proj_inputs(x, wpack, bias, H, d):
    """x [B, N, C] bf16, wpack the packed weights for 3 H d outputs, bias
    [3 H d] fp32 or None (layouts only; devices are checked by the caller)."""
    import torch
    _as_tensor("x", x)
    if x.dim() != 3:
        raise ValueError(f"x must be [B, N, C], got shape {tuple(x.shape)}")
    _check_layout("x", x, None, torch.bfloat16)
    C = x.shape[2]
    n_out = 3 * H * d
    _check_bytes("wpack", wpack)
    if wpack.numel() * wpack.element_size() != mxfp4_packed_bytes(n_out, C):
        raise ValueError(f"wpack holds {wpack.numel() * wpack.element_size()} bytes, expected "
                         f"{mxfp4_packed_bytes(n_out, C)} for {n_out} outputs of C = {C}")
    if bias is not None:
        _check_layout("bias", bias, (n_out,), torch.float32)


def sva_qkv_proj_mxfp4(x, wpack, bias, H: int, d: int, *, q=None, k=None, v=None, stream=None):
    """x [B, N, C] bf16; wpack from sva_mxfp4_pack_weights; bias [3 H d]
    fp32 or None.  Returns (q, k, v), each [B, H, N, d] bf16."""
    import torch
    _check_proj_inputs(x, wpack, bias, H, d)
    B, N, C = x.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t is not None:
            _check_layout(name, t, (B, H, N, d), torch.bfloat16)
    _check_devices("x", x, [("wpack", wpack), ("bias", bias), ("q", q), ("k", k), ("v", v)])
    desc = SvaProjDesc(B, N, C, H, d, 0)
    outs = []
    for t in (q, k, v):
        outs.append(torch.empty((B, H, N, d), dtype=torch.bfloat16, device=x.device) if t is None else t)
    st = lib().sva_qkv_proj_mxfp4(ctypes.byref(desc), _ptr(x), _ptr(wpack), _ptr(bias),
                                  _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]), _stream(stream))
    _check(st, "sva_qkv_proj_mxfp4")
    return tuple(outs)


def mxfp4_acts_bytes(M: int, C: int) -> int:
    """Bytes of M token rows of C channels in MXFP4: codes then scales."""
    return M * C // 2 + M * C // 32


def sva_mxfp4_quant_acts(x, *, out=None, stream=None):
    """x [B, N, C] bf16 -> the MXFP4 activations (uint8 tensor of
    mxfp4_acts_bytes(B N, C) bytes: codes [B N, C / 2], then scales
    [B N, C / 32]) that sva_qkv_proj_w4a4 takes."""
    import torch
    _as_tensor("x", x)
    if x.dim() != 3:
        raise ValueError(f"x must be [B, N, C], got shape {tuple(x.shape)}")
    _check_layout("x", x, None, torch.bfloat16)
    B, N, C = x.shape
    nbytes = mxfp4_acts_bytes(B * N, C)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    else:
        _check_bytes("out", out)
        if out.numel() * out.element_size() != nbytes:
            raise ValueError(f"out holds {out.numel() * out.element_size()} bytes, expected {nbytes}")
    _check_devices("x", x, [("out", out)])
    desc = SvaProjDesc(B, N, C, 1, 64, 0)  # H, d do not enter the conversion
    st = lib().sva_mxfp4_quant_acts(ctypes.byref(desc), _ptr(x), _ptr(out), _stream(stream))
    _check(st, "sva_mxfp4_quant_acts")
    return out


def sva_qkv_proj_w4a4(xq, wpack, bias, B: int, N: int, C: int, H: int, d: int, *, q=None, k=None, v=None,
                      stream=None):
    """xq from sva_mxfp4_quant_acts of an x [B, N, C]; wpack from
    sva_mxfp4_pack_weights; bias [3 H d] fp32 or None.  Returns (q, k, v),
    each [B, H, N, d] bf16."""
    import torch
    _check_w4a4_inputs(xq, wpack, bias, B, N, C, H, d)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t is not None:
            _check_layout(name, t, (B, H, N, d), torch.bfloat16)
    _check_devices("xq", xq, [("wpack", wpack), ("bias", bias), ("q", q), ("k", k), ("v", v)])
    desc = SvaProjDesc(B, N, C, H, d, 0)
    outs = []
    for t in (q, k, v):
        outs.append(torch.empty((B, H, N, d), dtype=torch.bfloat16, device=xq.device) if t is None else t)
    st = lib().sva_qkv_proj_w4a4(ctypes.byref(desc), _ptr(xq), _ptr(wpack), _ptr(bias),
                                 _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]), _stream(stream))
    _check(st, "sva_qkv_proj_w4a4")
    return tuple(outs)


def _check_w4a4_inputs(xq, wpack, bias, B, N, C, H, d):
    """xq the MXFP4 activations of an x [B, N, C], wpack the packed weights
    for 3 H d outputs, bias [3 H d] fp32 or None (layouts only)."""
    import torch
    _check_bytes("xq", xq)
    if xq.numel() * xq.element_size() != mxfp4_acts_bytes(B * N, C):
        raise ValueError(f"xq holds {xq.numel() * xq.element_size()} bytes, expected "
                         f"{mxfp4_acts_bytes(B * N, C)} for {B * N} rows of C = {C}")
    n_out = 3 * H * d
    _check_bytes("wpack", wpack)
    if wpack.numel() * wpack.element_size() != mxfp4_packed_bytes(n_out, C):
        raise ValueError(f"wpack holds {wpack.numel() * wpack.element_size()} bytes, expected "
                         f"{mxfp4_packed_bytes(n_out, C)} for {n_out} outputs of C = {C}")
    if bias is not None:
        _check_layout("bias", bias, (n_out,), torch.float32)


def _proj_lin_attn(fn_name, xin, xname, wpack, bias, B, N, C, H, grid, frames_per_block, t0, rope, split, base,
                   eps, S0, z0, S_out, z_out, out, ws, stream, range_tokens):
    """The fused projection + attention calls' common part: the output and
    cache checks, the descriptors, the workspace and the call."""
    import torch
    _pair("S0", S0, "z0", z0)
    _pair("S_out", S_out, "z_out", z_out)
    T, Hs, Ws = grid
    if N != T * Hs * Ws:
        raise ValueError(f"{xname} holds {N} tokens per sample but the grid {T}x{Hs}x{Ws} has {T * Hs * Ws}")
    if out is not None:
        _check_layout("out", out, (B, H, N, 64), torch.bfloat16)
    for name, t, shape in (("S0", S0, (B, H, 64, 64)), ("z0", z0, (B, H, 64)), ("S_out", S_out, (B, H, 64, 64)),
                           ("z_out", z_out, (B, H, 64))):
        if t is not None:
            _check_layout(name, t, shape, torch.float32)
    if ws is not None:
        _check_bytes("ws", ws)
    _check_devices(xname, xin, [("wpack", wpack), ("bias", bias), ("out", out), ("S0", S0), ("z0", z0),
                                ("S_out", S_out), ("z_out", z_out), ("ws", ws)])
    q_like = torch.empty((B, H, N, 64), dtype=torch.bfloat16, device=xin.device) if out is None else out
    desc = _desc_from(q_like, grid, frames_per_block, t0, rope, split, base, eps)
    pdesc = SvaProjDesc(B, N, C, H, 64, int(range_tokens))
    n = ctypes.c_size_t()
    _check(lib().sva_proj_lin_attn_fwd_workspace(ctypes.byref(desc), ctypes.byref(pdesc), ctypes.byref(n)),
           "sva_proj_lin_attn_fwd_workspace")
    ws = _workspace(n.value, xin, ws)
    st = getattr(lib(), fn_name)(ctypes.byref(desc), ctypes.byref(pdesc), _ptr(xin), _ptr(wpack), _ptr(bias),
                                 _ptr(q_like), _ptr(S0), _ptr(z0), _ptr(S_out), _ptr(z_out), _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(stream))
    _check(st, fn_name)
    return q_like


def sva_proj_lin_attn_fwd(x, wpack, bias, H: int, grid: Tuple[int, int, int], frames_per_block: int, *,
                          t0: int = 0, rope: bool = False, split=None, base: float = 10000.0, eps: float = 1e-6,
                          S0=None, z0=None, S_out=None, z_out=None, out=None, ws=None, stream=None,
                          range_tokens: int = 0):
    """Projection and attention fused (sva_proj_lin_attn_fwd): x [B, N, C]
    bf16 with N = T * Hs * Ws; wpack from sva_mxfp4_pack_weights for H heads
    of d = 64; bias [3 H 64] fp32 or None.  range_tokens: tokens per
    reduction range (0: chosen by the library; else a divisor of the block
    length).  Returns out [B, H, N, 64] bf16."""
    _check_proj_inputs(x, wpack, bias, H, 64)
    B, N, C = x.shape
    return _proj_lin_attn("sva_proj_lin_attn_fwd", x, "x", wpack, bias, B, N, C, H, grid, frames_per_block, t0,
                          rope, split, base, eps, S0, z0, S_out, z_out, out, ws, stream, range_tokens)


def sva_proj_lin_attn_fwd_w4a4(xq, wpack, bias, B: int, C: int, H: int, grid: Tuple[int, int, int],
                               frames_per_block: int, *, t0: int = 0, rope: bool = False, split=None,
                               base: float = 10000.0, eps: float = 1e-6, S0=None, z0=None, S_out=None, z_out=None,
                               out=None, ws=None, stream=None, range_tokens: int = 0):
    """The same on 4-bit activations (sva_proj_lin_attn_fwd_w4a4): xq from
    sva_mxfp4_quant_acts of an x [B, N, C] with N = T * Hs * Ws; the rest as
    for sva_proj_lin_attn_fwd.  Returns out [B, H, N, 64] bf16."""
    T, Hs, Ws = grid
    N = T * Hs * Ws
    _check_w4a4_inputs(xq, wpack, bias, B, N, C, H, 64)
    return _proj_lin_attn("sva_proj_lin_attn_fwd_w4a4", xq, "xq", wpack, bias, B, N, C, H, grid, frames_per_block,
                          t0, rope, split, base, eps, S0, z0, S_out, z_out, out, ws, stream, range_tokens)
