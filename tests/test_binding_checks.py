"""The Python binding checks tensor arguments before it calls the library:
the C ABI receives bare pointers, so a wrong shape, dtype, layout or device
must raise here, and never reach a kernel.  CPU tensors only; the library is
replaced by a stub that fails the test if anything calls it."""
import pytest
import torch

from block_causal_linear_phi_amd import sva


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def forbidden():
        raise AssertionError("the library was called before the argument checks finished")
    monkeypatch.setattr(sva, "lib", forbidden)


GRID, F = (4, 3, 5), 2
N = GRID[0] * GRID[1] * GRID[2]


def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def _qkv(B=1, H=2, d=64, dtype=torch.bfloat16):
    return _t(B, H, N, d, dtype=dtype), _t(B, H, N, d, dtype=dtype), _t(B, H, N, d, dtype=dtype)


@pytest.mark.parametrize("entry", ["call", "prepare"])
def test_fwd_rejects_each_bad_argument(entry):
    """The forward, and its prepared form (checked once, at preparation)."""
    fwd = sva.sva_lin_attn_fwd if entry == "call" else sva.prepare_lin_attn_fwd
    q, k, v = _qkv()
    cases = [
        (dict(k=_t(1, 2, N + 1, 64)), "shape"),                       # k longer than q
        (dict(v=_t(1, 2, N, 64, dtype=torch.float32)), "dtype"),      # v fp32, q bf16
        (dict(k=_t(1, 2, 64, N).transpose(2, 3)), "contiguous"),      # a transposed view
        (dict(out=_t(1, 2, N, 32)), "shape"),
        (dict(q=_t(1, 2, N + 3, 64)), "tokens"),                      # N != T Hs Ws
        (dict(q=_t(2, N, 64)), r"\[B, H, N, d\]"),
        (dict(S0=_t(1, 2, 64, 64, dtype=torch.float32), z0=_t(1, 2, 64)), "dtype"),  # z0 bf16
        (dict(S0=_t(1, 2, 64, 63, dtype=torch.float32), z0=_t(1, 2, 64, dtype=torch.float32)), "shape"),
        (dict(S0=_t(1, 2, 64, 64, dtype=torch.float32)), "together"),  # S0 without z0
        (dict(ws=_t(64, 8, dtype=torch.uint8).t()), "contiguous"),
        (dict(), "GPU"),                                               # all fine, but on the CPU
    ]
    for kw, msg in cases:
        args = dict(q=q, k=k, v=v)
        args.update(kw)
        with pytest.raises(ValueError, match=msg):
            fwd(args.pop("q"), args.pop("k"), args.pop("v"), GRID, F, **args)


def test_fwd_rejects_unsupported_dtype_and_non_tensors():
    q, k, v = _qkv(dtype=torch.float16)
    with pytest.raises(TypeError):
        sva.sva_lin_attn_fwd(q, k, v, GRID, F)
    q, k, v = _qkv()
    with pytest.raises(TypeError):
        sva.sva_lin_attn_fwd(q, [1, 2], v, GRID, F)


def test_mixed_devices_are_rejected():
    q, k, v = _qkv()
    meta = torch.empty(q.shape, dtype=q.dtype, device="meta")
    with pytest.raises(ValueError, match="GPU|device"):
        sva.sva_lin_attn_fwd(q, meta, v, GRID, F)


def test_fwd_save_and_bwd_check_their_extra_arguments():
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="contiguous"):
        sva.sva_lin_attn_fwd_save(q, k, v, GRID, F, states=_t(64, 8, dtype=torch.uint8).t())
    good = _t(1, 2, N, 64)
    with pytest.raises(ValueError, match="shape"):
        sva.sva_lin_attn_bwd(q, k, v, _t(1, 2, N, 32), GRID, F)          # dout
    with pytest.raises(ValueError, match="dtype"):
        sva.sva_lin_attn_bwd(q, k, v, good, GRID, F, dq=_t(1, 2, N, 64, dtype=torch.float32))
    with pytest.raises(ValueError, match="together"):
        sva.sva_lin_attn_bwd(q, k, v, good, GRID, F, dS0=_t(1, 2, 64, 64, dtype=torch.float32))
    with pytest.raises(ValueError, match="GPU"):
        sva.sva_lin_attn_bwd(q, k, v, good, GRID, F)


def test_cache_calls_check_the_cache():
    fg = (F, GRID[1], GRID[2])
    n = F * GRID[1] * GRID[2]
    q, k, v = _t(1, 2, n, 64), _t(1, 2, n, 64), _t(1, 2, n, 64)
    S, z = _t(1, 2, 64, 64, dtype=torch.float32), _t(1, 2, 64, dtype=torch.float32)
    with pytest.raises(ValueError, match="shape"):
        sva.sva_block_cache_apply(S, _t(1, 2, 32, dtype=torch.float32), q, k, v, fg, t0=0)
    with pytest.raises(ValueError, match="dtype"):
        sva.sva_block_cache_apply(S.double(), z, q, k, v, fg, t0=0)
    with pytest.raises(ValueError, match="tokens"):
        sva.sva_block_cache_apply(S, z, q, k, v, (F + 1, GRID[1], GRID[2]), t0=0)
    with pytest.raises(ValueError, match="shape"):
        sva.sva_block_cache_commit(S, z, k, _t(1, 2, n, 32), fg, t0=0)
    with pytest.raises(ValueError, match="contiguous"):
        sva.sva_block_cache_commit(S.transpose(2, 3), z, k, v, fg, t0=0)
    with pytest.raises(ValueError, match="GPU"):
        sva.sva_block_cache_commit(S, z, k, v, fg, t0=0)


def test_tconv_checks():
    x = _t(1, 6, 3, 5, 16)
    w = _t(16, 3, dtype=torch.float32)
    with pytest.raises(ValueError, match="shape"):
        sva.sva_tconv_fwd(x, _t(16, 2, dtype=torch.float32), None, 3)
    with pytest.raises(ValueError, match="dtype"):
        sva.sva_tconv_fwd(x, w, _t(16), 3)                                   # bf16 bias
    with pytest.raises(ValueError, match="shape"):
        sva.sva_tconv_fwd(x, w, None, 3, cache_in=_t(1, 3, 5, 8))
    with pytest.raises(ValueError, match="contiguous"):
        sva.sva_tconv_fwd(x.transpose(2, 3).contiguous().transpose(2, 3), w, None, 3)
    with pytest.raises(ValueError, match="shape"):
        sva.sva_tconv_apply(_t(1, 3, 5, 16), x[:, :3], w, None, y=_t(1, 3, 3, 5, 8))
    with pytest.raises(ValueError, match="shape"):
        sva.sva_tconv_commit(_t(1, 3, 4, 16), x[:, :3].contiguous())
    with pytest.raises(ValueError, match="GPU"):
        sva.sva_tconv_fwd(x, w, None, 3)


def test_projection_checks():
    H, d, C = 2, 64, 256
    x = _t(1, N, C)
    wp = _t(sva.mxfp4_packed_bytes(3 * H * d, C), dtype=torch.uint8)
    with pytest.raises(ValueError, match="bytes"):
        sva.sva_qkv_proj_mxfp4(x, wp[:-16], None, H, d)
    with pytest.raises(ValueError, match="dtype"):
        sva.sva_qkv_proj_mxfp4(x.float(), wp, None, H, d)
    with pytest.raises(ValueError, match="shape"):
        sva.sva_qkv_proj_mxfp4(x, wp, _t(3 * H * d + 1, dtype=torch.float32), H, d)
    with pytest.raises(ValueError, match="shape"):
        sva.sva_qkv_proj_mxfp4(x, wp, None, H, d, k=_t(1, H, N + 1, d))
    with pytest.raises(ValueError, match="GPU"):
        sva.sva_qkv_proj_mxfp4(x, wp, None, H, d)
    codes = _t(3 * H * d, C // 2, dtype=torch.uint8)
    with pytest.raises(ValueError, match="shape"):
        sva.sva_mxfp4_pack_weights(codes, _t(3 * H * d, C // 16, dtype=torch.uint8), H, d)
    with pytest.raises(ValueError, match="rows"):
        sva.sva_mxfp4_pack_weights(codes[:-1], _t(3 * H * d - 1, C // 32, dtype=torch.uint8), H, d)
    with pytest.raises(ValueError, match="tokens"):
        sva.sva_proj_lin_attn_fwd(x, wp, None, H, (GRID[0] + 2, GRID[1], GRID[2]), F)
    with pytest.raises(ValueError, match="shape"):
        sva.sva_proj_lin_attn_fwd(x, wp, None, H, GRID, F, S0=_t(1, H, 64, 64, dtype=torch.float32),
                                  z0=_t(1, H, 63, dtype=torch.float32))
    with pytest.raises(ValueError, match="GPU"):
        sva.sva_proj_lin_attn_fwd(x, wp, None, H, GRID, F)


def test_w4a4_checks():
    H, d, C = 2, 64, 256
    xq = _t(sva.mxfp4_acts_bytes(N, C), dtype=torch.uint8)
    wp = _t(sva.mxfp4_packed_bytes(3 * H * d, C), dtype=torch.uint8)
    with pytest.raises(ValueError, match="bytes"):
        sva.sva_qkv_proj_w4a4(xq[:-1], wp, None, 1, N, C, H, d)
    with pytest.raises(ValueError, match="bytes"):
        sva.sva_qkv_proj_w4a4(xq, wp[:-16], None, 1, N, C, H, d)
    with pytest.raises(ValueError, match="bytes"):
        # the grid holds more tokens than xq's rows
        sva.sva_proj_lin_attn_fwd_w4a4(xq, wp, None, 1, C, H, (GRID[0] + 2, GRID[1], GRID[2]), F)
    with pytest.raises(ValueError, match="shape"):
        sva.sva_proj_lin_attn_fwd_w4a4(xq, wp, _t(3 * H * d - 1, dtype=torch.float32), 1, C, H, GRID, F)
    with pytest.raises(ValueError, match="shape"):
        sva.sva_proj_lin_attn_fwd_w4a4(xq, wp, None, 1, C, H, GRID, F, out=_t(1, H, N, 32))
    with pytest.raises(ValueError, match="GPU"):
        sva.sva_proj_lin_attn_fwd_w4a4(xq, wp, None, 1, C, H, GRID, F)
