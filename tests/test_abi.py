"""The C-ABI library on the CPU: it loads, exports every function that
include/*.h declares, sizes its workspaces as documented, and rejects bad
descriptors before launching anything (no GPU is touched by these calls)."""
import ctypes
import os
import re

import pytest

from block_causal_linear_phi_amd import sva

# The checks below hand the library fake device addresses that validation must
# reject before any launch.  They run only where no GPU is reachable, so a
# validation bug can never turn into a launch on those addresses.
try:
    import torch
    _GPU_VISIBLE = torch.cuda.device_count() > 0
except Exception:  # pragma: no cover
    _GPU_VISIBLE = False
fake_pointers = pytest.mark.skipif(_GPU_VISIBLE, reason="fake device pointers; host-only check")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(os.path.join(ROOT, "include", n) for n in os.listdir(os.path.join(ROOT, "include"))
                 if n.endswith(".h"))


def _header_text():
    return "\n".join(open(h).read() for h in HEADERS)


def _declared_functions():
    text = _header_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sva_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert len(names) >= 9
    lib = ctypes.CDLL(sva.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(sva._SIG), "binding and header disagree"


def test_version_and_status_strings():
    assert sva.lib().sva_version() == 1
    for code in (0, -1, -2, -3, -4):
        assert sva.status_string(code)
    assert sva.status_string(-99) == "unknown status"


def _desc(**kw):
    base = dict(B=1, H=16, d=64, grid=(21, 45, 80), frames_per_block=3, rope=True,
                split=(16, 24, 24), dtype=sva.SVA_BF16)
    base.update(kw)
    grid = base.pop("grid")
    F = base.pop("frames_per_block")
    return sva.make_desc(base.pop("B"), base.pop("H"), base.pop("d"), grid, F, **base)


def test_cache_workspace_is_independent_of_stream_length():
    """[talk] constant memory: the one-block apply/commit workspace and the
    cache never depend on how many blocks came before (t0)."""
    sizes = {sva.sva_block_cache_workspace(_desc(grid=(3, 30, 52), t0=t0)) for t0 in (0, 3, 90, 237)}
    assert len(sizes) == 1


def test_fwd_workspace_is_small_relative_to_inputs():
    n = sva.sva_lin_attn_fwd_workspace(_desc())
    traffic = 4 * 16 * 75600 * 64 * 2          # q, k, v read + out written, bf16
    assert 0 < n < 0.05 * traffic


BAD = [
    (dict(d=48), sva.SVA_ERR_UNSUPPORTED),
    (dict(dtype=7), sva.SVA_ERR_UNSUPPORTED),
    (dict(split=(16, 24, 22)), sva.SVA_ERR_UNSUPPORTED),
    (dict(split=(15, 25, 24)), sva.SVA_ERR_UNSUPPORTED),
    (dict(base=-1.0), sva.SVA_ERR_UNSUPPORTED),
    (dict(frames_per_block=4), sva.SVA_ERR_INVALID_ARG),   # 21 % 4 != 0
    (dict(B=0), sva.SVA_ERR_INVALID_ARG),
    (dict(eps=-1.0), sva.SVA_ERR_INVALID_ARG),
    (dict(t0=-3), sva.SVA_ERR_INVALID_ARG),
    (dict(grid=(240, 400, 400)), sva.SVA_ERR_UNSUPPORTED),  # RoPE table too large
    # small table, but h does not fit the 10-bit packed coordinate
    (dict(grid=(21, 1025, 4), split=(2, 2, 60)), sva.SVA_ERR_UNSUPPORTED),
]


@fake_pointers
@pytest.mark.parametrize("kw,code", BAD)
def test_bad_descriptors_are_rejected(kw, code):
    d = _desc(**kw)
    n = ctypes.c_size_t(123)
    assert sva.lib().sva_lin_attn_fwd_workspace(ctypes.byref(d), ctypes.byref(n)) == code
    assert n.value == 123  # nothing written on error
    # the compute entry points validate before touching any pointer or the GPU
    st = sva.lib().sva_lin_attn_fwd(ctypes.byref(d), 16, 16, 16, 4096, None, None, None, None, 16, 1 << 40, None)
    assert st == code


@fake_pointers
def test_pointer_checks_happen_before_launch():
    d = _desc()
    lib = sva.lib()
    big = 1 << 40
    # null q
    assert lib.sva_lin_attn_fwd(ctypes.byref(d), None, 16, 32, 1 << 36, None, None, None, None, 16, big, None) \
        == sva.SVA_ERR_INVALID_ARG
    # misaligned k
    assert lib.sva_lin_attn_fwd(ctypes.byref(d), 16, 24, 1 << 33, 1 << 36, None, None, None, None, 16, big, None) \
        == sva.SVA_ERR_INVALID_ARG
    # out overlapping q
    assert lib.sva_lin_attn_fwd(ctypes.byref(d), 1 << 30, 1 << 33, 1 << 34, (1 << 30) + 4096, None, None, None,
                                None, 16, big, None) == sva.SVA_ERR_INVALID_ARG
    # only one of S0/z0
    assert lib.sva_lin_attn_fwd(ctypes.byref(d), 1 << 30, 1 << 33, 1 << 34, 1 << 36, 1 << 20, None, None,
                                None, 16, big, None) == sva.SVA_ERR_INVALID_ARG
    # workspace too small
    assert lib.sva_lin_attn_fwd(ctypes.byref(d), 1 << 30, 1 << 33, 1 << 34, 1 << 36, None, None, None, None,
                                16, 64, None) == sva.SVA_ERR_WORKSPACE
    # apply/commit need exactly one block
    assert lib.sva_block_cache_apply(ctypes.byref(d), 16, 32, 1 << 30, 1 << 33, 1 << 34, 1 << 36, 16, big,
                                     None) == sva.SVA_ERR_INVALID_ARG
    assert lib.sva_block_cache_commit(ctypes.byref(d), 16, 32, 1 << 30, 1 << 33, 16, big, None) \
        == sva.SVA_ERR_INVALID_ARG


@fake_pointers
@pytest.mark.parametrize("stages", [0, 8, -1])
def test_stages_mask_is_checked(stages):
    d = _desc()
    st = sva.lib().sva_lin_attn_fwd_stages(ctypes.byref(d), 1 << 30, 1 << 33, 1 << 34, 1 << 36, None, None,
                                           None, None, 16, 1 << 40, None, stages)
    assert st == sva.SVA_ERR_INVALID_ARG


def test_workspace_starts_with_the_counters():
    """The forward's workspace grows by the B*H arrival counters (one 256-byte
    aligned region) over its partials and prefix states."""
    d = _desc()
    n = sva.sva_lin_attn_fwd_workspace(d)
    E, nb, BH = 64 * 64 + 64, 7, 16
    assert n >= 256 + (BH * nb) * E * 4 + BH * nb * (64 * 64 * 2 + 64 * 4)


def test_bwd_workspace_and_dtype():
    assert sva.sva_lin_attn_bwd_workspace(_desc()) == sva.sva_lin_attn_fwd_workspace(_desc())
    n = ctypes.c_size_t(5)
    d = _desc(dtype=sva.SVA_F32)
    assert sva.lib().sva_lin_attn_bwd_workspace(ctypes.byref(d), ctypes.byref(n)) == sva.SVA_ERR_UNSUPPORTED
    assert n.value == 5


@fake_pointers
@pytest.mark.parametrize("kw,code", BAD + [(dict(dtype=sva.SVA_F32), sva.SVA_ERR_UNSUPPORTED)])
def test_bwd_bad_descriptors_are_rejected(kw, code):
    d = _desc(**kw)
    big = 1 << 36  # fake, widely spaced device addresses; nothing is touched
    ptrs = [big * (i + 1) for i in range(8)]
    st = sva.lib().sva_lin_attn_bwd(ctypes.byref(d), ptrs[0], ptrs[1], ptrs[2], ptrs[3], None, None,
                                    None, None, None, ptrs[5], ptrs[6], ptrs[7], None, None, 16, 1 << 40, None)
    assert st == code


@fake_pointers
def test_bwd_pointer_checks_happen_before_launch():
    d = _desc()
    big = 1 << 36
    p = [big * (i + 1) for i in range(8)]
    lib = sva.lib()
    # arguments after `d`, with states (NULL) inserted after dz_out
    call = lambda *a: lib.sva_lin_attn_bwd(ctypes.byref(d), *a[:8], None, *a[8:])
    # a gradient buffer overlapping an input
    assert call(p[0], p[1], p[2], p[3], None, None, None, None, p[0], p[6], p[7], None, None, 16,
                1 << 40, None) == sva.SVA_ERR_INVALID_ARG
    # two gradient buffers overlapping each other
    assert call(p[0], p[1], p[2], p[3], None, None, None, None, p[5], p[5] + 64, p[7], None, None, 16,
                1 << 40, None) == sva.SVA_ERR_INVALID_ARG
    # dS0 without dz0
    assert call(p[0], p[1], p[2], p[3], None, None, None, None, p[5], p[6], p[7], 4096, None, 16,
                1 << 40, None) == sva.SVA_ERR_INVALID_ARG
    # missing dout
    assert call(p[0], p[1], p[2], None, None, None, None, None, p[5], p[6], p[7], None, None, 16,
                1 << 40, None) == sva.SVA_ERR_INVALID_ARG
    # workspace too small
    assert call(p[0], p[1], p[2], p[3], None, None, None, None, p[5], p[6], p[7], None, None, 16,
                16, None) == sva.SVA_ERR_WORKSPACE


def _declared_arg_counts():
    """Parameter count of every function declared in the header."""
    text = re.sub(r"/\*.*?\*/", "", _header_text(), flags=re.S)
    out = {}
    for name, params in re.findall(r"\b(sva_[a-z0-9_]+)\s*\(([^)]*)\)\s*;", text):
        params = params.strip()
        out[name] = 0 if params in ("", "void") else params.count(",") + 1
    return out


def test_binding_signatures_match_the_header():
    """Every ctypes signature in the binding has the header's argument count,
    so no argument is dropped or converted by ctypes' defaults."""
    counts = _declared_arg_counts()
    assert set(counts) == set(sva._SIG)
    for name, (_, argtypes) in sva._SIG.items():
        assert len(argtypes) == counts[name], name


def test_states_bytes():
    n = sva.sva_lin_attn_states_bytes(_desc())
    d, nb, BH = 64, 7, 16
    # bf16: the operands S_c^T, their bf16 remainders, and Z_c
    exact = BH * nb * (2 * d * d * 2 + d * 4)
    assert exact <= n <= exact + 768


@fake_pointers
def test_fwd_save_needs_states():
    d = _desc()
    st = sva.lib().sva_lin_attn_fwd_save(ctypes.byref(d), 1 << 36, 2 << 36, 3 << 36, 4 << 36, None, None, None,
                                         None, None, 16, 1 << 40, None)
    assert st == sva.SVA_ERR_INVALID_ARG


# Causal temporal convolution (include/sva_tconv.h)

def _tdesc(**kw):
    base = dict(B=1, T=21, Hs=45, Ws=80, C=1024, frames_per_block=3, dtype=sva.SVA_BF16)
    base.update(kw)
    return sva.make_tconv_desc(**base)


TCONV_BAD = [
    (dict(dtype=7), sva.SVA_ERR_UNSUPPORTED),
    (dict(C=12), sva.SVA_ERR_UNSUPPORTED),          # bf16 needs whole 8-channel vectors
    (dict(C=6, dtype=sva.SVA_F32), sva.SVA_ERR_UNSUPPORTED),
    (dict(T=20), sva.SVA_ERR_INVALID_ARG),          # not a whole number of blocks
    (dict(frames_per_block=0), sva.SVA_ERR_INVALID_ARG),
    (dict(B=0), sva.SVA_ERR_INVALID_ARG),
    (dict(Hs=0), sva.SVA_ERR_INVALID_ARG),
    (dict(C=0), sva.SVA_ERR_INVALID_ARG),
]


@fake_pointers
@pytest.mark.parametrize("kw,code", TCONV_BAD)
def test_tconv_bad_descriptors_are_rejected(kw, code):
    d = _tdesc(**kw)
    lib = sva.lib()
    assert lib.sva_tconv_fwd(ctypes.byref(d), 1 << 30, 16, None, None, 1 << 36, None, None) == code
    assert lib.sva_tconv_commit(ctypes.byref(d), 16, 1 << 30, None) in (code, sva.SVA_ERR_INVALID_ARG)


@fake_pointers
def test_tconv_pointer_checks_happen_before_launch():
    d = _tdesc()
    lib = sva.lib()
    X, Y, W, CI, CO = 1 << 30, 1 << 36, 16, 1 << 20, 1 << 24
    inv = sva.SVA_ERR_INVALID_ARG
    assert lib.sva_tconv_fwd(ctypes.byref(d), None, W, None, None, Y, None, None) == inv   # null x
    assert lib.sva_tconv_fwd(ctypes.byref(d), X, None, None, None, Y, None, None) == inv   # null w
    assert lib.sva_tconv_fwd(ctypes.byref(d), X, W, None, None, None, None, None) == inv   # null y
    assert lib.sva_tconv_fwd(ctypes.byref(d), X + 8, W, None, None, Y, None, None) == inv  # misaligned x
    assert lib.sva_tconv_fwd(ctypes.byref(d), X, W + 4, None, None, Y, None, None) == inv  # misaligned w
    assert lib.sva_tconv_fwd(ctypes.byref(d), X, W, W + 8, None, Y, None, None) == inv     # misaligned bias
    assert lib.sva_tconv_fwd(ctypes.byref(d), X, W, None, None, X + 4096, None, None) == inv  # y over x
    assert lib.sva_tconv_fwd(ctypes.byref(d), X, W, None, X + 4096, Y, None, None) == inv     # cache_in in x
    assert lib.sva_tconv_fwd(ctypes.byref(d), X, W, None, None, Y, Y + 4096, None) == inv     # cache_out in y
    assert lib.sva_tconv_fwd(ctypes.byref(d), X, W, None, CI, Y, CI + 4096, None) == inv      # partial alias
    # apply and commit take exactly one block, and apply needs its cache
    assert lib.sva_tconv_apply(ctypes.byref(d), CI, X, W, None, Y, None) == inv
    one = _tdesc(T=3)
    assert lib.sva_tconv_apply(ctypes.byref(one), None, X, W, None, Y, None) == inv
    assert lib.sva_tconv_commit(ctypes.byref(d), CO, X, None) == inv
    assert lib.sva_tconv_commit(ctypes.byref(one), X + 4096, X, None) == inv  # cache inside x
    assert lib.sva_tconv_commit(ctypes.byref(one), None, X, None) == inv


# QKV projection (include/sva_proj.h)

@fake_pointers
def test_proj_checks_happen_before_launch():
    lib = sva.lib()
    inv, uns = sva.SVA_ERR_INVALID_ARG, sva.SVA_ERR_UNSUPPORTED
    X, W, Q, K, V = 1 << 30, 1 << 20, 1 << 34, 1 << 35, 1 << 36

    def call(**kw):
        base = dict(B=1, N=75600, C=1024, H=16, d=64)
        base.update(kw)
        dsc = sva.SvaProjDesc(base["B"], base["N"], base["C"], base["H"], base["d"])
        return lambda *p: lib.sva_qkv_proj_mxfp4(ctypes.byref(dsc), *p, None)

    assert call(C=96)(X, W, None, Q, K, V) == uns        # C not a multiple of 128
    assert call(C=192)(X, W, None, Q, K, V) == uns
    assert call(H=1, d=32)(X, W, None, Q, K, V) == uns   # H d not a multiple of 64
    assert call(d=36, H=32)(X, W, None, Q, K, V) == uns  # d not a multiple of 8
    assert call(N=0)(X, W, None, Q, K, V) == inv
    ok = call()
    assert ok(None, W, None, Q, K, V) == inv            # null x
    assert ok(X, None, None, Q, K, V) == inv            # null weights
    assert ok(X, W, None, Q, None, V) == inv            # null k
    assert ok(X + 8, W, None, Q, K, V) == inv           # misaligned x
    assert ok(X, W + 8, None, Q, K, V) == inv           # misaligned weights
    assert ok(X, W, 8, Q, K, V) == inv                  # misaligned bias
    assert ok(X, W, None, X + 4096, K, V) == inv        # q over x
    assert ok(X, W, None, W + 4096, K, V) == inv        # q over the weights
    assert ok(X, W, None, Q, Q + 4096, V) == inv        # k over q


@fake_pointers
def test_pack_checks_happen_before_launch():
    lib = sva.lib()
    inv, uns = sva.SVA_ERR_INVALID_ARG, sva.SVA_ERR_UNSUPPORTED
    Cd, S, P = 1 << 30, 1 << 31, 1 << 32

    def call(**kw):
        base = dict(B=1, N=1, C=1024, H=16, d=64)
        base.update(kw)
        dsc = sva.SvaProjDesc(base["B"], base["N"], base["C"], base["H"], base["d"])
        return lambda *p: lib.sva_mxfp4_pack_weights(ctypes.byref(dsc), *p, None)

    assert call(C=64)(Cd, S, P) == uns                   # C not a multiple of 128
    assert call(H=1, d=32)(Cd, S, P) == uns              # H d not a multiple of 64
    ok = call()
    assert ok(None, S, P) == inv
    assert ok(Cd, None, P) == inv
    assert ok(Cd, S, None) == inv
    assert ok(Cd + 4, S, P) == inv                       # misaligned codes
    assert ok(Cd, S, P + 8) == inv                       # misaligned output
    assert ok(Cd, S, Cd + 4096) == inv                   # output over the codes
    assert ok(Cd, S, S - 4096) == inv                    # output over the scales

def test_fused_workspace_checks(monkeypatch):
    """The fused projection + attention takes an even number of 128-channel
    stages and an explicit range length only where it divides the block; the
    environment does not change the plan."""
    lib = sva.lib()
    grid, F = (21, 45, 80), 3
    fdesc = sva.make_desc(1, 16, 64, grid, F, dtype=sva.SVA_BF16, rope=True, split=(16, 24, 24))

    def query(C, range_tokens=0):
        n = ctypes.c_size_t()
        pdesc = sva.SvaProjDesc(1, 21 * 45 * 80, C, 16, 64, range_tokens)
        return lib.sva_proj_lin_attn_fwd_workspace(ctypes.byref(fdesc), ctypes.byref(pdesc), ctypes.byref(n)), n.value

    st, auto_bytes = query(1024)
    assert st == sva.SVA_OK and auto_bytes > 0
    assert query(384)[0] == sva.SVA_ERR_UNSUPPORTED   # three stages
    assert query(128)[0] == sva.SVA_ERR_UNSUPPORTED
    st, long_bytes = query(1024, 1800)                # divides 3 * 45 * 80
    assert st == sva.SVA_OK and long_bytes < auto_bytes  # fewer partials
    assert query(1024, 1000)[0] == sva.SVA_ERR_INVALID_ARG
    assert query(1024, -5)[0] == sva.SVA_ERR_INVALID_ARG
    monkeypatch.setenv("SVA_PROJ_RANGE_TOKENS", "1800")  # an old override: no effect
    assert query(1024) == (sva.SVA_OK, auto_bytes)


@fake_pointers
def test_fused_pointer_checks_happen_before_launch():
    """The fused projection + attention validates every pointer, the
    workspace and the overlaps before any launch (fake device addresses)."""
    lib = sva.lib()
    grid, F, H, C = (21, 45, 80), 3, 16, 1024
    N = grid[0] * grid[1] * grid[2]
    fdesc = sva.make_desc(1, H, 64, grid, F, dtype=sva.SVA_BF16, rope=True, split=(16, 24, 24))
    pdesc = sva.SvaProjDesc(1, N, C, H, 64)
    n = ctypes.c_size_t()
    assert lib.sva_proj_lin_attn_fwd_workspace(ctypes.byref(fdesc), ctypes.byref(pdesc), ctypes.byref(n)) == sva.SVA_OK
    X, W, O, WS = 1 << 36, 1 << 37, 1 << 38, 1 << 39   # x, packed weights, out, workspace
    inv = sva.SVA_ERR_INVALID_ARG

    def call(x=X, w=W, out=O, ws=WS, ws_bytes=None, bias=None, S=None, z=None):
        return lib.sva_proj_lin_attn_fwd(ctypes.byref(fdesc), ctypes.byref(pdesc), x, w, bias, out, None, None,
                                         S, z, ws, n.value if ws_bytes is None else ws_bytes, None)

    assert call(x=None) == inv
    assert call(w=None) == inv
    assert call(out=None) == inv
    assert call(x=X + 8) == inv                              # misaligned
    assert call(bias=8) == inv
    assert call(S=1 << 40, z=None) == inv                    # S_out without z_out
    assert call(ws=None) == sva.SVA_ERR_WORKSPACE
    assert call(ws_bytes=n.value - 16) == sva.SVA_ERR_WORKSPACE
    assert call(out=X + 4096) == inv                         # out over x
    assert call(out=W + 4096) == inv                         # out over the weights
    assert call(ws=X + 4096) == inv                          # workspace over x
    assert call(ws=W + 4096) == inv                          # workspace over the weights
    assert call(ws=O + 4096) == inv                          # workspace over out
    assert call(S=WS + 4096, z=1 << 41) == inv               # cache over the workspace
