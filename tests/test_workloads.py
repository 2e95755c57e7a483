"""The seeded input generator: reproducible, bf16 rounding is RNE (checked
against torch's own float32 -> bfloat16 conversion), and shapes match the
workload table."""
import numpy as np
import torch

from block_causal_linear_phi_amd import workloads as wl


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 7,
                        np.array([0.0, -0.0, 1.0, -1.0, 1.00390625, 1.005859375, 3.3e38, 1e-40],
                                 dtype=np.float32)])
    ours = wl.round_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_slices_are_reproducible_and_distinct():
    w = wl.WORKLOADS["480p"]
    a, _ = wl.slice_qkv(w, "q", 0, 3, n_tokens=1000)
    b, _ = wl.slice_qkv(w, "q", 0, 3, n_tokens=1000)
    c, _ = wl.slice_qkv(w, "k", 0, 3, n_tokens=1000)
    np.testing.assert_array_equal(a, b)
    assert not np.array_equal(a, c)


def test_k_scale_and_shapes():
    w = wl.WORKLOADS["720p"]
    assert (w.N, w.nb, w.block_tokens) == (75600, 7, 10800)
    k, _ = wl.slice_qkv(w, "k", 0, 0, n_tokens=20000)
    assert 0.45 < k.std() < 0.55
    assert wl.WORKLOADS["minute"].nb == 80 and wl.WORKLOADS["minute"].N == 374400
    assert wl.WORKLOADS["480p"].N == 32760
