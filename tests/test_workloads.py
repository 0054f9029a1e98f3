"""The seeded input generator: determinism, shapes, bf16 rounding."""
import numpy as np
import torch

from circulant_softmax_attention_amd import workloads as W


def test_table_shapes():
    t = W.WORKLOADS
    assert t[W.HEADLINE].N == 1024 and t[W.HEADLINE].D == 768 and t[W.HEADLINE].H == 12
    for wl in t.values():
        assert wl.D % wl.H == 0
        if wl.kind == "2d":
            assert wl.N == wl.Hg * wl.Wg


def test_inputs_are_deterministic_and_shaped():
    wl = W.WORKLOADS["cat1d_tiny_n64"]
    a, b = W.make_inputs(wl), W.make_inputs(wl)
    for k, v in a.arrays().items():
        np.testing.assert_array_equal(v, b.arrays()[k])
    assert a.X.shape == (1, 64, 64) and a.W_A.shape == (64, 4) and a.W_V.shape == (64, 64)
    assert a.X.dtype == np.float32


def test_bf16_rounding_matches_torch_rne():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 10
    # include exact ties (low 16 bits == 0x8000) in both parities
    ties = (np.arange(64, dtype=np.uint32) << 16 | 0x8000).astype(np.uint32) + np.uint32(0x3F800000)
    x = np.concatenate([x, ties.view(np.float32)])
    ours = W.round_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(W.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_bf16_workload_values_are_bf16_exact():
    wl = W.WORKLOADS["cat1d_clipL_n256_bf16"].with_(B=1)
    inp = W.make_inputs(wl, batch=1)
    for name, arr in inp.arrays().items():
        np.testing.assert_array_equal(W.bf16_bits_to_f32(inp.bits[name]), arr)
