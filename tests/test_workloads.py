"""The seeded input generator: determinism and the bf16 rounding it applies."""
import numpy as np
import torch

from sequence_chunked_exact_amd import workloads as W


def test_bf16_rounding_matches_torch_cast():
    x = np.random.default_rng(0).standard_normal(100000) * np.logspace(-30, 30, 100000)
    x = np.concatenate([x, [0.0, -0.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9]])
    bits = W.round_to_bf16_bits(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(bits.view(np.int16), ref)
    back = W.bf16_bits_to_f64(bits)
    assert np.array_equal(back, torch.from_numpy(ref).view(torch.bfloat16).double().numpy())


def test_inputs_deterministic_and_shaped():
    wl = W.WORKLOADS["tiny"]
    a, b = W.make_inputs(wl), W.make_inputs(wl)
    for n in ("q", "k", "v", "do"):
        assert np.array_equal(a.raw[n], b.raw[n])
    assert a.raw["q"].shape == (1, 4, 512, 64) and a.raw["k"].shape == (1, 4, 512, 64)
    assert a.raw["q"].dtype == np.float32
    assert abs(a.f64["q"].std() * 8 - 1) < 0.02


def test_spike_makes_logits_peaky():
    wl = W.WORKLOADS["8b_layer"]
    inp = W.make_inputs(wl, seq_len=256)
    q, k = inp.f64["q"][0, 0], inp.f64["k"][0, 0]
    assert 2.0 < (q @ k.T).std() < 4.0          # ~3 with the rank-4 amplitude-3 spike
    plain = W.make_inputs(W.WORKLOADS["4b_layer"], seq_len=256)
    assert (plain.f64["q"][0, 0] @ plain.f64["k"][0, 0].T).std() < 0.2


def test_chunk_bounds():
    wl = W.WORKLOADS["4b_layer"]
    assert wl.n_chunks == 17 and wl.chunk_bounds(16) == (8000, 192)
    assert W.WORKLOADS["sparse_64k"].n_chunks == 64
