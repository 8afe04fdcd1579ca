"""The seeded input generators: bf16 rounding, code-byte structure, lengths."""
import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    g = np.random.Generator(np.random.PCG64(0))
    a = np.concatenate([g.standard_normal(100_000).astype(np.float32),
                        np.array([1.0, -2.5, 3.0e-3, 65504.0, 1.00390625, 1.01171875], np.float32)])
    bits = synth.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    back = synth.bf16_bits_to_f32(bits)
    assert np.array_equal(back, torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_seeds_are_reproducible_and_distinct():
    a = synth.normal_bf16(synth.rng(1, 3, synth.T_Q), (4, 5))
    b = synth.normal_bf16(synth.rng(1, 3, synth.T_Q), (4, 5))
    c = synth.normal_bf16(synth.rng(1, 4, synth.T_Q), (4, 5))
    assert np.array_equal(a, b) and not np.array_equal(a, c)


def test_uniform_code_bytes():
    g = synth.rng(9, 0, synth.T_CODES)
    even = synth.uniform_code_bytes(g, (2, 5000), 64)
    assert even.shape == (2, 5000, 32)
    lo, hi = even & 0xF, even >> 4
    for nib in (lo, hi):
        counts = np.bincount(nib.ravel(), minlength=16)
        assert counts.min() > 0.9 * nib.size / 16
    odd = synth.uniform_code_bytes(g, (3, 100), 83)
    assert odd.shape == (3, 100, 42) and np.all(odd[..., -1] >> 4 == 0)


def test_ragged_lengths_in_range():
    w = synth.WORKLOADS["qwen3_1p7b_ragged"]
    lens = synth.seq_lens(w)
    assert lens.dtype == np.int32 and len(lens) == 16
    assert lens.min() >= 4096 and lens.max() <= 65536
    assert len(set(lens.tolist())) > 8


def test_workload_shapes():
    w = synth.WORKLOADS["qwen3_8b_g84"]
    assert (w.layers, w.C, w.n_q, w.n_kv, w.d_h, w.G, w.P, w.context) == (36, 4096, 32, 8, 128, 84, 42, 131072)
    E, W = synth.layer_weights(synth.WORKLOADS["tiny"], 0)
    assert E.shape == (64, 1024) and W.shape == (2 * 8 * 128, 64)
