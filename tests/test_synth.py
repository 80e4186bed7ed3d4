"""The seeded input generator: determinism and bf16 round-to-nearest-even encoding."""
import numpy as np
import torch

import synth


def test_same_seed_same_bits():
    a = synth.normal_operand(1234, (17, 33), 0.5, "bf16")
    b = synth.normal_operand(1234, (17, 33), 0.5, "bf16")
    np.testing.assert_array_equal(a.bits, b.bits)
    c = synth.normal_operand(1235, (17, 33), 0.5, "bf16")
    assert (a.bits != c.bits).any()


def test_bf16_rounding_matches_torch_rne():
    g = np.random.Generator(np.random.PCG64(7))
    v = (g.standard_normal(100000) * np.exp(g.uniform(-20, 20, 100000))).astype(np.float32)
    # include exact ties: values halfway between two bf16 neighbours
    ties = (np.arange(1, 2001, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    v = np.concatenate([v, ties, -ties])
    ours = synth.bf16_bits_from_f32(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_f64_value_is_exact():
    op = synth.normal_operand(99, (64, 64), 1.0, "bf16")
    back = torch.from_numpy(op.bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(op.f64, back)
    f = synth.normal_operand(99, (8, 8), 1.0, "f32")
    np.testing.assert_array_equal(f.f64, f.bits.astype(np.float64))


def test_std_and_positions():
    w = synth.normal_operand(5, (512, 512), 512 ** -0.5, "f32")
    assert abs(w.f64.std() * 512 ** 0.5 - 1.0) < 0.01
    p = synth.random_positions(3, 10000, 4096)
    assert p.min() >= 0 and p.max() < 4096
    np.testing.assert_array_equal(synth.cyclic_positions(6, seq_len=4, offset=1), [1, 2, 3, 4, 1, 2])
