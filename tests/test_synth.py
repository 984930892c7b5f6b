"""The seeded input generator: published Philox4x32-10 answers, distributions, reproducibility."""
import numpy as np

import synth


def test_philox_known_answers():
    # Known-answer vectors published with Random123 for philox4x32-10 (Salmon et al., SC'11).
    assert list(synth.philox4x32_10([0, 0, 0, 0], [0, 0])) == [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]
    assert list(synth.philox4x32_10([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2)) == [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]
    assert list(synth.philox4x32_10([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0])) == \
        [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]


def test_normal_moments_and_bf16():
    b, f = synth.fill((1 << 20,), synth.tensor_key(9, 0, "x"), "normal", 0.02, fmt="both")
    assert abs(f.mean()) < 1e-4 and abs(f.std() - 0.02) < 2e-4
    assert np.array_equal(synth.bf16_bits_to_f32(b), f)
    assert np.array_equal(synth.f32_to_bf16_bits(f), b)      # values are bf16-representable
    assert np.abs(f).max() <= 0.02 * 4.9 * 1.01                # Irwin-Hall(8) tails are bounded


def test_uniform_range_and_reproducible():
    k = synth.tensor_key(9, 1, "u")
    u1 = synth.fill((4096,), k, "uniform")
    u2 = synth.fill((4096,), k, "uniform")
    assert np.array_equal(u1, u2)
    assert u1.min() >= -1.0 and u1.max() <= 1.0 and abs(u1.mean()) < 0.05
    assert not np.array_equal(u1, synth.fill((4096,), synth.tensor_key(9, 2, "u"), "uniform"))


def test_bf16_rounding_ties_to_even():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 1.0 + 2 ** -9], dtype=np.float32)
    r = synth.round_bf16(x)
    assert list(r) == [1.0, 1.0 + 2 ** -6, -1.0, 1.0]


def test_timesteps_in_unit_interval():
    t = synth.workloads.timesteps(synth.WORKLOADS[3], 1000)
    assert t.min() >= 0 and t.max() < 1 and abs(t.mean() - 0.5) < 0.05


def test_matrix_classification_matches_abi_contract():
    # The C ABI reads Linear weights ([out, in]) in the model dtype and every other tensor as float32;
    # the uploader must classify each tensor exactly that way (a vector mistaken for a matrix would be
    # stored as bf16 and read as float, past its end).
    from synth.workloads import global_tensors, is_matrix, layer_tensors
    w = synth.WORKLOADS[3]
    for name, shape, _, _ in global_tensors(w) + layer_tensors(w):
        linear = len(shape) == 2 and name not in ("mod", "head_mod")
        assert is_matrix(name) == linear, name
