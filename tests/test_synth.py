"""The shared seeded input generator: known-answer vectors for its random
number generator, determinism, slice independence and the encoder's
conversions (checked against numpy)."""
import ctypes

import numpy as np
import pytest

import synth


def _philox(c, k):
    c = np.array(c, dtype=np.uint32)
    k = np.array(k, dtype=np.uint32)
    o = np.zeros(4, dtype=np.uint32)
    synth.lib().synth_philox4x32_10(c.ctypes.data_as(ctypes.c_void_p), k.ctypes.data_as(ctypes.c_void_p),
                                    o.ctypes.data_as(ctypes.c_void_p))
    return [int(v) for v in o]


def test_philox4x32_10_known_answers():
    # known-answer vectors published with the Random123 library (Salmon et al., SC'11)
    assert _philox([0, 0, 0, 0], [0, 0]) == [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]
    assert _philox([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2) == [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]
    assert _philox([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0]) == \
        [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]


def test_normals_deterministic_and_sliceable():
    k = synth.key(9, 9, 9)
    a = synth.normal_f32(k, 10000)
    assert np.array_equal(a, synth.normal_f32(k, 10000))
    for start in (0, 1, 3, 4, 777):
        assert np.array_equal(synth.normal_f32(k, 50, start=start), a[start:start + 50])
    assert abs(a.mean()) < 0.05 and abs(a.std() - 1) < 0.03
    assert not np.array_equal(a[:100], synth.normal_f32(synth.key(9, 9, 8), 100))


def test_f16_encoding_matches_numpy_rne():
    rng = np.random.default_rng(0)
    vals = np.concatenate([rng.standard_normal(20000) * np.exp(rng.uniform(-20, 11, 20000)),
                           [0.0, 6.1e-5, 5.96e-8, 2.98e-8, 65504.0, 65519.0, 1e-4, 0.5 + 2 ** -12]])
    for v in vals:
        ref = int(np.array([v]).astype(np.float16).view(np.uint16)[0])
        assert synth.lib().synth_f64_to_f16(float(v)) == ref, v


def test_bf16_encoding_is_nearest_even():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(50000) * 3).astype(np.float32)
    b = synth.f32_to_bf16_bits(x)
    xb = synth.bf16_bits_to_f32(b).astype(np.float64)
    up = synth.bf16_bits_to_f32(b + 1).astype(np.float64)
    dn = synth.bf16_bits_to_f32(b - 1).astype(np.float64)
    err = np.abs(x - xb)
    assert np.all(err <= np.abs(x - up)) and np.all(err <= np.abs(x - dn))


def test_expert_matrix_deterministic_and_matches_batch():
    S = synth.TINY
    a = synth.expert_matrix(S, 0, 3, synth.DOWN)
    assert a.shape == (256, 2, 144)
    b = synth.layer_experts(S, 0, synth.DOWN, experts=[1, 3])
    assert np.array_equal(b[1], a)
    assert not np.array_equal(b[0], a)
    assert np.array_equal(synth.quantize_rows(synth.expert_matrix_f32(S, 0, 3, synth.DOWN)), a)


def test_distinct_layers_have_distinct_weights():
    S = synth.QWEN3_30B_A3B
    assert not np.array_equal(synth.router(S, 0), synth.router(S, 1))
    assert not np.array_equal(synth.expert_matrix(S, 0, 0, synth.GATE)[:4], synth.expert_matrix(S, 1, 0, synth.GATE)[:4])


def test_zipf_offsets_are_a_permutation_of_log_ranks():
    S = synth.QWEN3_30B_A3B
    off = synth.zipf_offsets(S, 5, 1.1)
    ranks = np.exp(-off / 1.1)
    assert np.allclose(np.sort(ranks), np.arange(1, 129))
    lg = synth.logits_f32(S, 5, 64, zipf_s=1.1)
    base = synth.logits_f32(S, 5, 64)
    assert lg.dtype == np.float32 and lg.shape == (64, 128)
    assert np.allclose(lg - base, off[None, :].astype(np.float32), atol=1e-5)


def test_shapes():
    assert synth.QWEN3_30B_A3B.expert_bytes == 2_654_208
    assert synth.TINY.expert_bytes == 221_184
    x = synth.x_bf16(synth.QWEN3_30B_A3B, 0, 0, T=4)
    assert x.shape == (4, 2048) and x.dtype == np.uint16
