"""The seeded input generator: determinism, stream independence and bf16 rounding."""
import numpy as np

from llama_decoder_transformer_amd import inputs


def test_bf16_round_to_nearest_even_known_values():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5, 0.0, 3.0e38],
                 np.float32)
    bits = inputs.f32_to_bf16_bits(f)
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 ties up to 1+2^-6... (mantissa 0x81 is odd -> 0x82)
    np.testing.assert_array_equal(bits[:4], [0x3F80, 0x3F80, 0x3F82, 0x3F81])
    assert bits[4] == 0xC020 and bits[5] == 0
    back = inputs.bf16_bits_to_f32(bits)
    assert back[0] == 1.0 and back[4] == -2.5
    assert abs(back[6] - 3.0e38) / 3.0e38 < 2 ** -8


def test_streams_deterministic_blocked_and_independent():
    a = inputs.normal_f32((0, 5), inputs.BLOCK + 1000, 1.0)
    b = inputs.normal_f32((0, 5), inputs.BLOCK + 1000, 1.0)
    np.testing.assert_array_equal(a, b)
    c = inputs.normal_f32((0, 6), 1000, 1.0)
    assert not np.array_equal(a[:1000], c)
    # a prefix of a stream family is the same whatever the total length
    np.testing.assert_array_equal(inputs.normal_f32((0, 5), 777, 1.0), a[:777])
    bits = inputs.normal_bf16_bits((0, 5), 777, 1.0)
    np.testing.assert_array_equal(bits, inputs.f32_to_bf16_bits(a[:777]))


def test_weight_distribution_and_norms():
    s = inputs.STORIES15M
    w = inputs.weight(s, "layers.0.feed_forward.w1.weight")
    assert w.shape == (768, 288) and w.dtype == np.float32
    assert abs(w.std() - 0.02) < 5e-4 and abs(w.mean()) < 5e-4
    assert np.all(inputs.weight(s, "layers.3.ffn_norm.weight") == 1.0)
    s8 = inputs.LLAMA3_8B.replace(n_layers=1, vocab_size=64, dim=256, n_heads=2, n_kv_heads=1,
                                  ffn_hidden_dim=512)
    wb = inputs.weight(s8, "layers.0.attention.wk.weight")
    assert wb.dtype == np.uint16 and wb.shape == (128, 256)
    wf = inputs.weight(s8, "layers.0.attention.wk.weight", as_bits=False)
    np.testing.assert_array_equal(inputs.f32_to_bf16_bits(wf), wb)
    assert np.all(inputs.weight(s8, "norm.weight") == 0x3F80)


def test_other_inputs():
    t = inputs.token_ids(32000, 8)
    assert t.dtype == np.int32 and t.min() >= 0 and t.max() < 32000
    np.testing.assert_array_equal(t, inputs.token_ids(32000, 8))
    L = inputs.kv_lengths(64, 1024, 8192)
    assert L.min() >= 1024 and L.max() <= 8192 and len(set(L.tolist())) > 50
    kv = inputs.kv_contents_bf16_bits(3, 1, 7, 2, 100, 128)
    assert kv.shape == (100, 128) and kv.dtype == np.uint16
    x = inputs.bf16_bits_to_f32(inputs.activations_bf16_bits(64, 64))
    assert abs(x.std() - 1.0) < 0.05
