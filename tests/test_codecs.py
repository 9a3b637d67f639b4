"""Oracle codecs (bf16, OCP e4m3) and the input generator's bf16 rounding, against torch CPU casts."""
import numpy as np
import torch

from oracle import codecs
from tiled_online_softmax_amd import inputs


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = codecs.e4m3_to_f64(codes)
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert nan.sum() == 2  # S.1111.111 only
    np.testing.assert_array_equal(got[~nan], ref[~nan])


def test_e4m3_hand_values():
    # from the format definition: bias 7, 3 mantissa bits, subnormals at exponent 0
    assert codecs.e4m3_to_f64(np.uint8(0x38)) == 1.0
    assert codecs.e4m3_to_f64(np.uint8(0x7E)) == 448.0
    assert codecs.e4m3_to_f64(np.uint8(0x01)) == 2.0 ** -9
    assert codecs.e4m3_to_f64(np.uint8(0x08)) == 2.0 ** -6
    assert codecs.e4m3_to_f64(np.uint8(0xC0)) == -2.0


def test_e4m3_encode_matches_torch_rne():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(400000).astype(np.float32) * 60,
        rng.standard_normal(200000).astype(np.float32) * 1e-2,   # subnormal range
        (rng.uniform(-448, 448, 200000)).astype(np.float32),
    ])
    # exact midpoints between neighbouring codes (ties) and the codes themselves
    pos = codecs.E4M3_TABLE[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids, pos.astype(np.float32)])
    got = codecs.f64_to_e4m3(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got, ref)


def test_e4m3_saturates():
    got = codecs.f64_to_e4m3(np.array([448.0, 460.0, 1e6, -1e6]))
    np.testing.assert_array_equal(got, [0x7E, 0x7E, 0x7E, 0xFE])


def test_quantize_per_tensor_recipe():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((3, 5, 77)).astype(np.float32)
    codes, descale = codecs.quantize_per_tensor(x)
    amax = np.abs(x).max()
    assert descale == np.float32(amax / np.float32(448))
    # the element of largest magnitude maps to +-448 exactly, nothing saturates beyond it
    vals = codecs.e4m3_to_f64(codes)
    assert np.abs(vals).max() == 448.0
    # torch reproduces the codes from the same float32 product
    s = np.float32(448) / np.float32(amax)
    ref = torch.from_numpy((x * s).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codes, ref)
    # dequantised values are within half an e4m3 step (relative 2^-4) of the input
    deq = codecs.dequantize(codes, descale)
    big = np.abs(x) > amax * 2.0 ** -6
    assert (np.abs(deq - x)[big] <= np.abs(x[big]) * 2.0 ** -4 + 1e-7).all()


def test_quantize_zero_tensor():
    codes, descale = codecs.quantize_per_tensor(np.zeros(10, np.float32))
    assert descale == 1.0 and (codes == 0).all()


def test_bf16_round_trip_matches_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(500000).astype(np.float32),
                        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -1.0 - 2.0 ** -8], np.float32)])
    bits = inputs.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)
    np.testing.assert_array_equal(codecs.bf16_to_f64(bits),
                                  torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy())


def test_inputs_are_seeded_and_ordered():
    w = inputs.WORKLOADS["bwd_causal_bf16"]
    a = inputs.make(w, shape=(1, 2, 8, 4))
    b = inputs.make(w, shape=(1, 2, 8, 4))
    for n in ("q", "k", "v", "do"):
        np.testing.assert_array_equal(a[n], b[n])
    rng = np.random.default_rng(w.seed)
    np.testing.assert_array_equal(a["q"], rng.standard_normal((1, 2, 8, 4), dtype=np.float32))
    np.testing.assert_array_equal(a["k"], rng.standard_normal((1, 2, 8, 4), dtype=np.float32))
    half = inputs.make(inputs.WORKLOADS["d256_bf16"], shape=(1, 1, 4, 4))
    full = inputs.draw((1, 1, 4, 4), inputs.WORKLOADS["d256_bf16"].seed, 3)
    np.testing.assert_array_equal(half["v"], full[2] * np.float32(0.5))
