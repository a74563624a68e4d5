"""Pins of the oracle's number-format decoders and of the generator's quantisers."""
import numpy as np
import torch

from oracle.numformats import decode_bf16_bits, decode_e4m3fn_bits
from synth import bf16_bits_from_f32, e4m3fn_bits_from_f32


def test_e4m3fn_decoder_matches_torch_on_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = decode_e4m3fn_bits(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2                                   # 0x7F and 0xFF
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9   # max normal, min subnormal


def test_e4m3fn_quantiser_is_nearest_even_and_saturating():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 100,
                        np.array([448.0, 449.0, 470.0, 1e6, -1e6, 0.0, -0.0, 2.0 ** -10,
                                  3 * 2.0 ** -11], np.float32)])
    q = decode_e4m3fn_bits(e4m3fn_bits_from_f32(x))
    table = decode_e4m3fn_bits(np.arange(256, dtype=np.uint8))
    finite = table[~np.isnan(table)]
    xc = np.clip(x.astype(np.float64), -448, 448)
    # brute force: the result is one of the closest representable values
    dist = np.abs(finite[None, :] - xc[:, None])
    best = dist.min(axis=1)
    assert np.all(np.abs(q - xc) == best)
    # exact ties go to the even mantissa: 3 * 2^-11 lies between 2^-10 (m=0 sub... ) codes
    assert np.all(np.abs(q) <= 448.0)


def test_bf16_decoder_and_quantiser():
    rng = np.random.default_rng(2)
    bits = rng.integers(0, 2 ** 16, size=50000).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = decode_bf16_bits(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # quantiser: nearest-even rounding of float32 to 8 significant bits
    x = rng.standard_normal(50000).astype(np.float32)
    b = bf16_bits_from_f32(x)
    xb = decode_bf16_bits(b)
    ulp = np.spacing(np.abs(xb).astype(np.float32)).astype(np.float64) * 2 ** 16
    assert np.all(np.abs(xb - x) <= ulp / 2 + 1e-300)
