"""Pins of the oracle's number formats against the format definitions and torch's casts."""
import numpy as np
import torch

import oracle


def test_e4m3_table_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = oracle.E4M3_VALUES
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(ref[~nan], ours[~nan])
    # signed zero kept
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


def test_e4m3_definition_points():
    # OCP E4M3: bias 7, 3 mantissa bits, largest finite 448, smallest normal 2^-6,
    # smallest subnormal 2^-9
    v = oracle.e4m3_decode(np.array([0x7E, 0x08, 0x01, 0x38, 0xB8, 0x07, 0x0F, 0x77, 0x7D, 0x30],
                                    np.uint8))
    assert list(v) == [448.0, 2.0 ** -6, 2.0 ** -9, 1.0, -1.0, 7 * 2.0 ** -9, 1.875 * 2.0 ** -6,
                       240.0, 416.0, 0.5]


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, 20000, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    man = bits & 0x7F
    bits = bits[~((exp == 0xFF) & (man != 0))]
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.bf16_decode(bits), ref)


def test_latent_row_fp8_layout_reading():
    # nope codes 0x38 (=1.0) and 0xB0 (=-0.5); rope bf16 0x4040 (=3.0); scale 0.25
    row = np.zeros((1, 656), np.uint8)
    row[0, :256] = 0x38
    row[0, 256:512] = 0xB0
    row[0, 512:640] = np.frombuffer(np.full(64, 0x4040, np.uint16).tobytes(), np.uint8)
    row[0, 640:644] = np.frombuffer(np.float32(0.25).tobytes(), np.uint8)
    lat = oracle.decode_latent_rows(row, 1)
    assert lat.shape == (1, 576)
    assert np.all(lat[0, :256] == 0.25) and np.all(lat[0, 256:512] == -0.125)
    assert np.all(lat[0, 512:] == 3.0)


def test_latent_row_bf16():
    vals = ((np.arange(576) % 97) - 48).astype(np.float32) * 0.25   # exact in bf16
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    lat = oracle.decode_latent_rows(bits.view(np.uint8).reshape(1, 1152), 0)
    assert np.array_equal(lat[0], vals.astype(np.float64))


def test_idx_key_dequant_is_exact_product():
    codes = np.array([[0x38] * 128, [0x7E] * 128], np.uint8)
    scale = np.array([0.1, 3.0], np.float32)
    k = oracle.dequant_idx_keys(codes, scale)
    assert k[0, 0] == float(np.float32(0.1)) and k[1, 5] == 448.0 * 3.0
