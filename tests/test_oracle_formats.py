"""Pins for the oracle's storage decoding and its fp8 (e4m3fn) codec.

The codec is pinned to a library routine (torch's float8_e4m3fn cast, after
clamping to the finite range) exhaustively over every fp16 bit pattern and a
million random fp32 values, and to hand-worked values of the format.
"""
import numpy as np
import pytest
import torch

from oracle import formats
from oracle.formats import decode, e4m3_encode

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def torch_encode(y32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.asarray(y32, np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_table_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = formats.e4m3_decode_table()
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])      # the only NaN codes
    assert np.isnan(got).sum() == 2


def test_decode_hand_values():
    t = formats.e4m3_decode_table()
    assert t[0x7E] == 448.0                      # largest finite
    assert t[0x01] == 2.0 ** -9                  # smallest subnormal
    assert t[0x08] == 2.0 ** -6                  # smallest normal
    assert t[0x38] == 1.0                        # exponent field 7 = bias
    assert t[0xB8] == -1.0
    assert t[0x80] == 0.0 and np.signbit(t[0x80])


@pytest.mark.parametrize("scale", [1.0, 2.0 ** -3, 3.7])
def test_encode_matches_torch_exhaustive_fp16(scale):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16).astype(np.float32)
    x = x[~np.isnan(x)]
    inv = np.float32(1.0) / np.float32(scale)
    y = x * inv
    assert np.array_equal(e4m3_encode(y), torch_encode(y))


def test_encode_matches_torch_random_fp32():
    rng = np.random.default_rng(1234)
    mag = np.exp2(rng.uniform(-14, 10, size=1_000_000)).astype(np.float32)
    y = (mag * rng.choice([-1, 1], size=mag.size)).astype(np.float32)
    assert np.array_equal(e4m3_encode(y), torch_encode(y))


def test_encode_special_values():
    y = np.array([448, 464, 1e30, np.inf, -np.inf, np.nan, -np.nan, 0.0, -0.0,
                  2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, 1.0625, 1.1875], dtype=np.float32)
    c = e4m3_encode(y)
    assert c[0] == 0x7E and c[1] == 0x7E and c[2] == 0x7E and c[3] == 0x7E   # saturate
    assert c[4] == 0xFE
    assert (c[5] & 0x7F) == 0x7F and (c[6] & 0x7F) == 0x7F                 # NaN stays NaN
    assert c[7] == 0x00 and c[8] == 0x80
    assert c[9] == 0x01
    assert c[10] == 0x00              # half of the smallest subnormal ties to even (zero)
    assert c[11] == 0x02              # 1.5 x smallest subnormal ties up to even code 2
    assert c[12] == 0x38              # 1.0625 is halfway 1.0/1.125: ties to even mantissa (1.0)
    assert c[13] == 0x3A              # 1.1875 is halfway 1.125/1.25: ties to 1.25 (even)


def test_roundtrip_all_finite_codes():
    t = formats.e4m3_decode_table()
    codes = np.array([c for c in range(256) if not np.isnan(t[c])], dtype=np.uint8)
    back = e4m3_encode(t[codes].astype(np.float32))
    assert np.array_equal(back, codes)


def test_decode_bf16_and_f16_match_torch():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(10000).astype(np.float32) * 100
    bf = torch.from_numpy(x).to(torch.bfloat16)
    raw = bf.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(decode(raw, "bf16"), bf.to(torch.float64).numpy())
    h = x.astype(np.float16)
    assert np.array_equal(decode(h, "f16"), torch.from_numpy(h).to(torch.float64).numpy())
    codes = rng.integers(0, 256, 1000).astype(np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]
    assert np.allclose(decode(codes, "fp8_e4m3", 0.25),
                       torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy() * 0.25,
                       rtol=0, atol=0)
