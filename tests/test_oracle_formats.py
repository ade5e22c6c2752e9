"""Pins of the oracle's storage codecs (CPU only).

The fp8 decode is checked against hand-written OCP E4M3 values (tests/golden)
and against torch's float8_e4m3fn cast for all 256 codes; the fp8 encode
against torch's cast (after clamping to +-448, since torch's cast does not
saturate) on every rounding midpoint and its float32 neighbours, and against
the round-to-nearest property itself.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import formats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3fn_values.txt")


def _golden_rows():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        code, val = line.split()
        rows.append((int(code, 16), float(val)))
    return rows


def test_e4m3fn_golden_values():
    rows = _golden_rows()
    assert len(rows) >= 25
    for code, val in rows:
        got = formats.e4m3fn_to_f64(np.array([code], np.uint8))[0]
        if math.isnan(val):
            assert math.isnan(got), hex(code)
        else:
            assert got == val, hex(code)
            assert math.copysign(1.0, got) == math.copysign(1.0, val), hex(code)


def test_e4m3fn_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = formats.e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))
    # Exactly two NaN codes, no infinities, largest finite 448.
    assert nan.sum() == 2 and not np.isinf(ours).any()
    assert np.nanmax(ours) == 448.0


def _torch_encode(x: np.ndarray) -> np.ndarray:
    c = np.clip(x, -448.0, 448.0).astype(np.float32)
    return torch.from_numpy(c).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3fn_encode_midpoints_vs_torch():
    vals = np.unique(formats.E4M3FN_TABLE[:0x7F])            # 127 non-negative values
    mids = (vals[:-1] + vals[1:]) / 2.0                       # exact in float32
    mids32 = mids.astype(np.float32)
    assert np.array_equal(mids32.astype(np.float64), mids)
    probe = np.concatenate([
        vals.astype(np.float32), mids32,
        np.nextafter(mids32, np.float32(np.inf)), np.nextafter(mids32, np.float32(0)),
        np.array([448.0, 449.0, 463.99, 464.0, 470.0, 1e9, np.float32(3.4e38)], np.float32),
    ]).astype(np.float32)
    probe = np.concatenate([probe, -probe])
    ours = formats.f32_to_e4m3fn(probe)
    assert np.array_equal(ours, _torch_encode(probe))


def test_e4m3fn_encode_random_vs_torch():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(2_000_000) * np.exp(rng.uniform(-12, 7, 2_000_000))).astype(np.float32)
    assert np.array_equal(formats.f32_to_e4m3fn(x), _torch_encode(x))


def test_e4m3fn_encode_is_nearest():
    # Independent of torch: the chosen value is at least as close as every other.
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(20000) * 60).astype(np.float32)
    x = np.clip(x, -448, 448)
    code = formats.f32_to_e4m3fn(x)
    got = formats.e4m3fn_to_f64(code)
    finite = formats.E4M3FN_TABLE[~np.isnan(formats.E4M3FN_TABLE)]
    best = np.abs(x.astype(np.float64)[:, None] - finite[None, :]).min(axis=1)
    assert np.array_equal(np.abs(got - x.astype(np.float64)), best)


def test_e4m3fn_encode_special_cases():
    f = lambda v: int(formats.f32_to_e4m3fn(np.array([v], np.float32))[0])
    assert f(0.0) == 0x00 and f(-0.0) == 0x80
    assert f(-1e-30) == 0x80                          # underflow keeps the sign
    assert f(1e-30) == 0x00
    assert f(470.0) == 0x7E and f(-1e9) == 0xFE       # saturate, never NaN
    assert f(float("nan")) & 0x7F == 0x7F
    assert f(2.0 ** -10) == 0x00                      # half of min subnormal: tie -> even (0)
    assert f(3 * 2.0 ** -10) == 0x02                  # 1.5 * 2^-9: tie -> even code 0x02
    assert f(1.0625) == 0x38                          # tie between 1.0 (0x38) and 1.125 (0x39)
    assert f(1.1875) == 0x3A                          # tie between 0x39 and 0x3A -> 0x3A


def test_bf16_decode_vs_torch():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    ours = formats.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


# ------------------------------------------------------------------ int8 ----
def test_int8_exact_multiples_and_ties():
    """Symmetric int8 codes: integers map to themselves, ties go to the even
    neighbour (round half to even), at a power-of-two scale where x / scale
    is exact."""
    k = np.arange(-127, 128)
    scale = np.float32(2.0 ** -3)
    x = (k * 2.0 ** -3).astype(np.float32)
    assert np.array_equal(formats.f32_to_int8_sym(x / scale), k.astype(np.int8))
    q = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 125.5, -126.5], dtype=np.float32)
    want = np.array([0, 2, 2, 0, -2, -2, 126, -126], dtype=np.int8)
    assert np.array_equal(formats.f32_to_int8_sym(q), want)


def test_int8_saturation_and_special_values():
    q = np.array([127.49, 127.5, 128.0, 1e30, np.inf, -127.5, -128.0, -np.inf, np.nan, -0.0],
                 dtype=np.float32)
    want = np.array([127, 127, 127, 127, 127, -127, -127, -127, 0, 0], dtype=np.int8)
    assert np.array_equal(formats.f32_to_int8_sym(q), want)
    rng = np.random.default_rng(3)
    codes = formats.f32_to_int8_sym(rng.normal(0, 300, 100000).astype(np.float32))
    assert codes.min() == -127 and codes.max() == 127     # -128 is never produced


def test_int8_encode_vs_torch_quantize_per_tensor():
    """torch's per-tensor qint8 quantizer (round half to even of x * (1/scale),
    zero point 0) on values inside +-126 code steps, at a power-of-two scale
    (where x * (1/scale) equals x / scale exactly)."""
    rng = np.random.default_rng(5)
    scale = 2.0 ** -5
    x = (rng.uniform(-126, 126, 200000) * scale).astype(np.float32)
    x[:505] = (np.arange(-252, 253) * 0.5 * scale).astype(np.float32)       # ties within +-126
    ref = torch.quantize_per_tensor(torch.from_numpy(x), scale, 0, torch.qint8).int_repr()
    ours = formats.f32_to_int8_sym(x / np.float32(scale))
    assert np.array_equal(ours, ref.numpy())


def test_int8_round_trip_error_bound():
    """|c * scale - x| <= scale * (1/2 + 2^-18) inside the range (the
    quotient x / scale is first rounded to float32: half an ulp, at most
    2^-18 code steps below 128); beyond it the error is |x| - 127 * scale."""
    rng = np.random.default_rng(6)
    scale = np.float32(0.0371)
    x = rng.normal(0, 3, 100000).astype(np.float32)
    c = formats.f32_to_int8_sym(x / scale)
    back = formats.int8_to_f64(c) * np.float64(scale)
    inside = np.abs(x.astype(np.float64)) <= 127 * np.float64(scale)
    err = np.abs(back - x.astype(np.float64))
    assert err[inside].max() <= np.float64(scale) * (0.5 + 2.0 ** -18)
    assert np.allclose(err[~inside], np.abs(x[~inside].astype(np.float64)) - 127 * np.float64(scale))
