"""Pins of the oracle's number-format decoding (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import formats
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_e4m3_matches_torch_cast_all_codes():
    # Library routine: torch's float8_e4m3fn -> float64 conversion (OCP E4M3FN).
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    finite = ~np.isnan(lib)
    assert set(np.nonzero(~finite)[0].tolist()) == {0x7F, 0xFF}
    np.testing.assert_array_equal(formats.e4m3_to_f64(codes[finite]), lib[finite])
    assert np.signbit(formats.e4m3_to_f64(np.array([0x80], np.uint8)))[0]


def test_e4m3_golden_and_nan_rejected():
    g = _gold("e3_fp8.json")
    for c in g["cases"]:
        assert formats.e4m3_to_f64(np.array([c["code"]], np.uint8))[0] == c["value"]
    for n in g["nan_codes"]:
        with pytest.raises(formats.FormatError):
            formats.e4m3_to_f64(np.array([n], np.uint8))


def test_e8m0_matches_torch_cast():
    codes = np.arange(255, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    np.testing.assert_array_equal(formats.e8m0_to_f64(codes), lib)
    with pytest.raises(formats.FormatError):
        formats.e8m0_to_f64(np.array([255], np.uint8))


def test_e2m1_matches_ocp_value_listing():
    # OCP MX v1.0 lists the E2M1 magnitudes for codes 0..7 as below; codes
    # 8..15 are their negatives.
    listing = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = formats.e2m1_to_f64(np.arange(16, dtype=np.uint8))
    np.testing.assert_array_equal(got[:8], listing)
    np.testing.assert_array_equal(got[8:], [-v for v in listing])


def test_mxfp4_golden_bytes():
    for c in _gold("e2_mxfp4.json")["cases"]:
        b = np.zeros(16, np.uint8)
        b[0] = c["byte"]
        sc = np.full(1, c["scale_code"], np.uint8)
        v = formats.mxfp4_to_f64(b, sc)
        np.testing.assert_array_equal(v[:2], c["elements"])
        assert np.signbit(v[0]) == np.signbit(c["elements"][0])


def test_mxfp4_scale_applies_per_32_elements():
    b = np.full(256, 0x22, np.uint8)            # every element 1.0
    sc = np.arange(120, 136, dtype=np.uint8)    # 16 different scales
    v = formats.mxfp4_to_f64(b, sc)
    for g in range(16):
        np.testing.assert_array_equal(v[32 * g:32 * g + 32], 2.0 ** (int(sc[g]) - 127))


def test_mxfp4_roundtrip_error_bound():
    # Decoding the independent encoder's bytes must give each input back to
    # within half a grid step of its binade (OCP MX rounding), or the
    # saturation error for |x / 2^X| > 6.
    x = torch.randn(64, 512, generator=torch.Generator().manual_seed(7), dtype=torch.float32)
    p, s = synth.to_mxfp4(x)
    dec = formats.mxfp4_to_f64(p.numpy(), s.numpy())
    xd = x.double().numpy()
    scale = np.repeat(formats.e8m0_to_f64(s.numpy()), 32, axis=-1)
    a = np.abs(xd) / scale
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    bound = np.where(a <= 6, step / 2, a - 6) * scale
    assert np.all(np.abs(dec - xd) <= bound + 1e-12)
    # The block maximum lands in the top binade [4, 8) before saturation.
    amax = np.abs(xd).reshape(64, 16, 32).max(-1)
    r = amax / formats.e8m0_to_f64(s.numpy())
    assert np.all((r >= 4) & (r < 8))


def test_bf16_matches_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = formats.bf16_to_f64(bits)
    ok = ~np.isnan(lib)
    np.testing.assert_array_equal(got[ok], lib[ok])
    assert np.all(np.isnan(got[~ok]))
